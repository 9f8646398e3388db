// Step 2 backward, bf16 inputs, on gfx950 MFMA (v_mfma_f32_32x32x16_bf16).
//
// The pages describe no backward; this is the chain rule of the forward
// (page "Hugging Face并行加速", nmedialink.com, section "Ulysses的工作原理",
// step 4) with P recomputed from the saved log-sum-exp, which keeps memory
// linear in N as the tiled forward does (same page, section
// "超长序列训练的挑战"):
//   delta_c = sum_d dO_c O_c,   P = exp(scale Q K^T - lse),   dP = dO V^T,
//   dS = P * (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
// Query columns interleave the G query heads of a KV head (column
// c = token * G + head_in_group), so dK and dV sum over the group for free.
//
// Three kernels, no atomics (bitwise deterministic):
//  * delta_bf16_kernel: delta per query column (fp32).
//  * dkdv_kernel (key-outer): a work-group owns 128 keys, whose K and V rows
//    stay in LDS; its 8 waves (two per SIMD) pair up on 32-key blocks and
//    split every query tile into halves, accumulating dK^T and dV^T in
//    registers over every query tile that can see their keys.  Scores are
//    formed as S = Q K^T (columns x keys) so that P and dS come out of the MFMA
//    already shaped as the B operand of dV^T += dO^T P and dK^T += Q^T dS.  Q
//    and dO tiles are staged row-major in LDS (rows permuted so each
//    accumulator group covers 8 consecutive columns, 16-byte chunks XOR
//    swizzled against bank conflicts); the transposed A operands dO^T and Q^T
//    are read from the same tiles with the gfx950 LDS transpose read
//    (ds_read_b64_tr_b16), so only 32 KiB per 64-column tile crosses from L2;
//    those tiles are copied global -> LDS by DMA.
//  * dq_kernel_1w (D = 128) and dq_kernel (D = 64), query-outer like the
//    forward: a wave owns 64 (dq_kernel_1w, one wave per SIMD) or 32 query
//    columns with Q and dO in registers; S^T and dP^T are recomputed per key
//    tile and dQ^T += K^T dS^T takes K^T from the K tile by transpose reads.
// Tiles outside the causal band and outside the documents are never visited;
// tiles that are fully visible skip the per-element mask.
#include "ul_internal.h"

#include <math.h>

#include <type_traits>

namespace ul {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }
// LDS row of tile row r (0..63): permuted within each half of 32
__device__ __forceinline__ int tile_row(int r) { return (r & 32) | perm_row(r & 31); }

// Byte offset of 16-byte chunk `chunk` of physical row `prow` in an unpadded
// [64][D] bf16 LDS tile whose chunks are XOR-swizzled per row (chunk c of row
// r sits in slot c ^ swz(r)).  The swizzle keeps both access patterns used
// here free of bank conflicts: 16 consecutive rows read at the same chunk
// (MFMA row operands), and 4 consecutive rows x 4 consecutive chunks read by
// 32 lanes (transpose reads).
template <int D>
__device__ __forceinline__ int lds_off(int prow, int chunk) {
  constexpr int CPR = D / 8;
  const int swz = (((prow & 3) << 2) ^ ((prow >> 2) & 3)) & (CPR - 1);
  return prow * (D * 2) + ((chunk ^ swz) << 4);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)s[base + e];
  return r;
}

__device__ __forceinline__ int64_t col_offset(int64_t c, int lgG, int Hkv, int hk, int D) {
  // element offset of query column c of KV group hk in a [N][Hq][D] tensor
  return ((((c >> lgG) * Hkv + hk) << lgG) + (c & ((1 << lgG) - 1))) * D;
}

// a pointer that is the same in every lane, moved to scalar registers
__device__ __forceinline__ const bf16* uniform_ptr(const bf16* p) {
  const uint64_t x = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x), hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return reinterpret_cast<const bf16*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// A operand of a 32x32x16 MFMA whose rows are the feature axis of a row-major
// [64 rows][D] bf16 LDS tile (rows stored at tile_row(), chunks swizzled) and
// whose k axis is the tile's row axis: lane l gets feature d0 + (l & 31) of
// rows k0 + 8*(l >> 5) + 0..7.  Within each 16-lane group the transpose read
// hands lane j element (j & 3) of the 8-byte chunks read by lanes
// (j >> 2) + 4e, e = 0..3, so lane s reads row k + (s >> 2), features
// n0 + 4*(s & 3) .. +3.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_a(const char* tile, int d0, int k0, int lane) {
  const int m = lane >> 4, s = lane & 15;
  const int n = d0 + (m & 1) * 16 + 4 * (s & 3);
  const int k = k0 + (m >> 1) * 8 + (s >> 2);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const lds_s16x4* p1 = (const lds_s16x4*)(tile + lds_off<D>(tile_row(k), n >> 3) + (n & 7) * 2);
  const lds_s16x4* p2 = (const lds_s16x4*)(tile + lds_off<D>(tile_row(k + 4), n >> 3) + (n & 7) * 2);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p1);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p2);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// ------------------------------------------------------------------ delta --
template <int D>
__global__ void __launch_bounds__(256) delta_bf16_kernel(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                       float* __restrict__ delta, int64_t NG, int Hkv, int lgG) {
  constexpr int LPC = D / 8;        // lanes per column (8 elements each)
  constexpr int CPB = 256 / LPC;    // columns per block
  const int hk = blockIdx.y;
  const int64_t c = (int64_t)blockIdx.x * CPB + threadIdx.x / LPC;
  const int part = threadIdx.x % LPC;
  float s = 0.0f;
  if (c < NG) {
    const int64_t off = col_offset(c, lgG, Hkv, hk, D) + part * 8;
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + off);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)a[e], (float)b[e], s);
  }
#pragma unroll
  for (int m = LPC / 2; m > 0; m >>= 1) s += __shfl_xor(s, m, 64);
  if (c < NG && part == 0) delta[(int64_t)hk * NG + c] = s;
}

// ------------------------------------------------------------------- dK dV --
// A work-group owns 128 keys of one KV head; their K and V rows sit in LDS
// for the whole kernel.  Eight waves, two per SIMD: waves w and w+4 share the
// 32-key block (w & 3) and split every 64-column query tile into halves, each
// accumulating partial dK^T and dV^T in registers; the halves are summed
// through LDS at the end.
// Prologue padding (executed once per wave) that places a kernel's tile loop
// at a measured-good offset within the 64-byte lines the instructions are
// fetched in: an earlier eight-wave dQ kernel ran 3 % slower with its loop 44
// bytes into a line than at 0, 24 or 32 (same box, N = 1M, identical loop
// code), and dK/dV's offsets spread over 1.5 %.  The count holds for the code
// as it stands; any change to a prologue moves its loop
// (tests/test_code_layout.py disassembles the build and checks the offsets).
#define UL_CODE_PAD(n) asm volatile(".rept " #n "\ns_nop 0\n.endr")

template <int D>
struct DkvCfg {
  static constexpr int NW = 8;
  static constexpr int kThreads = NW * 64;
  static constexpr int BNK = 128;          // keys per work-group
  static constexpr int BQ = 64;            // query columns per tile
  static constexpr int KSTR = D * 2 + 16;  // LDS bytes per K / V row (padded)
  static constexpr int KVBYTES = BNK * KSTR;
  static constexpr int RSTR = D * 2;       // LDS bytes per Q / dO row (swizzled, unpadded)
  static constexpr int RBYTES = BQ * RSTR;
  static constexpr int AUX = BQ * 2 * 4;   // lse2, -delta per column
  // aux first: every operand offset of the second stage then fits a 16-bit
  // LDS immediate
  static constexpr int AUX_OFF = 0, Q_OFF = AUX, DO_OFF = AUX + RBYTES;
  static constexpr int STAGE = AUX + 2 * RBYTES;
  static constexpr int K_LDS = 2 * STAGE, V_LDS = 2 * STAGE + KVBYTES;
  static constexpr int SMEM = 2 * STAGE + 2 * KVBYTES;
  static constexpr int RCH = BQ * D / 8;   // 16-byte chunks per row tile
  static constexpr int RPT = RCH / kThreads;
  static constexpr int KVCH = BNK * D / 8;
  static constexpr int KVPT = KVCH / kThreads;
  static constexpr int RED_BYTES = 4 * 64 * (D / 32) * 16 * 4;  // one accumulator set of the four upper waves
  static_assert(RCH % kThreads == 0 && KVCH % kThreads == 0, "tile chunks must split evenly");
  static_assert(RED_BYTES <= SMEM, "reduction buffer must fit in LDS");
};

// Query-tile windows: a key block whose tiles reach at least two windows of
// `win_tiles` tiles beyond the window that holds its diagonal tile has them
// split at the window bounds.  One launch (win < 0) takes every key block's
// tiles inside its diagonal window (or all of them, for a key block that is
// not split) and writes dK / dV; then one launch per later window takes the
// split key blocks that see that window from below and adds to dK / dV.  All
// work-groups of such a launch sweep the same window from its top, so the
// ones resident together stay within a few tiles of each other and share the
// window's Q / dO tiles in L2 (one sweep over a long document drifts apart by
// more than the L2 holds).  Key blocks of shorter documents keep one sweep:
// split, their few window parts would run as a short tail of mostly idle
// launches.
template <int D>
__global__ void __launch_bounds__(DkvCfg<D>::kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) dkdv_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ doc_start, const int32_t* __restrict__ doc_end, const int32_t* __restrict__ order,
    float* __restrict__ dk, float* __restrict__ dv, int N, int Hkv, int lgG, float sl2, float scale, int win_tiles,
    int win) {
  using C = DkvCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
  UL_CODE_PAD(2);  // tile loop at 40 bytes into a 64-byte line (D = 128)
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lc = l & 31;
  const int kbw = w & 3;   // this wave's 32-key block
  const int qh = w >> 2;   // this wave's half of every query tile
  const int G = 1 << lgG;
  const int hk = blockIdx.x % Hkv;
  const int kblk = order[blockIdx.x / Hkv];  // heaviest key blocks first
  const int64_t NG = (int64_t)N << lgG;
  const int kb0 = kblk * C::BNK;
  const int kb_last = min(N - 1, kb0 + C::BNK - 1);
  const int row_end = doc_end[kb_last];
  const int de0 = doc_end[kb0];  // rows after it belong to later documents than key kb0
  // every query tile that sees a key of this block, then this launch's part of it
  const int tq_first = (int)(((int64_t)kb0 << lgG) / C::BQ);
  const int tq_last = (int)((((int64_t)(row_end + 1) << lgG) - 1) / C::BQ);
  const int diag_win = tq_first / win_tiles;
  const bool split = tq_last / win_tiles - diag_win >= 2;
  const bool accumulate = win >= 0;
  if (accumulate && (!split || diag_win >= win || tq_last < win * win_tiles)) return;  // nothing here (uniform)
  const int tq_lo = accumulate ? win * win_tiles : tq_first;
  const int tq_hi = split ? min(tq_last, (accumulate ? win : diag_win) * win_tiles + win_tiles - 1) : tq_last;
  const int key = kb0 + kbw * 32 + lc;
  const bool kvalid = key < N;
  // query column c sees this lane's key iff key <= row(c) <= doc_end[key], i.e.
  // key * G <= c < col_end (past the sequence nothing is visible)
  const int col_end = (int)min<int64_t>((int64_t)(doc_end[min(key, N - 1)] + 1) << lgG, NG);

  // K and V rows of the work-group's keys into LDS (zero past N)
#pragma unroll
  for (int i = 0; i < C::KVPT; ++i) {
    const int ch = tid + i * C::kThreads;
    const int r = ch / (D / 8), part = ch % (D / 8);
    const int kr = kb0 + r;
    u32x4 kv4 = {0u, 0u, 0u, 0u}, vv4 = {0u, 0u, 0u, 0u};
    if (kr < N) {
      const int64_t off = ((int64_t)kr * Hkv + hk) * D + part * 8;
      kv4 = *reinterpret_cast<const u32x4*>(k + off);
      vv4 = *reinterpret_cast<const u32x4*>(v + off);
    }
    *reinterpret_cast<u32x4*>(smem + C::K_LDS + r * C::KSTR + part * 16) = kv4;
    *reinterpret_cast<u32x4*>(smem + C::V_LDS + r * C::KSTR + part * 16) = vv4;
  }

  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) { dkt[db][i] = 0.0f; dvt[db][i] = 0.0f; }

  float a_lse = 0.0f, a_dl = 0.0f;
  // Q and dO tiles go global -> LDS by DMA (global_load_lds_dwordx4): lane l
  // of wave w's i-th copy writes the 16 bytes at byte (w * RPT + i) * 1024 +
  // l * 16 of the tile, so it fetches the tile row and chunk that the permuted,
  // swizzled layout keeps there.  Moving a tile down by BQ columns (BQ / G
  // whole tokens) moves every source address by a constant; only the first
  // tile visited (the one that may run past the end of the sequence, with
  // clamped columns) computes its addresses in full.  The copies are inline
  // assembly so that the compiler does not order this tile's LDS reads behind
  // them; each wave waits for its own copies before the tile's last barrier.
  int dr[C::RPT], dch[C::RPT];
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) {
    const int pb = (w * C::RPT + i) * 1024 + l * 16;
    const int prow = pb / (D * 2), slot = (pb % (D * 2)) >> 4;
    constexpr int CPR = D / 8;
    dch[i] = slot ^ ((((prow & 3) << 2) ^ ((prow >> 2) & 3)) & (CPR - 1));
    dr[i] = tile_row(prow);  // tile_row is an involution
  }
  // A tile wholly inside the sequence starts at token tq * BQ / G; relative to that token every lane's
  // source lies at the same byte offset in every tile, so those copies take a scalar base per tile and
  // a 32-bit lane offset computed once (tile columns are whole tokens: G divides BQ)
  uint32_t dlane[C::RPT];
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) dlane[i] = (uint32_t)((col_offset(dr[i], lgG, Hkv, hk, D) + dch[i] * 8) * 2);
  const int64_t token_elems = (int64_t)(Hkv << lgG) * D;  // elements per token of q / dout
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds0 + w * C::RPT * 1024);
  auto dma_full = [&](int st, int tq) {
    const int64_t tok = ((int64_t)tq * C::BQ) >> lgG;
    const bf16* qb = uniform_ptr(q + tok * token_elems);
    const bf16* ob = uniform_ptr(dout + tok * token_elems);
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      const uint32_t mq = lds_w + st * C::STAGE + C::Q_OFF + i * 1024;
      const uint32_t md = mq + (C::DO_OFF - C::Q_OFF);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(mq), "v"(dlane[i]),
                   "s"(qb) : "memory", "m0");
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(md), "v"(dlane[i]),
                   "s"(ob) : "memory", "m0");
    }
  };
  auto dma = [&](int st, const int64_t* off) {
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      const uint32_t mq = __builtin_amdgcn_readfirstlane(lds0 + st * C::STAGE + C::Q_OFF + (w * C::RPT + i) * 1024);
      const uint32_t md = mq + (C::DO_OFF - C::Q_OFF);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(mq), "v"(q + off[i])
                   : "memory", "m0");
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(md), "v"(dout + off[i])
                   : "memory", "m0");
    }
  };
  auto dma_wait = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  const int hq_col = (hk << lgG) + (tid & (G - 1));   // query head of aux column tid (tc0 is a multiple of G)
  int arow = (int)(((int64_t)tq_hi * C::BQ + tid) >> lgG);
  int64_t acol = (int64_t)tq_hi * C::BQ + tid;
  auto gload_first = [&](int tq) {  // into stage 0
    const int64_t tc0 = (int64_t)tq * C::BQ;
    int64_t off[C::RPT];
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      // columns past the end read the last column instead (their P and dS are
      // masked to zero), so the copies carry no branch
      const int64_t c = min<int64_t>(tc0 + dr[i], NG - 1);
      off[i] = col_offset(c, lgG, Hkv, hk, D) + dch[i] * 8;
    }
    dma(0, off);
    if (tid < C::BQ) {
      const int64_t c = min<int64_t>(tc0 + tid, NG - 1);
      const int row = (int)(c >> lgG);
      const int h = (hk << lgG) + (int)(c & (G - 1));
      a_lse = lse[(int64_t)h * N + row];  // scaled by log2(e) when stored, after the load has landed
      a_dl = delta[(int64_t)hk * NG + c];
    }
  };
  auto gload_next = [&](int st, int tq) {  // the tile below the one loaded last (always inside the sequence)
    dma_full(st, tq);
    arow -= C::BQ >> lgG;
    acol -= C::BQ;
    if (tid < C::BQ) {
      a_lse = lse[(int64_t)hq_col * N + arow];
      a_dl = delta[(int64_t)hk * NG + acol];
    }
  };
  auto lstore = [&](int st) {  // the aux values of the tile copied last
    char* b = smem + st * C::STAGE;
    if (tid < C::BQ) {
      float* af = reinterpret_cast<float*>(b + C::AUX_OFF);
      af[tid] = a_lse * kLog2e;
      af[C::BQ + tid] = -a_dl;  // stored negated: it seeds the dP accumulator
    }
  };

  // Query tiles are visited from the document end downwards: the work-groups
  // resident at the same time hold adjacent key blocks, so they all start at
  // the same tile and stream the same Q / dO tiles through L2 in step.
  gload_first(tq_hi);
  lstore(0);
  dma_wait();
  __syncthreads();
  const char* kl = smem + C::K_LDS + (kbw * 32 + lc) * C::KSTR + g * 16;
  const char* vl = smem + C::V_LDS + (kbw * 32 + lc) * C::KSTR + g * 16;
  // two tiles per iteration so that each tile's LDS stage is a compile-time
  // constant (operand addresses then differ by immediate offsets only)
  auto tile = [&](auto stage, int tq) {
    constexpr int st = decltype(stage)::value;
    if (tq > tq_lo) gload_next(st ^ 1, tq - 1);  // the other stage is free since the last barrier
    const char* b = smem + st * C::STAGE;
    const float* aux_lse = reinterpret_cast<const float*>(b + C::AUX_OFF);
    const float* aux_dl = aux_lse + C::BQ;
    const int64_t tc0 = (int64_t)tq * C::BQ;
    const int first_row = (int)(tc0 >> lgG);
    const int last_row = (int)(min<int64_t>(NG - 1, tc0 + C::BQ - 1) >> lgG);
    const bool need_mask = first_row < kb_last || last_row > de0 || tc0 + C::BQ > NG;

    // register i holds query column qh*32 + (i>>3)*16 + g*8 + (i&7) of the
    // tile; dP accumulates onto -delta of its column, so the MFMAs give dP - delta
    f32x16 s, dp;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cb = qh * 32 + half * 16 + g * 8;
      const f32x4 d0 = *reinterpret_cast<const f32x4*>(aux_dl + cb);
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(aux_dl + cb + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dp[half * 8 + e] = d0[e];
        dp[half * 8 + 4 + e] = d1[e];
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 aq = *reinterpret_cast<const bf16x8*>(b + C::Q_OFF + lds_off<D>(qh * 32 + lc, ks * 2 + g));
      const bf16x8 bk = *reinterpret_cast<const bf16x8*>(kl + ks * 32);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, bk, s, 0, 0, 0);
      const bf16x8 ad = *reinterpret_cast<const bf16x8*>(b + C::DO_OFF + lds_off<D>(qh * 32 + lc, ks * 2 + g));
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(vl + ks * 32);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad, bv, dp, 0, 0, 0);
    }
    // schedule: the operand reads run three MFMAs ahead of the S and dP MFMAs
    // (the delta seeds are read first);
    // the fence keeps the softmax's LDS reads out of this phase (hoisted, they
    // hold registers the read-ahead needs)
    __builtin_amdgcn_sched_group_barrier(0x100, 6 + 4, 0);  // + the 4 delta seed reads
#pragma unroll
    for (int j = 0; j < 2 * (D / 16) - 3; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 pr, dsr;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int cb = qh * 32 + half * 16 + g * 8;
      const f32x4 l0 = *reinterpret_cast<const f32x4*>(aux_lse + cb);
      const f32x4 l1 = *reinterpret_cast<const f32x4*>(aux_lse + cb + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = half * 8 + e;
        const float lv = e < 4 ? l0[e] : l1[e - 4];
        pr[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl2, -lv));
        dsr[i] = dp[i];
      }
    }
    // one uniform branch around the masking of the whole tile (branch-free inside)
    if (need_mask) {
      // register i holds tile column cbase + (i>>3)*16 + (i&7); visible iff that
      // offset lies in [lo, lo + span]
      const int cbase = qh * 32 + g * 8;
      const int c0 = (int)tc0 + cbase;
      int lo = min(key, N) * G - c0;  // keys past the end: lo > hi below
      const int hi = col_end - 1 - c0;
      unsigned span = (unsigned)(hi - lo);
      if (hi < lo) {
        lo = 1 << 30;
        span = 0u;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = (i >> 3) * 16 + (i & 7);
        pr[i] = (unsigned)(off - lo) <= span ? pr[i] : 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dsr[i] *= pr[i];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 bp = pack8(pr, kk * 8);
      const bf16x8 bs = pack8(dsr, kk * 8);
      const int k0 = qh * 32 + kk * 16;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 adot = lds_tr_a<D>(b + C::DO_OFF, db * 32, k0, l);
        dvt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(adot, bp, dvt[db], 0, 0, 0);
        const bf16x8 aqt = lds_tr_a<D>(b + C::Q_OFF, db * 32, k0, l);
        dkt[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aqt, bs, dkt[db], 0, 0, 0);
      }
    }
    // schedule: 4 transpose reads in flight ahead of the dV/dK MFMAs (two per MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int j = 0; j < D / 8 - 2; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    if (tq > tq_lo) lstore(st ^ 1);
    dma_wait();
    __syncthreads();
  };
  for (int tq = tq_hi; tq >= tq_lo; tq -= 2) {
    tile(std::integral_constant<int, 0>(), tq);
    if (tq - 1 < tq_lo) break;
    tile(std::integral_constant<int, 1>(), tq - 1);
  }

  // sum the two halves: the upper waves hand their partial sums to the lower
  // ones through LDS (dK^T first, then dV^T)
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          red[((kbw * (D / 32) + db) * 16 + i) * 64 + l] = which == 0 ? dkt[db][i] : dvt[db][i];
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = red[((kbw * (D / 32) + db) * 16 + i) * 64 + l];
          if (which == 0) dkt[db][i] += x; else dvt[db][i] += x;
        }
    }
    __syncthreads();
  }

  if (qh == 0 && kvalid) {
    const int64_t base = ((int64_t)key * Hkv + hk) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + j * 8 + g * 4;
        f32x4 a, bb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = dkt[db][j * 4 + e] * scale;
          bb[e] = dvt[db][j * 4 + e];
        }
        if (accumulate) {  // the earlier windows' sums, in window order
          a += *reinterpret_cast<const f32x4*>(dk + base + d);
          bb += *reinterpret_cast<const f32x4*>(dv + base + d);
        }
        *reinterpret_cast<f32x4*>(dk + base + d) = a;
        *reinterpret_cast<f32x4*>(dv + base + d) = bb;
      }
  }
}

// ---------------------------------------------------------------------- dQ --
template <int D, int NW>
struct DqCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int BN = 64;            // keys per tile
  static constexpr int BMC = NW * 32;      // query columns per work-group
  static constexpr int RSTR = D * 2;       // LDS bytes per K / V row (swizzled, unpadded)
  static constexpr int RBYTES = BN * RSTR;
  static constexpr int K_OFF = 0, V_OFF = RBYTES;
  static constexpr int STAGE = 2 * RBYTES;
  static constexpr int RCH = BN * D / 8;
  static constexpr int RPT = RCH / kThreads;
  static_assert(RCH % kThreads == 0, "tile chunks must split evenly");
};

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) dq_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ doc_start, const int32_t* __restrict__ order, float* __restrict__ dq, int N,
    int Hkv, int lgG, float sl2, float scale) {
  using C = DqCfg<D, NW>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::STAGE];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lc = l & 31;
  const int G = 1 << lgG;
  const int hk = blockIdx.x % Hkv;
  const int cb = order[blockIdx.x / Hkv];  // heaviest column blocks first
  const int64_t NG = (int64_t)N << lgG;
  const int64_t c0 = (int64_t)cb * C::BMC;
  const int r_first = (int)(c0 >> lgG);
  const int r_last = (int)min<int64_t>(N - 1, (c0 + C::BMC - 1) >> lgG);
  const int t_lo = doc_start[r_first] / C::BN;
  const int t_hi = r_last / C::BN;
  const int ds_last = doc_start[r_last];

  const int64_t c = c0 + w * 32 + lc;
  const bool cvalid = c < NG;
  const int row = cvalid ? (int)(c >> lgG) : -1;
  const int ds_c = cvalid ? doc_start[row] : 0;
  const int64_t qoff = cvalid ? col_offset(c, lgG, Hkv, hk, D) : 0;
  float lse2 = 0.0f, dl = 0.0f;
  bf16x8 qreg[D / 16], doreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (cvalid) {
      qreg[ks] = *reinterpret_cast<const bf16x8*>(q + qoff + ks * 16 + g * 8);
      doreg[ks] = *reinterpret_cast<const bf16x8*>(dout + qoff + ks * 16 + g * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) { qreg[ks][e] = (bf16)0.0f; doreg[ks][e] = (bf16)0.0f; }
    }
  }
  if (cvalid) {
    const int h = (hk << lgG) + (int)(c & (G - 1));
    lse2 = lse[(int64_t)h * N + row] * kLog2e;
    dl = delta[(int64_t)hk * NG + c];
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;

  u32x4 rk[C::RPT], rv[C::RPT];
  auto gload = [&](int t) {
    const int t0 = t * C::BN;
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      const int ch = tid + i * C::kThreads;
      const int r = ch / (D / 8), part = ch % (D / 8);
      // keys past the end read the last key instead (their P is masked to zero)
      const int kv = min(t0 + r, N - 1);
      const int64_t off = ((int64_t)kv * Hkv + hk) * D + part * 8;
      rk[i] = *reinterpret_cast<const u32x4*>(k + off);
      rv[i] = *reinterpret_cast<const u32x4*>(v + off);
    }
  };
  auto lstore = [&](int st) {
    char* b = smem + st * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      const int ch = tid + i * C::kThreads;
      const int r = ch / (D / 8), part = ch % (D / 8);
      *reinterpret_cast<u32x4*>(b + C::K_OFF + lds_off<D>(tile_row(r), part)) = rk[i];
      *reinterpret_cast<u32x4*>(b + C::V_OFF + lds_off<D>(tile_row(r), part)) = rv[i];
    }
  };

  gload(t_lo);
  lstore(0);
  __syncthreads();
  for (int t = t_lo; t <= t_hi; ++t) {
    const int st = (t - t_lo) & 1;
    if (t < t_hi) gload(t + 1);
    const char* b = smem + st * C::STAGE;
    const int t0 = t * C::BN;
    const bool need_mask = t0 + C::BN - 1 > r_first || t0 < ds_last;
    // the two 32-key halves one after the other: S^T, dP^T, dS^T, then dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) { s[i] = 0.0f; dp[i] = 0.0f; }
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(b + C::K_OFF + lds_off<D>(kb * 32 + lc, ks * 2 + g));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qreg[ks], s, 0, 0, 0);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(b + C::V_OFF + lds_off<D>(kb * 32 + lc, ks * 2 + g));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, doreg[ks], dp, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl2, -lse2));
      // one uniform branch around the masking (branch-free inside)
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kv = t0 + kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          s[i] = (kv <= row && kv >= ds_c) ? s[i] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] *= dp[i] - dl;  // dS^T
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const bf16x8 bs = pack8(s, half * 8);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8 a = lds_tr_a<D>(b + C::K_OFF, db * 32, kb * 32 + half * 16, l);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs, acc[db], 0, 0, 0);
        }
      }
    }
    if (t < t_hi) lstore(st ^ 1);
    __syncthreads();
  }

  if (cvalid) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = acc[db][j * 4 + e] * scale;
        *reinterpret_cast<f32x4*>(dq + qoff + db * 32 + j * 8 + g * 4) = a;
      }
  }
}

// ------------------------------------------------------ dQ, one wave per SIMD --
// The same product as dq_kernel, for D = 128, with one wave per SIMD (512
// registers per lane).  A wave owns 64 query columns (two 32-column blocks), so
// every K, V and K^T fragment read from LDS feeds two MFMAs: half the LDS
// operand bytes per MFMA of dq_kernel, which is what bounds these kernels.  Q
// and dO (the B operands) and the dQ^T accumulators live in AGPRs for the whole
// key loop; the MFMAs are inline assembly so that the compiler keeps them
// there.  Each 32-key half-tile runs as S^T/dP^T MFMAs, then its softmax VALU
// work interleaved with the next half's S^T/dP^T MFMAs, then its dQ MFMAs.
// K/V tiles go global -> LDS by DMA into a ring of four stages, each copy two
// tiles ahead (a tile's K^T is still read for its second half's dQ after the
// next tile's first half).
//
// The compiler does not know that the asm statements are MFMAs, so it neither
// inserts the wait states the hardware needs around them nor keeps their
// operands from being reused too early.  The kernel supplies both:
//  * s_nop fences, with the registers as "+" operands, between an MFMA and the
//    first non-MFMA read of its result (q1_fence4, q1_fence_acc), and between a
//    VALU write and an MFMA reading it (q1_fence_pk);
//  * empty asm statements that use an MFMA's A operand in the slots after it,
//    so nothing is placed in its registers while the MFMA still reads them;
//  * no register copies into an accumulator: the first dQ MFMAs of a column
//    block start from C = 0 instead of a zero fill, and Q / dO are loaded
//    straight into AGPRs.
// A compile-time test scans the kernel's machine code for the two hazards.
template <int D>
struct Dq1wCfg {
  static constexpr int kThreads = 256;
  static constexpr int BN = 64;
  static constexpr int BMC = 256;
  static constexpr int RSTR = D * 2;
  static constexpr int RBYTES = BN * RSTR;
  static constexpr int K_OFF = 0, V_OFF = RBYTES;
  static constexpr int STAGE = 2 * RBYTES;
  static constexpr int NS = 4;
  static constexpr int RPT = BN * D / 8 / kThreads;
  static_assert(RPT * kThreads * 8 == BN * D, "tile copies must split evenly");
};

__device__ __forceinline__ void q1_mfma_v0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void q1_mfma_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// the first MFMA of a chain seeded with a register block the chain does not overwrite
__device__ __forceinline__ void q1_mfma_vc(f32x16& d, const bf16x8& a, const bf16x8& b, const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "a"(b), "v"(c));
}
__device__ __forceinline__ void q1_mfma_a0(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void q1_mfma_a(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// wait states after the last MFMA writing these (the compiler does not see the MFMAs)
__device__ __forceinline__ void q1_fence4(f32x16& a, f32x16& b, f32x16& c, f32x16& d) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
__device__ __forceinline__ void q1_fence_pk(bf16x8 (&p)[2][2]) {
  asm volatile("s_nop 4" : "+v"(p[0][0]), "+v"(p[0][1]), "+v"(p[1][0]), "+v"(p[1][1]));
}
template <int NB>
__device__ __forceinline__ void q1_fence_acc(f32x16 (&acc)[2][NB]) {
  if constexpr (NB == 4)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2"
                 : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                   "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3]));
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[1][0]), "+a"(acc[1][1]));
}
// keeps a register value live at this point
__device__ __forceinline__ void q1_keep(const bf16x8& x) { asm volatile("" ::"v"(x)); }
// four 16-byte fragments straight into AGPRs (waits in the same block)
__device__ __forceinline__ void q1_load4(bf16x8& r0, bf16x8& r1, bf16x8& r2, bf16x8& r3, const bf16* p, int stride) {
  asm volatile(
      "global_load_dwordx4 %0, %4, off\n\tglobal_load_dwordx4 %1, %5, off\n\t"
      "global_load_dwordx4 %2, %6, off\n\tglobal_load_dwordx4 %3, %7, off\n\ts_waitcnt vmcnt(0)"
      : "=&a"(r0), "=&a"(r1), "=&a"(r2), "=&a"(r3)
      : "v"(p), "v"(p + stride), "v"(p + 2 * stride), "v"(p + 3 * stride)
      : "memory");
}

template <int B, int E, class F>
__device__ __forceinline__ void q1_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    q1_for<B + 1, E>(f);
  }
}

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) dq_kernel_1w(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    const bf16* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ doc_start, const int32_t* __restrict__ order, float* __restrict__ dq, int N,
    int Hkv, int lgG, float sl2, float scale) {
  using C = Dq1wCfg<D>;
  __shared__ __attribute__((aligned(16))) char smem[C::NS * C::STAGE];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lc = l & 31;
  const int G = 1 << lgG;
  const int hk = blockIdx.x % Hkv;
  const int cb = order[blockIdx.x / Hkv];
  const int64_t NG = (int64_t)N << lgG;
  const int64_t c0 = (int64_t)cb * C::BMC;
  const int r_first = (int)(c0 >> lgG);
  const int r_last = (int)min<int64_t>(N - 1, (c0 + C::BMC - 1) >> lgG);
  const int t_lo = doc_start[r_first] / C::BN;
  const int t_hi = r_last / C::BN;
  const int ds_last = doc_start[r_last];

  int row[2], ds_c[2];
  bool cvalid[2];
  int64_t qoff[2];
  float lse2[2], dl[2];
  bf16x8 qreg[2][D / 16], doreg[2][D / 16];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t c = c0 + w * 64 + j * 32 + lc;
    cvalid[j] = c < NG;
    row[j] = cvalid[j] ? (int)(c >> lgG) : -1;
    ds_c[j] = cvalid[j] ? doc_start[row[j]] : 0;
    qoff[j] = cvalid[j] ? col_offset(c, lgG, Hkv, hk, D) : 0;  // a column past the end reads column 0
    lse2[j] = 0.0f;
    dl[j] = 0.0f;
    if (cvalid[j]) {
      const int h = (hk << lgG) + (int)(c & (G - 1));
      lse2[j] = lse[(int64_t)h * N + row[j]] * kLog2e;
      dl[j] = delta[(int64_t)hk * NG + c];
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ks += 4) {
      q1_load4(qreg[j][ks], qreg[j][ks + 1], qreg[j][ks + 2], qreg[j][ks + 3], q + qoff[j] + ks * 16 + g * 8, 16);
      q1_load4(doreg[j][ks], doreg[j][ks + 1], doreg[j][ks + 2], doreg[j][ks + 3], dout + qoff[j] + ks * 16 + g * 8,
               16);
    }
  }
  f32x16 acc[2][D / 32];  // set by the first tile's first dQ MFMAs (no zero fill to copy between registers)
  // -Delta of the lane's column in each 32-column half: the seeds of that half's dP^T chains, so they
  // produce dP - Delta directly (every lane's 16 values of a dP^T block belong to its one column); the
  // two blocks push the column offsets out to scratch across the loop (reloaded for the final stores)
  f32x16 ndl0;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndl0[i] = -dl[0];
  f32x16 ndl1;
#pragma unroll
  for (int i = 0; i < 16; ++i) ndl1[i] = -dl[1];

  // DMA of a K / V tile: lane l of wave w's i-th copy fills byte (w * RPT + i) * 1024 + 16 l of the tile,
  // the row and chunk the permuted, swizzled layout keeps there; keys past the end read the last key
  int kr[C::RPT];
  uint32_t kco[C::RPT];
#pragma unroll
  for (int i = 0; i < C::RPT; ++i) {
    const int pb = (w * C::RPT + i) * 1024 + l * 16;
    const int prow = pb / (D * 2), slot = (pb % (D * 2)) >> 4;
    constexpr int CPR = D / 8;
    kco[i] = (uint32_t)((slot ^ ((((prow & 3) << 2) ^ ((prow >> 2) & 3)) & (CPR - 1))) * 16);
    kr[i] = tile_row(prow);
  }
  const uint32_t kstride = (uint32_t)(Hkv * D * 2);
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  auto dma = [&](int t, int st) __attribute__((always_inline)) {
    const int t0 = t * C::BN;
    const int lim = N - 1 - t0;
    const bf16* kbase = uniform_ptr(k + ((int64_t)t0 * Hkv + hk) * D);
    const bf16* vbase = uniform_ptr(v + ((int64_t)t0 * Hkv + hk) * D);
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) {
      const uint32_t off = (uint32_t)min(kr[i], lim) * kstride + kco[i];
      const uint32_t mk = __builtin_amdgcn_readfirstlane(lds0 + st * C::STAGE + C::K_OFF + (w * C::RPT + i) * 1024);
      const uint32_t mv = mk + (C::V_OFF - C::K_OFF);
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(mk), "v"(off), "s"(kbase)
                   : "memory", "m0");
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(mv), "v"(off), "s"(vbase)
                   : "memory", "m0");
    }
  };
  auto dma_wait = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  // all but the last tile's copies (2 * RPT per thread) done
  auto dma_wait_prev = [&]() __attribute__((always_inline)) {
    static_assert(2 * C::RPT == 8, "copies per tile and thread");
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  };

  // K^T fragments by transpose reads (as lds_tr_a): the lane's byte offsets within a tile for each 32-row
  // block db of K^T and each of its two reads, so that the key-block and k-step parts of an address are
  // immediate offsets (the row permutation and the chunk swizzle only touch the low four row bits)
  int toff[D / 32][2];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = l >> 4, s = l & 15;
      const int n = db * 32 + (m & 1) * 16 + 4 * (s & 3);
      const int x = (m >> 1) * 8 + (s >> 2) + h * 4;
      toff[db][h] = lds_off<D>(tile_row(x), n >> 3) + (n & 7) * 2;
    }
  auto lds_tr_k = [&](const char* tile, int db, int k0) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + k0 * (D * 2) + toff[db][0]));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + k0 * (D * 2) + toff[db][1]));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_bit_cast(bf16x8, r);
  };

  // half-tile buffers: A for first halves (keys 0-31 of a tile), B for second halves
  f32x16 sA[2], dpA[2], sB[2], dpB[2];
  bf16x8 pkA[2][2], pkB[2][2];

  // softmax work of one half-tile in 30 steps: per column block eight steps of two exponentials, the
  // mask, four steps of dS, two of packing
  struct Half {
    f32x16* s;
    f32x16* dp;
    bf16x8 (*pk)[2];
    int t, kb;
    bool msk;
  };
  auto vstep = [&](auto k_c, const Half& h) __attribute__((always_inline)) {
    constexpr int kk = decltype(k_c)::value;
    constexpr int j = kk / 15, st = kk % 15;
    f32x16& sj = h.s[j];
    if constexpr (st < 8) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = st * 2 + e;
        sj[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sj[i], sl2, -lse2[j]));
      }
    } else if constexpr (st == 8) {
      if (h.msk) {
        const int t0 = h.t * C::BN;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kv = t0 + h.kb * 32 + (i >> 3) * 16 + g * 8 + (i & 7);
          sj[i] = (kv <= row[j] && kv >= ds_c[j]) ? sj[i] : 0.0f;
        }
      }
    } else if constexpr (st < 13) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = (st - 9) * 4 + e;
        sj[i] *= h.dp[j][i];  // the chain started from -Delta
      }
    } else {
      h.pk[j][st - 13] = pack8(sj, (st - 13) * 8);
    }
  };
  constexpr int NVSTEP = 30;
  auto pin = [&](const Half& h) __attribute__((always_inline)) {
    asm volatile("" : "+v"(h.s[0]), "+v"(h.s[1]), "+v"(h.pk[0][0]), "+v"(h.pk[0][1]), "+v"(h.pk[1][0]),
                 "+v"(h.pk[1][1]));
  };

  // operand ring of the S/dP phases: K and V fragments two ks steps ahead; a phase's first two are
  // read during the phase before it where that phase allows
  bf16x8 ak[3], av[3];
  // the lane's byte offset of its K / V row chunk for each ks within a 32-key block (the block's rows are
  // an immediate offset)
  int koff[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) koff[ks] = lds_off<D>(lc, ks * 2 + g);
  auto rd = [&](const char* sb, int kb, int ks, int x) __attribute__((always_inline)) {
    ak[x] = *reinterpret_cast<const bf16x8*>(sb + C::K_OFF + kb * 32 * (D * 2) + koff[ks]);
    av[x] = *reinterpret_cast<const bf16x8*>(sb + C::V_OFF + kb * 32 * (D * 2) + koff[ks]);
  };
  // S^T and dP^T of half kb of the tile in stage `sb` into (s, dp), with softmax steps [VLO, VHI) of
  // half-tile h between the MFMAs
  auto sdp = [&](const char* sb, auto kb_c, f32x16 (&s)[2], f32x16 (&dp)[2], auto vlo_c, auto vhi_c, const Half& h,
                 bool pre) __attribute__((always_inline)) {
    constexpr int kb = decltype(kb_c)::value;
    constexpr int VLO = decltype(vlo_c)::value, VHI = decltype(vhi_c)::value;
    if (!pre) {
      rd(sb, kb, 0, 0);
      rd(sb, kb, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NSLOT = 4 * (D / 16);
    q1_for<0, NSLOT>([&](auto m_c) __attribute__((always_inline)) {
      constexpr int m = decltype(m_c)::value, ks = m / 4, sub = m % 4;
      if constexpr (sub == 2 && ks + 2 < D / 16) {
        // the fragments replaced here were last MFMA sources two or more slots ago; keeping them live
        // until the load stops the compiler from putting temporaries there in between
        asm volatile("" ::"v"(ak[(ks + 2) % 3]), "v"(av[(ks + 2) % 3]));
        rd(sb, kb, ks + 2, (ks + 2) % 3);
      }
      if constexpr (sub == 0) {
        if constexpr (ks == 0) q1_mfma_v0(s[0], ak[0], qreg[0][0]); else q1_mfma_v(s[0], ak[ks % 3], qreg[0][ks]);
      } else if constexpr (sub == 1) {
        if constexpr (ks == 0) q1_mfma_v0(s[1], ak[0], qreg[1][0]); else q1_mfma_v(s[1], ak[ks % 3], qreg[1][ks]);
      } else if constexpr (sub == 2) {
        if constexpr (ks == 0) q1_mfma_vc(dp[0], av[0], doreg[0][0], ndl0); else q1_mfma_v(dp[0], av[ks % 3], doreg[0][ks]);
      } else {
        if constexpr (ks == 0) q1_mfma_vc(dp[1], av[0], doreg[1][0], ndl1); else q1_mfma_v(dp[1], av[ks % 3], doreg[1][ks]);
      }
      if constexpr (VHI > VLO) {
        constexpr int lo = VLO + m * (VHI - VLO) / NSLOT, hi = VLO + (m + 1) * (VHI - VLO) / NSLOT;
        q1_for<lo, hi>([&](auto k_c) __attribute__((always_inline)) { vstep(k_c, h); });
        pin(h);  // without a use here the compiler sinks the softmax to its consumers
      }
      // the A operands of this slot's and the two previous slots' MFMAs stay in their registers through
      // this slot (nothing the compiler places here may overwrite an operand an MFMA is still reading)
      q1_for<(m >= 2 ? m - 2 : 0), m + 1>([&](auto p_c) __attribute__((always_inline)) {
        constexpr int pm = decltype(p_c)::value, pks = pm / 4, psub = pm % 4;
        if constexpr (psub < 2)
          q1_keep(ak[pks % 3]);
        else
          q1_keep(av[pks % 3]);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    q1_fence4(s[0], s[1], dp[0], dp[1]);
    asm volatile("" ::"v"(ak[0]), "v"(ak[1]), "v"(ak[2]), "v"(av[0]), "v"(av[1]), "v"(av[2]));
  };
  // softmax steps [VLO, VHI) of half-tile h alone
  auto valu = [&](auto vlo_c, auto vhi_c, const Half& h) __attribute__((always_inline)) {
    constexpr int VLO = decltype(vlo_c)::value, VHI = decltype(vhi_c)::value;
    q1_for<VLO, VHI>([&](auto k_c) __attribute__((always_inline)) { vstep(k_c, h); });
  };
  // dQ^T += K^T dS^T for half kb of the tile in stage `sb` (dS packed in pk); optionally the next S/dP
  // phase's first operand reads
  auto dqp = [&](const char* sb, auto kb_c, bf16x8 (&pk)[2][2], const char* nsb, int nkb, auto first_c)
                 __attribute__((always_inline)) {
    constexpr int kb = decltype(kb_c)::value;
    constexpr bool first = decltype(first_c)::value;  // the accumulators' first products
    constexpr int NF = 2 * (D / 32);  // K^T fragments: (kk, db)
    q1_fence_pk(pk);
    bf16x8 ta[4];
    auto tr = [&](int f, int x) __attribute__((always_inline)) {
      ta[x] = lds_tr_k(sb + C::K_OFF, f % (D / 32), kb * 32 + (f / (D / 32)) * 16);
    };
    tr(0, 0);
    tr(1, 1);
    if (nsb != nullptr) {  // the next S/dP phase's first operands
      rd(nsb, nkb, 0, 0);
      rd(nsb, nkb, 1, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
    constexpr int NSLOT = NF;
    q1_for<0, NSLOT>([&](auto m_c) __attribute__((always_inline)) {
      constexpr int f = decltype(m_c)::value, kk = f / (D / 32), db = f % (D / 32);
      if constexpr (f + 2 < NF) tr(f + 2, (f + 2) % 4);
      if constexpr (first && kk == 0) {
        q1_mfma_a0(acc[0][db], ta[f % 4], pk[0][kk]);
        q1_mfma_a0(acc[1][db], ta[f % 4], pk[1][kk]);
      } else {
        q1_mfma_a(acc[0][db], ta[f % 4], pk[0][kk]);
        q1_mfma_a(acc[1][db], ta[f % 4], pk[1][kk]);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    // the last MFMAs' sources stay in their registers until these MFMAs have read them
    asm volatile("s_nop 7\n\ts_nop 7" ::"v"(pk[0][0]), "v"(pk[0][1]), "v"(pk[1][0]), "v"(pk[1][1]), "v"(ta[0]),
                 "v"(ta[1]), "v"(ta[2]), "v"(ta[3]));
  };
  auto need_mask = [&](int t) __attribute__((always_inline)) {
    const int t0 = t * C::BN;
    return t0 + C::BN - 1 > r_first || t0 < ds_last;
  };
  using K0 = std::integral_constant<int, 0>;
  using K1 = std::integral_constant<int, 1>;
  using V0 = std::integral_constant<int, 0>;
  using VN = std::integral_constant<int, NVSTEP>;
  using FIRST = std::integral_constant<bool, true>;
  using NOTFIRST = std::integral_constant<bool, false>;

  dma(t_lo, 0);
  if (t_lo + 1 <= t_hi) {
    dma(t_lo + 1, 1);
    dma_wait_prev();
  } else {
    dma_wait();
  }
  __syncthreads();
  // phases: S(t,0) | dQ(t-1,1) | S(t,1) | dQ(t,0) | S(t+1,0) | ...; the softmax of a half-tile runs in
  // the next S/dP phase
  const Half hA0{sA, dpA, pkA, t_lo, 0, false};
  {
    const char* cur = smem;
    const bool ahead = t_lo + 2 <= t_hi;
    if (ahead) dma(t_lo + 2, 2);  // two tiles ahead: tile t_lo + 1 is in flight already
    const Half hA{sA, dpA, pkA, t_lo, 0, need_mask(t_lo)};
    sdp(cur, K0(), sA, dpA, V0(), V0(), hA0, false);
    sdp(cur, K1(), sB, dpB, V0(), VN(), hA, false);  // (t_lo, 1st half)'s softmax
    dqp(cur, K0(), pkA, nullptr, 0, FIRST());
    q1_fence_acc(acc);  // the accumulators may be copied between register sets at the loop entry
    if (ahead) dma_wait_prev(); else dma_wait();  // tile t_lo + 1 has landed
    __syncthreads();
  }
  for (int t = t_lo + 1; t <= t_hi; ++t) {
    const int u = t - t_lo;
    const char* cur = smem + (u % 4) * C::STAGE;
    const char* prv = smem + ((u + 3) % 4) * C::STAGE;
    const bool ahead = t + 2 <= t_hi;
    if (ahead) dma(t + 2, (u + 2) % 4);  // into tile t - 2's stage, last read before the previous barrier
    const Half hBp{sB, dpB, pkB, t - 1, 1, need_mask(t - 1)};
    const Half hA{sA, dpA, pkA, t, 0, need_mask(t)};
    sdp(cur, K0(), sA, dpA, V0(), VN(), hBp, false);  // (t-1, 2nd half)'s softmax
    dqp(prv, K1(), pkB, cur, 1, NOTFIRST());
    sdp(cur, K1(), sB, dpB, V0(), VN(), hA, true);    // (t, 1st half)'s softmax
    dqp(cur, K0(), pkA, nullptr, 0, NOTFIRST());
    q1_fence_acc(acc);
    if (ahead) dma_wait_prev(); else dma_wait();  // tile t + 1 has landed
    __syncthreads();
  }
  // the last tile's second half
  {
    const Half hB{sB, dpB, pkB, t_hi, 1, need_mask(t_hi)};
    valu(V0(), VN(), hB);
    dqp(smem + ((t_hi - t_lo) % 4) * C::STAGE, K1(), pkB, nullptr, 0, NOTFIRST());
  }
  q1_fence_acc(acc);

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!cvalid[j]) continue;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        f32x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = acc[j][db][jj * 4 + e] * scale;
        *reinterpret_cast<f32x4*>(dq + qoff[j] + db * 32 + jj * 8 + g * 4) = a;
      }
  }
}

int ilog2_pow2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Query tiles per dK / dV window (2048 tiles of 64 columns: 32768 tokens of a
// 4-head group, 64 MiB of Q and dO tiles).
constexpr int kDkvWindowTiles = 2048;

}  // namespace

hipError_t launch_attn_bwd_bf16(const bf16* q, const bf16* k, const bf16* v, const bf16* o, const bf16* dout,
                                const float* lse, const int32_t* doc_start, const int32_t* doc_end, float* dq,
                                float* dk, float* dv, float* delta, int32_t* order_col, int32_t* order_key, int N,
                                int Hq, int Hkv, int D, float scale, hipStream_t s) {
  const int G = Hq / Hkv;
  const int lgG = ilog2_pow2(G);
  const int64_t NG = (int64_t)N * G;
  const float sl2 = scale * kLog2e;
  constexpr int NW = 8;
  static_assert(DkvCfg<128>::BNK == kKeyBlock && DkvCfg<128>::BQ == kColTile, "unit sizes of the order");
  static_assert(DkvCfg<64>::BNK == kKeyBlock && DkvCfg<64>::BQ == kColTile, "unit sizes of the order");
  static_assert(Dq1wCfg<128>::BMC == kColBlock && Dq1wCfg<128>::BN == kKeyTile, "unit sizes of the order");
  static_assert(DqCfg<64, NW>::BMC == kColBlock && DqCfg<64, NW>::BN == kKeyTile, "unit sizes of the order");
  const int nkb = (int)key_blocks(N), ncb = (int)col_blocks(N, G);
  {
    OrderJobs jobs{};
    jobs.j[0] = OrderJob{order_key, doc_end, 1, nkb, kKeyBlock, kColTile};
    jobs.j[1] = OrderJob{order_col, doc_start, 0, ncb, kColBlock, kKeyTile};
    hipError_t e = launch_order(jobs, 2, N, lgG, s);
    if (e != hipSuccess) return e;
  }
  {
    const int cpb = 256 / (D / 8);
    const dim3 grid((unsigned)((NG + cpb - 1) / cpb), Hkv);
    TimedLaunch timer("attn_bwd_delta", s);
    if (D == 128)
      hipLaunchKernelGGL(delta_bf16_kernel<128>, grid, dim3(256), 0, s, o, dout, delta, NG, Hkv, lgG);
    else
      hipLaunchKernelGGL(delta_bf16_kernel<64>, grid, dim3(256), 0, s, o, dout, delta, NG, Hkv, lgG);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    // the diagonal windows first (they write dK / dV), then every later
    // window in increasing order (each adds to dK / dV)
    const dim3 grid((unsigned)((int64_t)nkb * Hkv));
    const int ntiles = (int)((NG + kColTile - 1) / kColTile);
    const int nwin = (ntiles + kDkvWindowTiles - 1) / kDkvWindowTiles;
    for (int win = -1; win < nwin; ++win) {
      if (win == 0) continue;  // no key block sees window 0 from below
      TimedLaunch timer("attn_bwd_dkdv", s);
      if (D == 128)
        hipLaunchKernelGGL(dkdv_kernel<128>, grid, dim3(DkvCfg<128>::kThreads), 0, s, q, k, v, dout, lse, delta,
                           doc_start, doc_end, order_key, dk, dv, N, Hkv, lgG, sl2, scale, kDkvWindowTiles, win);
      else
        hipLaunchKernelGGL(dkdv_kernel<64>, grid, dim3(DkvCfg<64>::kThreads), 0, s, q, k, v, dout, lse, delta,
                           doc_start, doc_end, order_key, dk, dv, N, Hkv, lgG, sl2, scale, kDkvWindowTiles, win);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  {
    const dim3 grid((unsigned)((int64_t)ncb * Hkv)), block(NW * 64);
    TimedLaunch timer("attn_bwd_dq", s);
    if (D == 128)
      hipLaunchKernelGGL((dq_kernel_1w<128>), grid, dim3(Dq1wCfg<128>::kThreads), 0, s, q, k, v, dout, lse, delta,
                         doc_start, order_col, dq, N, Hkv, lgG, sl2, scale);
    else
      hipLaunchKernelGGL((dq_kernel<64, NW>), grid, block, 0, s, q, k, v, dout, lse, delta, doc_start, order_col, dq,
                         N, Hkv, lgG, sl2, scale);
  }
  return hipGetLastError();
}

}  // namespace ul
