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
//  * dq_kernel (query-outer, like the forward): a wave owns 32 query columns
//    with Q and dO in registers; S^T and dP^T are recomputed per key tile and
//    dQ^T += K^T dS^T takes K^T from the K tile by transpose reads.
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
// fetched in: with its loop starting 44 bytes into a line dQ ran 3 % slower
// than at 0, 24 or 32 bytes (same box, N = 1M, identical loop code).  The
// counts hold for the code as it stands; any change to a prologue moves its
// loop (tests/test_code_layout.py disassembles the build and checks both).
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
  UL_CODE_PAD(5);  // tile loop at 40 bytes into a 64-byte line (D = 128)
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
  const int64_t tile_step = (int64_t)C::BQ * Hkv * D;
  int64_t doff[C::RPT];
#pragma unroll
  for (int i = 0; i < C::RPT; ++i)
    doff[i] = col_offset((int64_t)tq_hi * C::BQ + dr[i], lgG, Hkv, hk, D) + dch[i] * 8;
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
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
  auto gload_next = [&](int st) {  // the tile below the one loaded last (always inside the sequence)
#pragma unroll
    for (int i = 0; i < C::RPT; ++i) doff[i] -= tile_step;
    dma(st, doff);
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
    if (tq > tq_lo) gload_next(st ^ 1);  // the other stage is free since the last barrier
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
  UL_CODE_PAD(11);  // tile loop at 24 bytes into a 64-byte line (D = 128)
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
  static_assert(DqCfg<128, NW>::BMC == kColBlock && DqCfg<128, NW>::BN == kKeyTile, "unit sizes of the order");
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
      hipLaunchKernelGGL((dq_kernel<128, NW>), grid, block, 0, s, q, k, v, dout, lse, delta, doc_start, order_col, dq,
                         N, Hkv, lgG, sl2, scale);
    else
      hipLaunchKernelGGL((dq_kernel<64, NW>), grid, block, 0, s, q, k, v, dout, lse, delta, doc_start, order_col, dq,
                         N, Hkv, lgG, sl2, scale);
  }
  return hipGetLastError();
}

}  // namespace ul
