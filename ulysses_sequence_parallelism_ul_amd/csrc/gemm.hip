// The projections on either side of the path (page "Hugging Face并行加速",
// nmedialink.com, section "Ulysses的工作原理", steps 2 and 6): each rank
// multiplies its own token shard by the projection weights.
//
// One bf16 NT GEMM on gfx950 MFMA, C[M][Nc] = A[M][K] * B[Nc][K]^T with fp32
// accumulation (A: tokens x features, B: one weight row per output feature,
// both row-major so every tile row is a contiguous run of K), and two
// epilogues:
//  * QKV projection: output column n is feature n of [q | k | v]; it is stored
//    straight into the all-to-all send blocks q_send [P][M][Hq/P][D],
//    k_send / v_send [P][M][Hkv/P][D] (block j goes to rank j), so no separate
//    pack pass reads the projection back from HBM.
//  * output projection: plain row-major y [M][Nc], reading the attention output
//    in the sequence layout [M][Hq*D] that head->seq produced, as is.
//
// Tiling: 256 x 256 output tile per work-group of 4 waves (one per SIMD), each
// wave 128 x 128 (8 x 8 blocks of v_mfma_f32_16x16x32_bf16), K in stages of 64
// double-buffered in LDS (rows of 128 bytes, 16-byte chunks XOR-swizzled by
// row), the next stage copied global -> LDS by DMA while the current one is
// multiplied, the instruction order fixed slot by slot (below), and the output
// staged through LDS so it leaves in 16-byte runs.  Work-groups are mapped so
// each XCD runs groups of 8 row tiles x 4 column tiles together, sharing every
// K stage's slices of A and B through its L2.  Under sustained load the board
// holds its power cap, and the 16x16x32 MFMA shape let it keep a higher clock
// than 32x32x16 for the same work (measured).
#include "ul_internal.h"

namespace ul {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 256;
constexpr int kRowBytes = kBK * 2;                  // 128 bytes per tile row
constexpr int kTileBytes = kBM * kRowBytes;         // 32 KiB per operand tile
constexpr int kStage = 2 * kTileBytes;              // A tile + B tile
constexpr int kDma = kTileBytes / 16 / kThreads;    // 8 copies of 16 bytes per operand and thread
constexpr int kXcds = 8;
constexpr int kGR = 8, kGC = 4;  // tile group per XCD: 8 row tiles x 4 column tiles

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

// An epilogue maps output column n to the address of its element in row 0
// and the stride between rows: element (m, n) lives at col(n).p + m * col(n).stride.
struct ColPtr {
  bf16* p;
  int64_t stride;
};

// vec(Nc): runs of eight columns starting at a multiple of 8 are contiguous and 16-byte aligned.
struct EpiRowMajor {
  bf16* y;
  int64_t ld;
  __device__ ColPtr col(int n) const { return ColPtr{y + n, ld}; }
  __device__ bool vec(int Nc) const { return (Nc & 7) == 0 && (ld & 7) == 0; }
};

struct EpiPackQKV {
  bf16 *q, *k, *v;
  int64_t M;                   // tokens of the shard
  int D, hq_r, hkv_r, qw, kw;  // head dim, heads per destination rank, q width Hq*D, k width Hkv*D
  __device__ ColPtr col(int n) const {
    bf16* base;
    int hr, f;
    if (n < qw) {
      base = q; hr = hq_r; f = n;
    } else if (n < qw + kw) {
      base = k; hr = hkv_r; f = n - qw;
    } else {
      base = v; hr = hkv_r; f = n - qw - kw;
    }
    const int h = f / D, d = f - h * D;
    const int j = h / hr, hl = h - j * hr;  // destination rank, head within its block
    // [j][m][hl][d]: row m of destination block j
    return ColPtr{base + ((int64_t)j * M * hr + hl) * D + d, (int64_t)hr * D};
  }
  __device__ bool vec(int) const { return (D & 7) == 0; }
};

template <class Epi>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_nt_bf16_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B, int64_t M, int Nc, int K,
                    int n_row_tiles, int n_col_tiles, Epi epi) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  // XCD-aware tile order: work-group b runs on XCD b % 8; the 32 consecutive
  // work-groups of one XCD form a group of 8 row tiles x 4 column tiles, whose
  // A and B slices of each K stage are shared through that XCD's L2.
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds, local = bid / kXcds;
  const int grp = (local / (kGR * kGC)) * kXcds + xcd, within = local % (kGR * kGC);
  const int ncg = (n_col_tiles + kGC - 1) / kGC;
  const int rt = (grp / ncg) * kGR + within / kGC;
  const int ct = (grp % ncg) * kGC + within % kGC;
  if (rt >= n_row_tiles || ct >= n_col_tiles) return;
  const int64_t m0 = (int64_t)rt * kBM;
  const int n0 = ct * kBN;
  const int wm = w >> 1, wn = w & 1;  // wave grid 2 x 2: 128 rows x 128 columns each

  // Copies go global -> LDS by DMA with a scalar base (the tile's first row, advanced by the K stage)
  // and a per-lane 32-bit byte offset: lane l of wave w's i-th copy fetches the 16-byte chunk of
  // tile row w * 64 + 8 i + l / 8 that the XOR-swizzled layout keeps at LDS block (w * kDma + i),
  // byte 16 l.  Rows past the end of the matrix read its last row.
  const bf16* a_tile = A + m0 * K;
  const bf16* b_tile = B + (int64_t)n0 * K;
  uint32_t oa[kDma], ob[kDma];
#pragma unroll
  for (int i = 0; i < kDma; ++i) {
    const int row = (w * kDma + i) * 8 + (l >> 3);
    const int chunk = (l & 7) ^ (row & 7);
    oa[i] = (uint32_t)((min<int64_t>(row, M - 1 - m0) * K + chunk * 8) * 2);
    ob[i] = (uint32_t)(((int64_t)min(row, Nc - 1 - n0) * K + chunk * 8) * 2);
  }
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  auto dma = [&](int kt, int st, int i) {
    const uint32_t ba = __builtin_amdgcn_readfirstlane(lds0 + st * kStage + (w * kDma + i) * 1024);
    const uint32_t bb = ba + kTileBytes;
    const bf16* sa = a_tile + kt * kBK;
    const bf16* sb = b_tile + kt * kBK;
    // one wait state between writing M0 and the LDS DMA that reads it; issued as inline assembly
    // so that the compiler does not order LDS reads of the other stage behind the copies
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(ba), "v"(oa[i]), "s"(sa)
                 : "memory", "m0");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(bb), "v"(ob[i]), "s"(sb)
                 : "memory", "m0");
  };
  auto dma_wait = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // v_mfma_f32_16x16x32_bf16: lane l holds row (column) l % 16 of a 16-row A (16-column B) block at
  // K chunk 4 ks + l / 16 of the 64-deep stage; the accumulator holds column l % 16, rows 4 (l / 16) + 0..3.
  const int r16 = l & 15, q = l >> 4;
  auto offa = [&](int i, int ks) { return swz(wm * 128 + i * 16 + r16, ks * 4 + q); };
  auto offb = [&](int j, int ks) { return kTileBytes + swz(wn * 128 + j * 16 + r16, ks * 4 + q); };

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;

  bf16x8 fa0[8], fb0[8], fa1[8], fb1[8];
  // one operand fragment: x < 8 is row block x of A, else column block x - 8 of B
  auto rd1 = [&](const char* s, int ks, bf16x8* fa, bf16x8* fb, int x) {
    if (x < 8)
      fa[x] = *reinterpret_cast<const bf16x8*>(s + offa(x, ks));
    else
      fb[x - 8] = *reinterpret_cast<const bf16x8*>(s + offb(x - 8, ks));
  };
  auto mf = [&](const bf16x8* fa, const bf16x8* fb, int t) {
    const int i = t >> 3, j = t & 7;
    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  const int nk = K / kBK;
  // Issue order, slot by slot (one MFMA per slot): after the barrier, k-step 0's sixteen reads with the
  // previous stage's last sixteen MFMAs; k-step 0's 64 MFMAs with k-step 1's reads in their first
  // sixteen slots; the next stage's copies spread over the first 60 slots; k-step 1's first 48 MFMAs,
  // then the barrier.  The last stage copies its own K range again into the idle buffer.
  auto stage = [&](int kt, int st, bool first) {
    const char* s = smem + st * kStage;
    const int kn = min(kt + 1, nk - 1);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      rd1(s, 0, fa0, fb0, t);
      if (!first) mf(fa1, fb1, 48 + t);
      if (t == 4 || t == 12) dma(kn, st ^ 1, t == 4 ? 0 : 1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 64; ++t) {
      mf(fa0, fb0, t);
      if (t < 16) rd1(s, 1, fa1, fb1, t);
      if (t % 8 == 4 && t < 48) dma(kn, st ^ 1, 2 + t / 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 0; t < 48; ++t) {
      mf(fa1, fb1, t);
      __builtin_amdgcn_sched_barrier(0);
    }
    dma_wait();
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

#pragma unroll
  for (int i = 0; i < kDma; ++i) dma(0, 0, i);
  dma_wait();
  __syncthreads();
  stage(0, 0, true);
  int kt = 1;
  for (; kt + 1 < nk; kt += 2) {
    stage(kt, 1, false);
    stage(kt + 1, 0, false);
  }
  if (kt < nk) stage(kt, 1, false);
#pragma unroll
  for (int t = 48; t < 64; ++t) mf(fa1, fb1, t);

  // Epilogue through LDS (free since the last barrier): each wave stages its 128 x 128 block as bf16
  // rows of 256 bytes, 16-byte chunks XOR-swizzled by row, and writes it back in runs of eight
  // columns (16 bytes), four rows of 256 bytes per store instruction.
  char* ws = smem + w * 32768;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = i * 16 + q * 4 + e, c = j * 16 + r16;
        *reinterpret_cast<bf16*>(ws + r * 256 + ((((c >> 3) ^ (r & 15))) << 4) + (c & 7) * 2) = (bf16)acc[i][j][e];
      }
  const bool vec = epi.vec(Nc);
#pragma unroll 4
  for (int qq = 0; qq < 32; ++qq) {
    const int x = qq * 64 + l, r = x >> 4, cc = x & 15;
    const bf16x8 val = *reinterpret_cast<const bf16x8*>(ws + r * 256 + ((cc ^ (r & 15)) << 4));
    const int64_t m = m0 + wm * 128 + r;
    const int n = n0 + wn * 128 + cc * 8;
    if (m >= M || n >= Nc) continue;
    if (vec) {
      const ColPtr cp = epi.col(n);
      *reinterpret_cast<bf16x8*>(cp.p + m * cp.stride) = val;
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (n + t < Nc) {
          const ColPtr cp = epi.col(n + t);
          cp.p[m * cp.stride] = val[t];
        }
    }
  }
}

template <class Epi>
hipError_t launch_gemm(const bf16* A, const bf16* B, int64_t M, int Nc, int K, const Epi& epi, const char* name,
                       hipStream_t s) {
  // K <= 2^22 keeps the copies' per-lane byte offsets (up to 255 rows of K) within 32 bits
  if (M < 1 || Nc < 1 || K < kBK || K % kBK != 0 || K > (1 << 22)) return hipErrorInvalidValue;
  const int64_t nrt = (M + kBM - 1) / kBM;
  const int nct = (Nc + kBN - 1) / kBN;
  const int64_t ngroups = ((nrt + kGR - 1) / kGR) * ((nct + kGC - 1) / kGC);
  const int64_t blocks = (ngroups + kXcds - 1) / kXcds * kXcds * (kGR * kGC);
  if (nrt > 0x7fffffffLL || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  TimedLaunch timer(name, s);
  hipLaunchKernelGGL(gemm_nt_bf16_kernel<Epi>, dim3((unsigned)blocks), dim3(kThreads), 0, s, A, B, M, Nc, K,
                     (int)nrt, nct, epi);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_proj_pack(const bf16* x, const bf16* w_qkv, bf16* q_send, bf16* k_send, bf16* v_send,
                                int64_t M, int hidden, int Hq, int Hkv, int D, int P, hipStream_t s) {
  EpiPackQKV epi{q_send, k_send, v_send, M, D, Hq / P, Hkv / P, Hq * D, Hkv * D};
  return launch_gemm(x, w_qkv, M, (Hq + 2 * Hkv) * D, hidden, epi, "qkv_proj_pack", s);
}

hipError_t launch_out_proj(const bf16* o_seq, const bf16* w_o, bf16* y, int64_t M, int hidden, int HqD,
                           hipStream_t s) {
  EpiRowMajor epi{y, hidden};
  return launch_gemm(o_seq, w_o, M, hidden, HqD, epi, "out_proj", s);
}

}  // namespace ul
