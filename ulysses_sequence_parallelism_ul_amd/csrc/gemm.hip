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
// Tiling: 256 x 256 output tile per work-group of 8 waves (two per SIMD), each
// wave 128 rows x 64 columns (4 x 2 blocks of v_mfma_f32_32x32x16_bf16), K in
// stages of 64 double-buffered in LDS (rows of 128 bytes, 16-byte chunks XOR
// swizzled by row so 32 rows read at one chunk hit distinct banks), the next
// stage copied global -> LDS by DMA while the current one is multiplied.
// Work-groups are mapped so each XCD runs groups of 8 row tiles x 4 column
// tiles together, sharing every K stage's slices of A and B through its L2.
#include "ul_internal.h"

namespace ul {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kThreads = 512;
constexpr int kRowBytes = kBK * 2;                  // 128 bytes per tile row
constexpr int kTileBytes = kBM * kRowBytes;         // 32 KiB per operand tile
constexpr int kStage = 2 * kTileBytes;              // A tile + B tile
constexpr int kChunksPerTile = kTileBytes / 16;     // 2048
constexpr int kLoadsPerThread = kChunksPerTile / kThreads;  // 4 per operand (16 bytes each)
constexpr int kXcds = 8;
constexpr int kGR = 8, kGC = 4;  // tile group per XCD: 8 row tiles x 4 column tiles

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

// An epilogue maps output column n to the address of its element in row 0
// and the stride between rows: element (m, n) lives at col(n).p + m * col(n).stride.
struct ColPtr {
  bf16* p;
  int64_t stride;
};

struct EpiRowMajor {
  bf16* y;
  int64_t ld;
  __device__ ColPtr col(int n) const { return ColPtr{y + n, ld}; }
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
};

template <class Epi>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_nt_bf16_kernel(const bf16* __restrict__ A, const bf16* __restrict__ B, int64_t M, int Nc, int K,
                    int n_row_tiles, int n_col_tiles, Epi epi) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, g = l >> 5, lc = l & 31;
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
  const int wm = w >> 2, wn = w & 3;  // wave grid 2 x 4: 128 rows x 64 columns each

  // Tiles go global -> LDS by DMA (global_load_lds_dwordx4): lane l of wave w's
  // i-th load writes the 16 bytes at LDS block (w * 4 + i) * 1024 + l * 16 of
  // the tile, so each lane fetches the global chunk that the XOR-swizzled
  // layout puts there.  Issued as inline assembly so that the compiler does
  // not order the MFMA phase's LDS reads (of the other stage) behind them; the
  // wave waits for its own copies before each barrier.
  const bf16* pa[kLoadsPerThread];
  const bf16* pb[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int row = (w * kLoadsPerThread + i) * 8 + (l >> 3);
    const int chunk = (l & 7) ^ (row & 7);
    const int64_t am = min<int64_t>(m0 + row, M - 1);   // rows past the end read the last row
    const int bn = min(n0 + row, Nc - 1);
    pa[i] = A + am * K + chunk * 8;
    pb[i] = B + (int64_t)bn * K + chunk * 8;
  }
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  auto dma = [&](int kt, int st) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      const uint32_t ba = __builtin_amdgcn_readfirstlane(lds0 + st * kStage + (w * kLoadsPerThread + i) * 1024);
      const uint32_t bb = ba + kTileBytes;
      // one wait state between writing M0 and the LDS DMA that reads it
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(ba), "v"(pa[i] + k0)
                   : "memory", "m0");
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(bb), "v"(pb[i] + k0)
                   : "memory", "m0");
    }
  };
  auto dma_wait = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const int nk = K / kBK;
  dma(0, 0);
  dma_wait();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < nk) dma(kt + 1, st ^ 1);  // the other stage is free since the last barrier
    const char* sa = smem + st * kStage;
    const char* sb = sa + kTileBytes;
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 a[4], b[2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(sa + swz(wm * 128 + i * 32 + lc, ks * 2 + g));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(sb + swz(wn * 64 + j * 32 + lc, ks * 2 + g));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    // schedule: nine operand reads ahead, then groups of four MFMAs and three
    // reads (each 16-deep step needs six reads for eight MFMAs)
    __builtin_amdgcn_sched_group_barrier(0x100, 9, 0);
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
    dma_wait();
    __syncthreads();
  }

  // C block (i, j): lane holds rows (e>>2)*8 + g*4 + (e&3) of column lc
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + lc;
      if (n >= Nc) continue;
      const ColPtr cp = epi.col(n);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + g * 4 + (e & 3);
        if (m < M) cp.p[m * cp.stride] = (bf16)acc[i][j][e];
      }
    }
}

template <class Epi>
hipError_t launch_gemm(const bf16* A, const bf16* B, int64_t M, int Nc, int K, const Epi& epi, const char* name,
                       hipStream_t s) {
  if (M < 1 || Nc < 1 || K < kBK || K % kBK != 0) return hipErrorInvalidValue;
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
