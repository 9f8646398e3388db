// Step 2 forward: rank-local causal attention with grouped-query heads and
// packed documents (page "Hugging Face并行加速：10倍提升超长序列训练效率",
// nmedialink.com, section "Ulysses的工作原理", step 4; page "Ulysses verteilt
// Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch, section
// "Integration in den Hugging-Face-Stack" for position-id masking; the
// tiling that keeps memory linear in N follows the page "Hugging Face并行加速",
// section "超长序列训练的挑战").
//
// bf16 kernel (gfx950, v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//  * "Query columns": the G query heads of KV head hk are interleaved, column
//    c = token * G + head_in_group, so one K/V tile serves all G heads and
//    the mask of column c is that of token c / G.
//  * A work-group of NW waves owns 32*NW consecutive columns; each wave owns
//    32 and keeps its Q operand in registers for the whole key loop.
//  * The scores are formed transposed, S^T = K Q^T (keys x columns), so every
//    lane holds one column: the row max and row sum are in-lane over the 32
//    keys the lane sees plus one exchange with lane l^32.  The K tile is
//    written to LDS with rows permuted (bits 2 and 3 of the row swapped) so
//    that the 8 keys of each MFMA accumulator group are consecutive, which
//    makes the probabilities directly usable, in registers, as the B operand
//    of O^T += V^T P^T.
//  * V^T comes from a blocked transposed copy (one pre-pass per call) so the
//    V tile is a contiguous 16 KiB block.
//  * Key tiles of 64 are double-buffered in LDS; one barrier per tile.
//  * Tiles entirely below the diagonal and inside every row's document skip
//    the mask; the tile loop starts at the document start of the first row,
//    so tiles of earlier documents are never visited.
//  * Online softmax in base 2 (log2(e) folded into the scale); the running
//    max is only moved when it grows by more than 8 (a factor 256), which
//    keeps fp32 sums exact enough and makes the O rescale rare.
//  * LSE is stored as a natural log.
//
// f32 kernel: one thread per query column with VALU arithmetic; used for
// small fp32 checks.
#include "ul_internal.h"

#include <math.h>

#include <type_traits>

namespace ul {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D, int NW>
struct FwdCfg {
  static constexpr int kThreads = NW * 64;
  static constexpr int BN = 64;            // keys per tile
  static constexpr int BMC = NW * 32;      // query columns per work-group
  static constexpr int KSTR = D * 2 + 16;  // LDS bytes per K row (16 B pad)
  static constexpr int VSTR = BN * 2 + 16; // LDS bytes per V^T row
  static constexpr int KBYTES = BN * KSTR;
  static constexpr int VBYTES = D * VSTR;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KCH = BN * D / 8;   // 16-byte chunks per K tile
  static constexpr int VCH = D * BN / 8;   // 16-byte chunks per V^T tile
  static constexpr int KPT = KCH / kThreads;
  static constexpr int VPT = VCH / kThreads;
  static_assert(KCH % kThreads == 0 && VCH % kThreads == 0, "tile chunks must split evenly");
};

// LDS row of key r within a 64-key tile: swap bits 2 and 3 (an involution).
__device__ __forceinline__ int perm_row(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ bf16x8 pack8(const f32x16& s, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (bf16)s[base + e];
  return r;
}

// Combine a value across the lane pair (l, l ^ 32) with v_permlane32_swap
// (no LDS round trip): after the swap one result holds lane (l & 31)'s value
// and the other lane (l | 32)'s, so the symmetric combination is the same on
// both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) attn_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ vt,
    const int32_t* __restrict__ doc_start, const int32_t* __restrict__ order, bf16* __restrict__ o,
    float* __restrict__ lse, int N, int Hkv, int lgG, float sl2, int nb) {
  using C = FwdCfg<D, NW>;
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

  // this lane's query column
  const int64_t c = c0 + w * 32 + lc;
  const bool cvalid = c < NG;
  const int row = cvalid ? (int)(c >> lgG) : -1;
  const int hg = (int)(c & (G - 1));
  const int ds_c = cvalid ? doc_start[row] : 0;
  const int64_t qoff = cvalid ? ((((int64_t)row * Hkv + hk) << lgG) + hg) * D : 0;

  bf16x8 qreg[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (cvalid) {
      qreg[ks] = *reinterpret_cast<const bf16x8*>(q + qoff + ks * 16 + g * 8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[ks][e] = (bf16)0.0f;
    }
  }

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  u32x4 kpre[C::KPT], vpre[C::VPT];
  // A thread loads 16-byte chunk part0 of K rows r0 + i * RSTEP; tiles are
  // loaded in increasing order, so the K offset advances by a constant and
  // only a tile that runs past the last key clamps its rows.  V^T tiles are
  // contiguous blocks.
  constexpr int RSTEP = C::kThreads / (D / 8);
  const int r0 = tid / (D / 8), part0 = tid % (D / 8);
  const int64_t row_step = (int64_t)RSTEP * Hkv * D, tile_step = (int64_t)C::BN * Hkv * D;
  int64_t koff = ((int64_t)(t_lo * C::BN + r0) * Hkv + hk) * D + part0 * 8;
  const bf16* vsrc = vt + ((int64_t)hk * nb + t_lo) * (int64_t)(D * C::BN) + tid * 8;
  auto gload = [&](int t) {
    const int t0 = t * C::BN;
    if (t0 + C::BN <= N) {
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) kpre[i] = *reinterpret_cast<const u32x4*>(k + koff + i * row_step);
    } else {
#pragma unroll
      for (int i = 0; i < C::KPT; ++i) {
        // keys past the end read the last key instead (masked out below)
        const int kv = min(t0 + r0 + i * RSTEP, N - 1);
        kpre[i] = *reinterpret_cast<const u32x4*>(k + ((int64_t)kv * Hkv + hk) * D + part0 * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) vpre[i] = *reinterpret_cast<const u32x4*>(vsrc + i * C::kThreads * 8);
    koff += tile_step;
    vsrc += D * C::BN;
  };
  auto lstore = [&](int st) {
    char* kb = smem + st * C::STAGE;
    char* vb = kb + C::KBYTES;
#pragma unroll
    for (int i = 0; i < C::KPT; ++i) {
      const int ch = tid + i * C::kThreads;
      const int r = ch / (D / 8), part = ch % (D / 8);
      *reinterpret_cast<u32x4*>(kb + perm_row(r) * C::KSTR + part * 16) = kpre[i];
    }
#pragma unroll
    for (int i = 0; i < C::VPT; ++i) {
      const int ch = tid + i * C::kThreads;
      const int d = ch / (C::BN / 8), part = ch % (C::BN / 8);
      *reinterpret_cast<u32x4*>(vb + d * C::VSTR + part * 16) = vpre[i];
    }
  };

  gload(t_lo);
  lstore(0);
  __syncthreads();
  // two tiles per iteration so that each tile's LDS stage is a compile-time
  // constant (operand addresses then differ by immediate offsets only)
  auto tile = [&](auto stage, int t) {
    constexpr int st = decltype(stage)::value;
    if (t < t_hi) gload(t + 1);
    const char* kb_l = smem + st * C::STAGE;
    const char* vb_l = kb_l + C::KBYTES;

    // S^T = K Q^T for 64 keys x 32 columns
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_l + (kb * 32 + lc) * C::KSTR + ks * 32 + g * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], s[kb], 0, 0, 0);
      }
    }
    // schedule: 8 K reads in flight ahead of the 16 MFMAs (the compiler's own
    // order waits on each read right before its MFMA)
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // 8 LDS reads
#pragma unroll
    for (int j = 0; j < 2 * (D / 16) - 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // the first two 16-key steps of V^T travel during the softmax
    bf16x8 va[2][D / 32];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        va[tt][db] = *reinterpret_cast<const bf16x8*>(vb_l + (db * 32 + lc) * C::VSTR + tt * 32 + g * 16);

    const int t0 = t * C::BN;
    if (t0 + C::BN - 1 > r_first || t0 < ds_last) {
      // register i of block kb holds key t0 + kb*32 + (i>>3)*16 + g*8 + (i&7);
      // visible iff it lies in [ds_c, row] (empty for a column past the end)
      const int kbase = t0 + g * 8;
      int lo = ds_c - kbase;
      const int hi = row - kbase;
      unsigned span = (unsigned)(hi - lo);
      if (hi < lo) {
        lo = 1 << 30;
        span = 0u;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((unsigned)(kb * 32 + (i >> 3) * 16 + (i & 7) - lo) > span) s[kb][i] = -INFINITY;
    }

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = pair_max(mx);
    const float mnew = mx * sl2;
    const bool up = mnew > m_run + kRescaleSlack;
    if (__any(up)) {
      const float mset = up ? mnew : m_run;
      const float alpha = up ? __builtin_amdgcn_exp2f(m_run - mset) : 1.0f;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      m_run = mset;
    }
    const float ms = m_run == -INFINITY ? 0.0f : m_run;
    float psum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], sl2, -ms));
        s[kb][i] = p;
        psum += p;
      }
    l_run += psum;

    // O^T += V^T P^T over the 64 keys (4 steps of 16)
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const bf16x8 pb = pack8(s[tt >> 1], (tt & 1) * 8);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 a =
            tt < 2 ? va[tt][db] : *reinterpret_cast<const bf16x8*>(vb_l + (db * 32 + lc) * C::VSTR + tt * 32 + g * 16);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, acc[db], 0, 0, 0);
      }
    }

    if (t < t_hi) lstore(st ^ 1);
    __syncthreads();
  };
  for (int t = t_lo; t <= t_hi; t += 2) {
    tile(std::integral_constant<int, 0>(), t);
    if (t + 1 > t_hi) break;
    tile(std::integral_constant<int, 1>(), t + 1);
  }

  const float l_tot = pair_sum(l_run);
  if (cvalid) {
    const float inv = 1.0f / l_tot;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(acc[db][j * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(o + qoff + db * 32 + j * 8 + g * 4) = ov;
      }
    if (g == 0) {
      const int h = (hk << lgG) + hg;
      lse[(int64_t)h * N + row] = (m_run + log2f(l_tot)) * kLn2;
    }
  }
}

// ---------------------------------------------------------------- fp32 --
template <int D>
__global__ void __launch_bounds__(64) attn_fwd_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v,
                                                        const int32_t* __restrict__ doc_start,
                                                        float* __restrict__ o, float* __restrict__ lse, int N,
                                                        int Hq, int Hkv, float sl2) {
  const int64_t c = (int64_t)blockIdx.x * 64 + threadIdx.x;  // token-major (row, head)
  if (c >= (int64_t)N * Hq) return;
  const int row = (int)(c / Hq), h = (int)(c % Hq);
  const int gkv = h / (Hq / Hkv);
  float qv[D], acc[D];
  for (int d = 0; d < D; ++d) { qv[d] = q[c * D + d]; acc[d] = 0.0f; }
  float m = -INFINITY, lsum = 0.0f;
  for (int j = doc_start[row]; j <= row; ++j) {
    const float* kr = k + ((int64_t)j * Hkv + gkv) * D;
    const float* vr = v + ((int64_t)j * Hkv + gkv) * D;
    float s = 0.0f;
    for (int d = 0; d < D; ++d) s = __builtin_fmaf(qv[d], kr[d], s);
    s *= sl2;
    if (s > m) {
      const float a = __builtin_amdgcn_exp2f(m - s);
      lsum *= a;
      for (int d = 0; d < D; ++d) acc[d] *= a;
      m = s;
    }
    const float p = __builtin_amdgcn_exp2f(s - m);
    lsum += p;
    for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(p, vr[d], acc[d]);
  }
  const float inv = 1.0f / lsum;
  for (int d = 0; d < D; ++d) o[c * D + d] = acc[d] * inv;
  lse[(int64_t)h * N + row] = (m + log2f(lsum)) * kLn2;
}

int ilog2_pow2(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const bf16* q, const bf16* k, const bf16* v, const int32_t* doc_start, bf16* o,
                                float* lse, bf16* vt_ws, int32_t* order_ws, int N, int Hq, int Hkv, int D, float scale,
                                hipStream_t s) {
  hipError_t e = launch_transpose_blocked(v, vt_ws, N, Hkv, Hkv, 0, D, s);
  if (e != hipSuccess) return e;
  const int lgG = ilog2_pow2(Hq / Hkv);
  const int nb = (N + kTB - 1) / kTB;
  const float sl2 = scale * kLog2e;
  constexpr int NW = 8;
  static_assert(FwdCfg<128, NW>::BMC == kColBlock && FwdCfg<128, NW>::BN == kKeyTile, "unit sizes of the order");
  static_assert(FwdCfg<64, NW>::BMC == kColBlock && FwdCfg<64, NW>::BN == kKeyTile, "unit sizes of the order");
  const int ncb = (int)col_blocks(N, Hq / Hkv);
  OrderJobs jobs{};
  jobs.j[0] = OrderJob{order_ws, doc_start, 0, ncb, kColBlock, kKeyTile};
  e = launch_order(jobs, 1, N, lgG, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((int64_t)ncb * Hkv)), block(NW * 64);
  TimedLaunch timer("attn_fwd_bf16", s);
  if (D == 128)
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<128, NW>), grid, block, 0, s, q, k, vt_ws, doc_start, order_ws, o, lse,
                       N, Hkv, lgG, sl2, nb);
  else
    hipLaunchKernelGGL((attn_fwd_bf16_kernel<64, NW>), grid, block, 0, s, q, k, vt_ws, doc_start, order_ws, o, lse,
                       N, Hkv, lgG, sl2, nb);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, const int32_t* doc_start, float* o,
                               float* lse, int N, int Hq, int Hkv, int D, float scale, hipStream_t s) {
  const int64_t ncols = (int64_t)N * Hq;
  const dim3 grid((unsigned)((ncols + 63) / 64)), block(64);
  const float sl2 = scale * kLog2e;
  TimedLaunch timer("attn_fwd_f32", s);
  if (D == 128)
    hipLaunchKernelGGL(attn_fwd_f32_kernel<128>, grid, block, 0, s, q, k, v, doc_start, o, lse, N, Hq, Hkv, sl2);
  else
    hipLaunchKernelGGL(attn_fwd_f32_kernel<64>, grid, block, 0, s, q, k, v, doc_start, o, lse, N, Hq, Hkv, sl2);
  return hipGetLastError();
}

}  // namespace ul
