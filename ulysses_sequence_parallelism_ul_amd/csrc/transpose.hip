// Blocked transposed copies of attention operands, kept in the workspace.
//
// The forward's P.V contraction runs over the token axis and needs V with
// tokens as the fast axis.  One pass per call rewrites a [cols][D] bf16
// matrix view into tiles [cols / kTB][D][kTB] (zero-padded past the last
// column), so a kTB x D tile is one contiguous 16 KiB block that the
// attention kernels stream into LDS with plain 16-byte loads.  This is
// O(N * D) traffic against the O(N^2 * D) attention it feeds.
//
// Column c of KV-head group `hk` addresses token c >> lgG, head
// (hk << lgG) + (c & (G-1)) of a [N][H][D] tensor (G = 1 for K and V, the
// query group size for Q and dO), so the query heads of a group interleave as
// "query columns".
#include "ul_internal.h"

namespace ul {
namespace {

template <int D>
__global__ void __launch_bounds__(256) transpose_blocked_kernel(const bf16* __restrict__ src, bf16* __restrict__ dst,
                                                              int64_t ncols, int H, int lgG, int nblk) {
  constexpr int PAD = 8;                  // elements of padding per LDS row
  __shared__ bf16 tile[kTB][D + PAD];     // [col][d]
  const int b = blockIdx.x, hk = blockIdx.y;
  const int G = 1 << lgG;
  constexpr int CH = D / 8;               // 16-byte chunks per source row
  for (int ch = threadIdx.x; ch < kTB * CH; ch += 256) {
    const int cl = ch / CH, part = ch % CH;
    const int64_t c = (int64_t)b * kTB + cl;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (c < ncols) {
      const int64_t off = (((c >> lgG) * H + ((int64_t)hk << lgG) + (c & (G - 1))) * D) + part * 8;
      val = *reinterpret_cast<const u32x4*>(src + off);
    }
    *reinterpret_cast<u32x4*>(&tile[cl][part * 8]) = val;
  }
  __syncthreads();
  bf16* out = dst + ((int64_t)hk * nblk + b) * (int64_t)(D * kTB);
  constexpr int OCH = kTB / 8;            // 16-byte chunks per output row
  for (int ch = threadIdx.x; ch < D * OCH; ch += 256) {
    const int d = ch / OCH, part = ch % OCH;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[part * 8 + e][d];
    *reinterpret_cast<bf16x8*>(out + (int64_t)d * kTB + part * 8) = v;
  }
}

}  // namespace

hipError_t launch_transpose_blocked(const bf16* src, bf16* dst, int64_t ncols, int H, int Hkv, int lgG, int D,
                                    hipStream_t s) {
  const int nblk = (int)((ncols + kTB - 1) / kTB);
  dim3 grid(nblk, Hkv);
  TimedLaunch timer("transpose_blocked", s);
  if (D == 128)
    hipLaunchKernelGGL(transpose_blocked_kernel<128>, grid, dim3(256), 0, s, src, dst, ncols, H, lgG, nblk);
  else if (D == 64)
    hipLaunchKernelGGL(transpose_blocked_kernel<64>, grid, dim3(256), 0, s, src, dst, ncols, H, lgG, nblk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace ul
