// Step 2 backward, fp32 inputs: VALU kernels, one thread per output row.
// Used for small fp32 checks; the bf16 MFMA kernels carry the long sequences.
//
// Backward of L = sum(dO * O) with P recomputed from the saved log-sum-exp:
// delta_i = sum_d dO_i O_i, dP_ij = dO_i . V_j, dS_ij = P_ij (dP_ij - delta_i),
// dQ_i = scale sum_j dS_ij K_j, dK_j = scale sum_i dS_ij Q_i, dV_j = sum_i P_ij dO_i
// (dK and dV summed over the query heads of the group).  The pages describe no
// backward; this is the chain rule of the forward they describe (page "Hugging
// Face并行加速", nmedialink.com, section "Ulysses的工作原理", step 4).
#include "ul_internal.h"

#include <math.h>

namespace ul {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ void __launch_bounds__(64) delta_f32_kernel(const float* __restrict__ o, const float* __restrict__ dout,
                                                     float* __restrict__ delta, int N, int Hq) {
  const int64_t c = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (c >= (int64_t)N * Hq) return;
  const int row = (int)(c / Hq), h = (int)(c % Hq);
  float s = 0.0f;
  for (int d = 0; d < D; ++d) s = __builtin_fmaf(o[c * D + d], dout[c * D + d], s);
  delta[(int64_t)h * N + row] = s;
}

template <int D>
__global__ void __launch_bounds__(64) dq_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                  const float* __restrict__ v, const float* __restrict__ dout,
                                                  const float* __restrict__ lse, const float* __restrict__ delta,
                                                  const int32_t* __restrict__ doc_start, float* __restrict__ dq,
                                                  int N, int Hq, int Hkv, float scale) {
  const int64_t c = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (c >= (int64_t)N * Hq) return;
  const int row = (int)(c / Hq), h = (int)(c % Hq);
  const int gkv = h / (Hq / Hkv);
  float qv[D], dov[D], acc[D];
  for (int d = 0; d < D; ++d) { qv[d] = q[c * D + d]; dov[d] = dout[c * D + d]; acc[d] = 0.0f; }
  const float l2 = lse[(int64_t)h * N + row] * kLog2e;
  const float dl = delta[(int64_t)h * N + row];
  const float sl2 = scale * kLog2e;
  for (int j = doc_start[row]; j <= row; ++j) {
    const float* kr = k + ((int64_t)j * Hkv + gkv) * D;
    const float* vr = v + ((int64_t)j * Hkv + gkv) * D;
    float s = 0.0f, dp = 0.0f;
    for (int d = 0; d < D; ++d) {
      s = __builtin_fmaf(qv[d], kr[d], s);
      dp = __builtin_fmaf(dov[d], vr[d], dp);
    }
    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, sl2, -l2));
    const float ds = p * (dp - dl);
    for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, kr[d], acc[d]);
  }
  for (int d = 0; d < D; ++d) dq[c * D + d] = acc[d] * scale;
}

template <int D>
__global__ void __launch_bounds__(64) dkdv_f32_kernel(const float* __restrict__ q, const float* __restrict__ k,
                                                    const float* __restrict__ v, const float* __restrict__ dout,
                                                    const float* __restrict__ lse, const float* __restrict__ delta,
                                                    const int32_t* __restrict__ doc_end, float* __restrict__ dk,
                                                    float* __restrict__ dv, int N, int Hq, int Hkv, float scale) {
  const int64_t c = (int64_t)blockIdx.x * 64 + threadIdx.x;  // (key row, kv head)
  if (c >= (int64_t)N * Hkv) return;
  const int j = (int)(c / Hkv), gkv = (int)(c % Hkv);
  const int G = Hq / Hkv;
  float kv_[D], vv[D], ak[D], av[D];
  for (int d = 0; d < D; ++d) { kv_[d] = k[c * D + d]; vv[d] = v[c * D + d]; ak[d] = 0.0f; av[d] = 0.0f; }
  const float sl2 = scale * kLog2e;
  const int iend = doc_end[j];
  for (int i = j; i <= iend; ++i) {
    for (int hh = 0; hh < G; ++hh) {
      const int h = gkv * G + hh;
      const float* qr = q + ((int64_t)i * Hq + h) * D;
      const float* dr = dout + ((int64_t)i * Hq + h) * D;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(qr[d], kv_[d], s);
        dp = __builtin_fmaf(dr[d], vv[d], dp);
      }
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, sl2, -lse[(int64_t)h * N + i] * kLog2e));
      const float ds = p * (dp - delta[(int64_t)h * N + i]);
      for (int d = 0; d < D; ++d) {
        av[d] = __builtin_fmaf(p, dr[d], av[d]);
        ak[d] = __builtin_fmaf(ds, qr[d], ak[d]);
      }
    }
  }
  for (int d = 0; d < D; ++d) {
    dk[c * D + d] = ak[d] * scale;
    dv[c * D + d] = av[d];
  }
}

}  // namespace

hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* dout,
                               const float* lse, const int32_t* doc_start, const int32_t* doc_end, float* dq,
                               float* dk, float* dv, float* delta, int N, int Hq, int Hkv, int D, float scale,
                               hipStream_t s) {
  const dim3 gq((unsigned)(((int64_t)N * Hq + 63) / 64)), gk((unsigned)(((int64_t)N * Hkv + 63) / 64)), b(64);
  TimedLaunch timer("attn_bwd_f32", s);
  if (D == 128) {
    hipLaunchKernelGGL(delta_f32_kernel<128>, gq, b, 0, s, o, dout, delta, N, Hq);
    hipLaunchKernelGGL(dq_f32_kernel<128>, gq, b, 0, s, q, k, v, dout, lse, delta, doc_start, dq, N, Hq, Hkv, scale);
    hipLaunchKernelGGL(dkdv_f32_kernel<128>, gk, b, 0, s, q, k, v, dout, lse, delta, doc_end, dk, dv, N, Hq, Hkv,
                       scale);
  } else {
    hipLaunchKernelGGL(delta_f32_kernel<64>, gq, b, 0, s, o, dout, delta, N, Hq);
    hipLaunchKernelGGL(dq_f32_kernel<64>, gq, b, 0, s, q, k, v, dout, lse, delta, doc_start, dq, N, Hq, Hkv, scale);
    hipLaunchKernelGGL(dkdv_f32_kernel<64>, gk, b, 0, s, q, k, v, dout, lse, delta, doc_end, dk, dv, N, Hq, Hkv,
                       scale);
  }
  return hipGetLastError();
}

}  // namespace ul
