// Token-weighted loss of a sequence-sharded step.
//
// The data loader shards the sequence and every rank computes the loss of its
// own shard (page "Ulysses 序列並行：百萬 Token 上下文訓練", setupai.cc, section
// "增強重點摘要"); the ranks' losses are then weighted by their numbers of
// valid tokens (page "Ulysses verteilt Millionen-Token-Kontexte auf mehrere
// GPUs", dailytechsnack.ch, section "Integration in den Hugging-Face-Stack").
// Next-token cross entropy is the loss; targets are shifted on the whole
// packed sequence before it is sharded.
//
// Kernels:
//  * shift_labels_kernel: target of token t = label of token t + 1 when that
//    token exists and is in the same document (position id != 0), else the
//    ignore index.  Elementwise.
//  * count_valid_kernel / sum_loss_kernel / combine_kernel: one work-group
//    each, fixed summation order (bitwise deterministic, no atomics).
//  * ce_row_kernel: one work-group of 1024 threads per token row of logits.
//    With NCH > 0 the whole row stays in registers (NCH 16-byte chunks per
//    thread): one HBM read of the row gives the log-sum-exp and, from the same
//    registers, the gradient row, so a forward+backward costs one read and one
//    write of the logits.  NCH == 0 streams the row twice (rows too long for
//    the register file).  Softmax arithmetic is fp32 in base 2.
#include "ul_internal.h"

#include <math.h>

namespace ul {
namespace {

constexpr int kCeThreads = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct Chunk;
template <>
struct Chunk<bf16> {
  typedef bf16x8 V;
  static constexpr int E = 8;
};
template <>
struct Chunk<float> {
  typedef f32x4 V;
  static constexpr int E = 4;
};

__global__ void __launch_bounds__(256) shift_labels_kernel(const int32_t* __restrict__ labels,
                                                          const int32_t* __restrict__ pos,
                                                          int32_t* __restrict__ out, int64_t N, int ign) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= N) return;
  int32_t y = ign;
  if (t + 1 < N && (pos == nullptr || pos[t + 1] != 0)) y = labels[t + 1];
  out[t] = y;
}

// --- fixed-order reductions over one work-group of kCeThreads threads ---
template <typename A>
__device__ __forceinline__ A block_sum(A v, A* red) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  if (l == 0) red[w] = v;
  __syncthreads();
  if (w == 0) {
    v = l < kCeThreads / 64 ? red[l] : (A)0;
#pragma unroll
    for (int m = 8; m > 0; m >>= 1) v += __shfl_xor(v, m, 64);
  }
  return v;  // valid in thread 0
}

__global__ void __launch_bounds__(kCeThreads) count_valid_kernel(const int32_t* __restrict__ labels, int64_t T,
                                                                int ign, int64_t* __restrict__ count) {
  __shared__ long long red[kCeThreads / 64];
  long long c = 0;
  for (int64_t t = threadIdx.x; t < T; t += kCeThreads) c += labels[t] != ign;
  c = block_sum<long long>(c, red);
  if (threadIdx.x == 0) count[0] = c;
}

__global__ void __launch_bounds__(kCeThreads) sum_loss_kernel(const float* __restrict__ loss_tok, int64_t T,
                                                             double* __restrict__ out) {
  __shared__ double red[kCeThreads / 64];
  double s = 0.0;
  for (int64_t t = threadIdx.x; t < T; t += kCeThreads) s += (double)loss_tok[t];
  s = block_sum<double>(s, red);
  if (threadIdx.x == 0) out[0] = s;
}

__global__ void __launch_bounds__(kCeThreads) combine_kernel(const double* __restrict__ loss_sums,
                                                            const int64_t* __restrict__ counts, int P,
                                                            int64_t* __restrict__ total_out,
                                                            double* __restrict__ loss_out) {
  __shared__ long long redc[kCeThreads / 64];
  __shared__ double reds[kCeThreads / 64];
  long long c = 0;
  double s = 0.0;
  for (int r = threadIdx.x; r < P; r += kCeThreads) {
    c += counts[r];
    if (loss_sums != nullptr) s += loss_sums[r];
  }
  c = block_sum<long long>(c, redc);
  s = block_sum<double>(s, reds);
  if (threadIdx.x == 0) {
    if (total_out != nullptr) total_out[0] = c;
    if (loss_out != nullptr) loss_out[0] = c > 0 ? s / (double)c : 0.0;
  }
}

// (max, sum) pair of a base-2 log-sum-exp: value = m + log2(s)
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    m = M;
    s = 0.0f;
    return;
  }
  s = s * __builtin_amdgcn_exp2f(m - M) + s2 * __builtin_amdgcn_exp2f(m2 - M);
  m = M;
}

template <typename T, int NCH>
__global__ void __launch_bounds__(kCeThreads) ce_row_kernel(const T* logits, const int32_t* __restrict__ labels,
                                                           float* __restrict__ loss_tok, T* dlogits,
                                                           const int64_t* __restrict__ total_count, float dloss,
                                                           int V, int ign) {
  typedef typename Chunk<T>::V CV;
  constexpr int E = Chunk<T>::E;
  __shared__ float red_m[kCeThreads / 64], red_s[kCeThreads / 64];
  __shared__ float row_lse2;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nch = V / E;
  const CV* x = reinterpret_cast<const CV*>(logits + row * (int64_t)V);
  const int y = labels[row];

  // base-2 scaled values a = x log2(e); per-thread max, then sum of 2^(a - max)
  float m = -INFINITY, s = 0.0f;
  CV r[NCH > 0 ? NCH : 1];
  if constexpr (NCH > 0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * kCeThreads;
      if (c < nch) r[i] = __builtin_nontemporal_load(x + c);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * kCeThreads;
      if (c < nch) {
#pragma unroll
        for (int e = 0; e < E; ++e) m = fmaxf(m, (float)r[i][e]);
      }
    }
    m *= kLog2e;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * kCeThreads;
      if (c < nch) {
#pragma unroll
        for (int e = 0; e < E; ++e) s += __builtin_amdgcn_exp2f(__builtin_fmaf((float)r[i][e], kLog2e, -m));
      }
    }
  } else {
    for (int c = tid; c < nch; c += kCeThreads) {
      const CV v = x[c];
      float cm = -INFINITY;
#pragma unroll
      for (int e = 0; e < E; ++e) cm = fmaxf(cm, (float)v[e]);
      cm *= kLog2e;
      float cs = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) cs += __builtin_amdgcn_exp2f(__builtin_fmaf((float)v[e], kLog2e, -cm));
      lse_merge(m, s, cm, cs);
    }
  }

  // work-group merge of the (max, sum) pairs in a fixed order
#pragma unroll
  for (int k = 32; k > 0; k >>= 1) {
    const float m2 = __shfl_xor(m, k, 64), s2 = __shfl_xor(s, k, 64);
    lse_merge(m, s, m2, s2);
  }
  const int w = tid >> 6, l = tid & 63;
  if (l == 0) {
    red_m[w] = m;
    red_s[w] = s;
  }
  __syncthreads();
  if (w == 0) {
    m = l < kCeThreads / 64 ? red_m[l] : -INFINITY;
    s = l < kCeThreads / 64 ? red_s[l] : 0.0f;
#pragma unroll
    for (int k = 8; k > 0; k >>= 1) {
      const float m2 = __shfl_xor(m, k, 64), s2 = __shfl_xor(s, k, 64);
      lse_merge(m, s, m2, s2);
    }
    if (l == 0) {
      const float lse2 = m + __log2f(s);
      row_lse2 = lse2;
      float loss = 0.0f;
      if (y != ign) loss = (unsigned)y < (unsigned)V ? lse2 * kLn2 - (float)logits[row * (int64_t)V + y] : NAN;
      loss_tok[row] = loss;
    }
  }
  if (dlogits == nullptr) return;
  __syncthreads();
  const float lse2 = row_lse2;
  const int64_t tot = total_count[0];
  const float gs = (y != ign && (unsigned)y < (unsigned)V && tot > 0) ? dloss / (float)tot : 0.0f;
  CV* g = reinterpret_cast<CV*>(dlogits + row * (int64_t)V);
  auto grad = [&](const CV& v, int c) {
    CV o;
    if (gs == 0.0f) {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] = (T)0.0f;
    } else {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf((float)v[e], kLog2e, -lse2));
        o[e] = (T)(gs * (c * E + e == y ? p - 1.0f : p));
      }
    }
    return o;
  };
  if constexpr (NCH > 0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = tid + i * kCeThreads;
      if (c < nch) __builtin_nontemporal_store(grad(r[i], c), g + c);
    }
  } else {
    for (int c = tid; c < nch; c += kCeThreads) g[c] = grad(x[c], c);
  }
}

template <typename T, int NCH>
hipError_t launch_ce_t(const T* logits, const int32_t* labels, float* loss_tok, T* dlogits,
                       const int64_t* total_count, float dloss, int64_t Tn, int V, int ign, hipStream_t s) {
  hipLaunchKernelGGL((ce_row_kernel<T, NCH>), dim3((unsigned)Tn), dim3(kCeThreads), 0, s, logits, labels, loss_tok,
                     dlogits, total_count, dloss, V, ign);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_ce_pick(const T* logits, const int32_t* labels, float* loss_tok, T* dlogits,
                          const int64_t* total_count, float dloss, int64_t Tn, int V, int ign, hipStream_t s) {
  const int per_thread = (V / Chunk<T>::E + kCeThreads - 1) / kCeThreads;
  if (per_thread <= 2) return launch_ce_t<T, 2>(logits, labels, loss_tok, dlogits, total_count, dloss, Tn, V, ign, s);
  if (per_thread <= 4) return launch_ce_t<T, 4>(logits, labels, loss_tok, dlogits, total_count, dloss, Tn, V, ign, s);
  if (per_thread <= 8) return launch_ce_t<T, 8>(logits, labels, loss_tok, dlogits, total_count, dloss, Tn, V, ign, s);
  if (per_thread <= 16) return launch_ce_t<T, 16>(logits, labels, loss_tok, dlogits, total_count, dloss, Tn, V, ign, s);
  if (per_thread <= 20) return launch_ce_t<T, 20>(logits, labels, loss_tok, dlogits, total_count, dloss, Tn, V, ign, s);
  return launch_ce_t<T, 0>(logits, labels, loss_tok, dlogits, total_count, dloss, Tn, V, ign, s);
}

}  // namespace

int ce_max_resident_vocab(int elem_bytes) { return 20 * kCeThreads * (16 / elem_bytes); }

hipError_t launch_shift_labels(const int32_t* labels, const int32_t* pos, int32_t* out, int64_t N, int ign,
                               hipStream_t s) {
  const int64_t blocks = (N + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  TimedLaunch timer("shift_labels", s);
  hipLaunchKernelGGL(shift_labels_kernel, dim3((unsigned)blocks), dim3(256), 0, s, labels, pos, out, N, ign);
  return hipGetLastError();
}

hipError_t launch_count_valid(const int32_t* labels, int64_t T, int ign, int64_t* count, hipStream_t s) {
  TimedLaunch timer("ce_count", s);
  hipLaunchKernelGGL(count_valid_kernel, dim3(1), dim3(kCeThreads), 0, s, labels, T, ign, count);
  return hipGetLastError();
}

hipError_t launch_cross_entropy(const void* logits, const int32_t* labels, float* loss_tok, double* loss_sum,
                                void* dlogits, const int64_t* total_count, float dloss, int64_t T, int V, int ign,
                                bool bf16_in, hipStream_t s) {
  hipError_t e;
  {
    TimedLaunch timer("ce_rows", s);
    if (bf16_in)
      e = launch_ce_pick<bf16>(static_cast<const bf16*>(logits), labels, loss_tok, static_cast<bf16*>(dlogits),
                               total_count, dloss, T, V, ign, s);
    else
      e = launch_ce_pick<float>(static_cast<const float*>(logits), labels, loss_tok, static_cast<float*>(dlogits),
                                total_count, dloss, T, V, ign, s);
  }
  if (e != hipSuccess) return e;
  TimedLaunch timer("ce_sum", s);
  hipLaunchKernelGGL(sum_loss_kernel, dim3(1), dim3(kCeThreads), 0, s, loss_tok, T, loss_sum);
  return hipGetLastError();
}

hipError_t launch_loss_combine(const double* loss_sums, const int64_t* counts, int P, int64_t* total_out,
                               double* loss_out, hipStream_t s) {
  TimedLaunch timer("loss_combine", s);
  hipLaunchKernelGGL(combine_kernel, dim3(1), dim3(kCeThreads), 0, s, loss_sums, counts, P, total_out, loss_out);
  return hipGetLastError();
}

}  // namespace ul
