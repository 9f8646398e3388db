// Document bounds of a packed sequence from its position ids (page "Ulysses
// verteilt Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch,
// section "Integration in den Hugging-Face-Stack": position ids replace the
// 4-D mask and keep the extra memory linear).
//
// A token t starts a document iff t == 0 or pos[t] == 0, and ends one iff
// t == N-1 or pos[t+1] == 0.  doc_start is the running maximum of the start
// candidates (t for a start, 0 otherwise) and doc_end the running minimum,
// from the right, of the end candidates (t for an end, N-1 otherwise).
// Two passes: per-block max/min, then a block scan seeded with the carries
// of the blocks before (max) and after (min).  O(N) bytes, negligible next to
// attention.
#include "ul_internal.h"

#include <mutex>

namespace ul {
namespace {

constexpr int kThreads = 256;
constexpr int kPer = kScanBlock / kThreads;  // 4 tokens per thread

__device__ inline int start_cand(const int32_t* pos, int t) {
  return (t == 0 || (pos != nullptr && pos[t] == 0)) ? t : 0;
}
__device__ inline int end_cand(const int32_t* pos, int t, int N) {
  return (t == N - 1 || (pos != nullptr && pos[t + 1] == 0)) ? t : N - 1;
}

__device__ inline int wave_max(int x) {
  for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ inline int wave_min(int x) {
  for (int o = 32; o > 0; o >>= 1) x = min(x, __shfl_xor(x, o, 64));
  return x;
}

__global__ void __launch_bounds__(kThreads) docb_reduce(const int32_t* __restrict__ pos, int32_t* __restrict__ scan,
                                                      int N, int nblk) {
  __shared__ int smax[kThreads / 64], smin[kThreads / 64];
  const int b = blockIdx.x;
  int mx = 0, mn = N - 1;
  for (int e = 0; e < kPer; ++e) {
    const int t = b * kScanBlock + threadIdx.x * kPer + e;
    if (t < N) {
      mx = max(mx, start_cand(pos, t));
      mn = min(mn, end_cand(pos, t, N));
    }
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  if (l == 0) { smax[w] = mx; smin[w] = mn; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) { mx = max(mx, smax[i]); mn = min(mn, smin[i]); }
    scan[b] = mx;
    scan[nblk + b] = mn;
  }
}

__global__ void __launch_bounds__(kThreads) docb_scan(const int32_t* __restrict__ pos, const int32_t* __restrict__ scan,
                                                    int32_t* __restrict__ doc_start, int32_t* __restrict__ doc_end,
                                                    int N, int nblk) {
  __shared__ int sa[kThreads / 64], sb[kThreads / 64];
  __shared__ int carry_max, carry_min;
  const int b = blockIdx.x;
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  // carries from the other blocks
  int cmax = 0, cmin = N - 1;
  for (int i = threadIdx.x; i < b; i += kThreads) cmax = max(cmax, scan[i]);
  for (int i = b + 1 + threadIdx.x; i < nblk; i += kThreads) cmin = min(cmin, scan[nblk + i]);
  cmax = wave_max(cmax);
  cmin = wave_min(cmin);
  if (l == 0) { sa[w] = cmax; sb[w] = cmin; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kThreads / 64; ++i) { cmax = max(cmax, sa[i]); cmin = min(cmin, sb[i]); }
    carry_max = cmax;
    carry_min = cmin;
  }
  __syncthreads();
  // thread-local candidates
  int s[kPer], e[kPer];
  const int t0 = b * kScanBlock + threadIdx.x * kPer;
  for (int j = 0; j < kPer; ++j) {
    const int t = t0 + j;
    s[j] = t < N ? start_cand(pos, t) : 0;
    e[j] = t < N ? end_cand(pos, t, N) : N - 1;
  }
  for (int j = 1; j < kPer; ++j) s[j] = max(s[j], s[j - 1]);
  for (int j = kPer - 2; j >= 0; --j) e[j] = min(e[j], e[j + 1]);
  // exclusive prefix max over threads to the left, exclusive suffix min over threads to the right
  int pm = s[kPer - 1], sm = e[0];
  for (int o = 1; o < 64; o <<= 1) {
    const int up = __shfl_up(pm, o, 64);
    const int dn = __shfl_down(sm, o, 64);
    if (l >= o) pm = max(pm, up);
    if (l + o < 64) sm = min(sm, dn);
  }
  // pm: inclusive prefix within the wave; sm: inclusive suffix within the wave
  __syncthreads();
  if (l == 63) sa[w] = pm;
  if (l == 0) sb[w] = sm;
  __syncthreads();
  int left = carry_max, right = carry_min;
  for (int i = 0; i < w; ++i) left = max(left, sa[i]);
  for (int i = w + 1; i < kThreads / 64; ++i) right = min(right, sb[i]);
  const int lpm = __shfl_up(pm, 1, 64);
  const int rsm = __shfl_down(sm, 1, 64);
  if (l > 0) left = max(left, lpm);
  if (l < 63) right = min(right, rsm);
  for (int j = 0; j < kPer; ++j) {
    const int t = t0 + j;
    if (t < N) {
      doc_start[t] = max(left, s[j]);
      doc_end[t] = min(right, e[j]);
    }
  }
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

// Scan partials of the allocation-free entry point: one array per GPU, held
// until the process ends.  In host code `scratch` is only a stand-in for the
// device symbol; its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) int32_t scratch[2 * ((kNoAllocMaxN + kScanBlock - 1) / kScanBlock)];

hipError_t noalloc_scan_scratch(hipStream_t stream, int32_t** out) {
  // the device the work will run on: the stream's, or the current one for the null stream
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // once per device, with that device current
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(ptr);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_doc_bounds(const int32_t* pos, int32_t* doc_start, int32_t* doc_end, int32_t* scan, int N,
                             hipStream_t s) {
  const int nblk = (N + kScanBlock - 1) / kScanBlock;
  TimedLaunch timer("doc_bounds", s);
  hipLaunchKernelGGL(docb_reduce, dim3(nblk), dim3(kThreads), 0, s, pos, scan, N, nblk);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(docb_scan, dim3(nblk), dim3(kThreads), 0, s, pos, scan, doc_start, doc_end, N, nblk);
  return hipGetLastError();
}

}  // namespace ul
