// Launch order of the bf16 attention work-groups: heaviest first.
//
// Not on the pages: an implementation choice.  With packed documents the
// work of a work-group (the number of tiles its loop visits) ranges from one
// tile to a whole document, and the hardware dispatches work-groups in
// blockIdx order.  A heavy work-group dispatched late (the first key block of
// a long document that sits at the end of the sequence, say) then runs alone
// at the end of the launch.  Dispatching in decreasing order of work is the
// classic longest-processing-time list schedule; this kernel computes that
// order from the document bounds on the device, so the host never waits.
//
// One work-group per order: the work of every unit, its maximum, histograms
// over kBuckets equal-width work buckets (one per wave, each over its own
// contiguous segment of units), the suffix sums of the totals (heaviest bucket
// first) and each wave's first place per bucket, then a stable scatter by all
// waves at once, so the order is deterministic.  Each unit writes only its own
// outputs: results do not depend on the order.
#include "ul_internal.h"

namespace ul {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBuckets = 2048;
constexpr int kPer = kBuckets / kThreads;
constexpr int kBatch = 4;

__device__ inline int unit_work(const OrderJob& J, int N, int lgG, int u) {
  if (J.key_blocks) {
    // key block u (J.unit keys) against the query-column tiles (J.tile columns)
    // from its own first column to the end of its last key's document
    const int k0 = u * J.unit;
    const int kl = min(N - 1, k0 + J.unit - 1);
    const int lo = (int)(((int64_t)k0 << lgG) / J.tile);
    const int hi = (int)((((int64_t)(J.bound[kl] + 1) << lgG) - 1) / J.tile);
    return hi - lo + 1;
  }
  // column block u (J.unit query columns) against the key tiles (J.tile keys)
  // from its first row's document start to its last row
  const int64_t c0 = (int64_t)u * J.unit;
  const int rf = (int)(c0 >> lgG);
  const int rl = (int)min<int64_t>(N - 1, (c0 + J.unit - 1) >> lgG);
  return rl / J.tile - J.bound[rf] / J.tile + 1;
}

__device__ inline int bucket_of(int w, int wmax) {
  const int b = (int)((int64_t)w * kBuckets / ((int64_t)wmax + 1));
  return min(max(b, 0), kBuckets - 1);
}

__global__ void __launch_bounds__(kThreads) order_kernel(OrderJobs jobs, int N, int lgG) {
  const OrderJob J = jobs.j[blockIdx.x];
  // hist[w][b]: units of bucket b in wave w's segment of the visit order, then
  // the place where the next of them goes
  __shared__ int hist[kWaves][kBuckets];
  __shared__ int wsum[kWaves];
  __shared__ int wmax_s;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int x = tid; x < kWaves * kBuckets; x += kThreads) (&hist[0][0])[x] = 0;
  if (tid == 0) wmax_s = 0;
  __syncthreads();

  // visit order: key blocks ascending, column blocks descending (the order in
  // which work grows inside a document); wave w owns visits [v0, v1)
  auto unit_at = [&](int i) { return J.key_blocks ? i : J.units - 1 - i; };
  const int seg = (J.units + kWaves - 1) / kWaves;
  const int v0 = min(J.units, wv * seg), v1 = min(J.units, v0 + seg);

  int m = 0;
  for (int u = tid; u < J.units; u += kThreads) m = max(m, unit_work(J, N, lgG, u));
  atomicMax(&wmax_s, m);
  __syncthreads();
  const int wmax = wmax_s;
  for (int i = v0 + lane; i < v1; i += 64) atomicAdd(&hist[wv][bucket_of(unit_work(J, N, lgG, unit_at(i)), wmax)], 1);
  __syncthreads();

  // bucket totals, exclusive sums from the heaviest bucket down (thread t owns
  // buckets kBuckets-1-(t*kPer+i)), then each wave's first place per bucket
  int c[kPer], s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = kBuckets - 1 - (tid * kPer + i);
    c[i] = 0;
    for (int w = 0; w < kWaves; ++w) c[i] += hist[w][b];
    s += c[i];
  }
  int incl = s;  // inclusive scan over the wave
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int base = incl - s;
  for (int i = 0; i < wv; ++i) base += wsum[i];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int b = kBuckets - 1 - (tid * kPer + i);
    int at = base;
    for (int w = 0; w < kWaves; ++w) {
      const int n = hist[w][b];
      hist[w][b] = at;
      at += n;
    }
    base += c[i];
  }
  __syncthreads();

  // stable scatter, each wave over its own segment, 64 visits per step: a
  // lane's place is its bucket's next place in this wave's row plus the number
  // of lower lanes in the same bucket.  The buckets of kBatch steps are
  // computed together so their loads overlap.
  const uint64_t below = (1ull << lane) - 1;
  for (int i0 = v0; i0 < v1; i0 += 64 * kBatch) {
    int bb[kBatch];
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int i = i0 + r * 64 + lane;
      bb[r] = i < v1 ? bucket_of(unit_work(J, N, lgG, unit_at(i)), wmax) : -1;
    }
#pragma unroll
    for (int r = 0; r < kBatch; ++r) {
      const int b = bb[r];
      int rank = 0, group = 0;
      uint64_t rem = __ballot(b >= 0);
      while (rem) {
        const int b0 = __builtin_amdgcn_readlane(b, __ffsll((unsigned long long)rem) - 1);
        const uint64_t m = __ballot(b == b0);
        if (b == b0) {
          rank = __popcll(m & below);
          group = __popcll(m);
        }
        rem &= ~m;
      }
      if (b >= 0) {
        const int at = hist[wv][b];
        J.order[at + rank] = unit_at(i0 + r * 64 + lane);
        if (rank == group - 1) hist[wv][b] = at + group;  // the group's last lane advances its bucket
      }
    }
  }
}

}  // namespace

hipError_t launch_order(const OrderJobs& jobs, int njobs, int N, int lgG, hipStream_t s) {
  for (int i = 0; i < njobs; ++i)
    if (jobs.j[i].units < 1 || jobs.j[i].unit < 1 || jobs.j[i].tile < 1) return hipErrorInvalidValue;
  TimedLaunch timer("attn_order", s);
  hipLaunchKernelGGL(order_kernel, dim3(njobs), dim3(kThreads), 0, s, jobs, N, lgG);
  return hipGetLastError();
}

}  // namespace ul
