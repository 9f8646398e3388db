// Steps 1 and 3 of the Ulysses path: the seq->head and head->seq exchanges
// of one rank (page "Hugging Face并行加速：10倍提升超长序列训练效率", nmedialink.com,
// section "Ulysses的工作原理", steps 1, 3 and 5).
//
// The rank's slice of a token row [H][D] is the contiguous run of heads
// [rank*H/P, (rank+1)*H/P), so each exchange copies N runs of (H/P)*D
// elements between a row stride of H*D (sequence layout) and a row stride of
// (H/P)*D (head layout).  Runs are 256 B - 2 KiB, so plain vector copies are
// coalesced on both sides without staging through LDS: consecutive lanes read
// and write consecutive 16-byte units of the same run.  The kernel is pure
// HBM traffic (one read and one write of every element of the slice).
#include "ul_internal.h"

namespace ul {
namespace {

template <typename T, int kThreads, int kUnroll>
__global__ void __launch_bounds__(kThreads) relayout_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                          int64_t total, int64_t run, int lg_run,
                                                          int64_t stride, int64_t off, int seq_to_head) {
  const int64_t base = (int64_t)blockIdx.x * (kThreads * kUnroll) + threadIdx.x;
  T v[kUnroll];
  int64_t other[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t idx = base + (int64_t)u * kThreads;
    const int64_t row = lg_run >= 0 ? (idx >> lg_run) : (idx / run);
    const int64_t col = idx - row * run;
    other[u] = row * stride + off + col;
  }
  if (seq_to_head) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t idx = base + (int64_t)u * kThreads;
      if (idx < total) v[u] = __builtin_nontemporal_load(src + other[u]);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t idx = base + (int64_t)u * kThreads;
      if (idx < total) __builtin_nontemporal_store(v[u], dst + idx);
    }
  } else {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t idx = base + (int64_t)u * kThreads;
      if (idx < total) v[u] = __builtin_nontemporal_load(src + idx);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t idx = base + (int64_t)u * kThreads;
      if (idx < total) __builtin_nontemporal_store(v[u], dst + other[u]);
    }
  }
}

int ilog2_exact(int64_t x) {
  if (x <= 0 || (x & (x - 1))) return -1;
  int l = 0;
  while ((int64_t(1) << l) < x) ++l;
  return l;
}

template <typename T, int kThreads, int kUnroll>
hipError_t launch_shape(const void* src, void* dst, int64_t N, int64_t run_bytes, int64_t row_bytes,
                        int64_t off_bytes, bool s2h, hipStream_t s) {
  const int64_t run = run_bytes / (int64_t)sizeof(T);
  const int64_t total = N * run;
  const int64_t per_block = (int64_t)kThreads * kUnroll;
  const int64_t blocks = (total + per_block - 1) / per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  TimedLaunch timer(s2h ? "relayout_seq_to_head" : "relayout_head_to_seq", s);
  hipLaunchKernelGGL((relayout_kernel<T, kThreads, kUnroll>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     static_cast<const T*>(src), static_cast<T*>(dst), total, run, ilog2_exact(run),
                     row_bytes / (int64_t)sizeof(T), off_bytes / (int64_t)sizeof(T), s2h ? 1 : 0);
  return hipGetLastError();
}

// Block size and units per thread by run length and direction, the fastest of {256, 512, 1024}
// threads x {1, 2} units measured per shape at the million-token share (256 B - 2 KiB runs, both
// directions): short runs favour small blocks, 2 KiB runs large ones, and the 512 B head->seq
// writes two units per thread.
template <typename T>
hipError_t launch_t(const void* src, void* dst, int64_t N, int64_t run_bytes, int64_t row_bytes,
                    int64_t off_bytes, bool s2h, hipStream_t s) {
  if (run_bytes >= 2048) return launch_shape<T, 1024, 1>(src, dst, N, run_bytes, row_bytes, off_bytes, s2h, s);
  if (run_bytes <= 256 || (s2h && run_bytes > 512))
    return launch_shape<T, 256, 1>(src, dst, N, run_bytes, row_bytes, off_bytes, s2h, s);
  if (!s2h && run_bytes <= 512) return launch_shape<T, 512, 2>(src, dst, N, run_bytes, row_bytes, off_bytes, s2h, s);
  return launch_shape<T, 512, 1>(src, dst, N, run_bytes, row_bytes, off_bytes, s2h, s);
}

}  // namespace

hipError_t launch_relayout(const void* src, void* dst, int64_t N, int H, int D, int P, int rank,
                           int elem_bytes, bool seq_to_head, hipStream_t s) {
  const int64_t hp = H / P;
  const int64_t run_bytes = hp * D * elem_bytes;
  const int64_t row_bytes = (int64_t)H * D * elem_bytes;
  const int64_t off_bytes = (int64_t)rank * run_bytes;
  // widest unit that divides every run, row stride and offset and both base addresses
  const uint64_t align = (uint64_t)run_bytes | (uint64_t)row_bytes | (uint64_t)off_bytes |
                         (uint64_t)(uintptr_t)src | (uint64_t)(uintptr_t)dst;
  if ((align & 15) == 0) return launch_t<u32x4>(src, dst, N, run_bytes, row_bytes, off_bytes, seq_to_head, s);
  if ((align & 7) == 0) return launch_t<u32x2>(src, dst, N, run_bytes, row_bytes, off_bytes, seq_to_head, s);
  if ((align & 3) == 0) return launch_t<uint32_t>(src, dst, N, run_bytes, row_bytes, off_bytes, seq_to_head, s);
  if ((align & 1) == 0) return launch_t<uint16_t>(src, dst, N, run_bytes, row_bytes, off_bytes, seq_to_head, s);
  return launch_t<uint8_t>(src, dst, N, run_bytes, row_bytes, off_bytes, seq_to_head, s);
}

}  // namespace ul
