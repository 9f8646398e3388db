// Calibration probe, not part of the attention path: the bf16 MFMA rate this
// board sustains with random operands, where the matrix units alone can hold
// it at its power cap.  Each wave (one per SIMD) keeps 256 accumulator
// registers and two sets of operand fragments loaded from a buffer of random
// bf16 values, and runs nothing but MFMAs on them, alternating the two sets,
// so the operand bits toggle as they do in real work.  bench.py --mfma-ceiling
// reports the result next to the attention kernels' rates.
//
// A second family of kernels adds, per MFMA, the other work of the attention
// kernels' tile loops in the proportions their compiled code has (LDS reads,
// transpose reads, exponentials, other vector ALU instructions, global loads
// staged into LDS), with no dependency that would stall the issue: the rate
// such a mix reaches is the ceiling of a kernel with that instruction mix at
// the same power cap.
//
// Built into its own library (libul_probe.so), outside the C ABI of ul.h.
#include <hip/hip_runtime.h>

#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // four waves, one per SIMD
constexpr int kBlocks = 1024;  // four work-groups per CU over 256 CUs

// v_mfma_f32_32x32x16_bf16: 4 x 4 accumulator blocks, 32 MFMAs (2^20 flops) per iteration and wave
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma32_kernel(const bf16x8* __restrict__ in, float* __restrict__ out, int iters) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a0[i] = in[t * 16 + i];
    b0[i] = in[t * 16 + 4 + i];
    a1[i] = in[t * 16 + 8 + i];
    b1[i] = in[t * 16 + 12 + i];
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[t] = s;
}

// v_mfma_f32_16x16x32_bf16: 8 x 8 accumulator blocks, 64 MFMAs (2^20 flops) per iteration and wave
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mfma16_kernel(const bf16x8* __restrict__ in, float* __restrict__ out, int iters) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a0[8], b0[8], a1[8], b1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a0[i] = in[t * 32 + i];
    b0[i] = in[t * 32 + 8 + i];
    a1[i] = in[t * 32 + 16 + i];
    b1[i] = in[t * 32 + 24 + i];
  }
  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
  for (int it = 0; it < iters; it += 2) {
    // two half-iterations per pass: the same 2^20 flops per iteration as the 32x32x16 kernel
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += acc[i][j][e];
  out[t] = s;
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

constexpr int kMixThreads = 512;       // eight waves, two per SIMD, as the attention kernels
constexpr int kMixBlocks = 256 * 4;    // four rounds of one work-group per CU
constexpr int kMixReadBytes = 65536;   // LDS the reads and the staged writes cycle over
constexpr int kMixLdsBytes = 98304;    // allocated per work-group, so that one work-group fits a CU
constexpr int kMixInChunks = 1 << 18;  // operand buffer: 4 MiB of random bf16, resident in L2

// Per body: NM MFMAs (v_mfma_f32_32x32x16_bf16), NB ds_read_b128, NT ds_read_b64_tr_b16 (in
// pairs, each pair one MFMA operand), NE v_exp_f32, NV other VALU instructions (NB of them
// consume the loaded words, NE add the exponentials, the rest are independent FMA chains), and
// NG 16-byte global loads written to LDS at the end of the body.  Slot J of the body holds
// MFMA J and the J-th share of every other count.
template <int NM, int NB, int NT, int NE, int NV, int NG>
struct Mix {
  static_assert(NT % 2 == 0 && NV >= NB + NE, "mix counts");
  static constexpr int kPlain = NV - NB - NE;
  struct State {
    f32x16 acc[4];
    float y[8];
    bf16x8 A, B;
    u32x4 g[NG > 0 ? NG : 1];
  };
  template <int J>
  static __device__ __forceinline__ void slot(State& st, const char* smem, const u32x4* __restrict__ in, int rbase,
                                              int tbase, int gbase) {
    // every read of a body has its own address (no two can be merged), and the bases move every
    // iteration (rbase, tbase), so nothing is hoisted out of the loop
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    constexpr int vk0 = J * NB / NM + J * NE / NM + J * kPlain / NM;
    int vk = vk0;
#pragma unroll
    for (int q = J * NG / NM; q < (J + 1) * NG / NM; ++q)
      st.g[q] = __builtin_nontemporal_load(in + ((gbase + q * 512) & (kMixInChunks - 1)));
    int nop = 0;
#pragma unroll
    for (int p = J * (NT / 2) / NM; p < (J + 1) * (NT / 2) / NM; ++p) {
      const int off = tbase + p * 1040;  // below 24576 + 512 + 31 * 1040 + 512 + 8
      const s16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off));
      const s16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off + 512));
      const s16x8 tt = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
      if (nop++ == 0) st.A = __builtin_bit_cast(bf16x8, tt); else st.B = __builtin_bit_cast(bf16x8, tt);
    }
#pragma unroll
    for (int r = J * NB / NM; r < (J + 1) * NB / NM; ++r) {
      const int off = rbase + r * 400;  // below 24576 + 8192 + 79 * 400 + 16
      const u32x4 v = *reinterpret_cast<const u32x4*>(smem + off);
      if (nop == 0) st.A = __builtin_bit_cast(bf16x8, v);
      else if (nop == 1) st.B = __builtin_bit_cast(bf16x8, v);
      ++nop;
      st.y[vk & 7] = __builtin_fmaf(st.y[vk & 7], 0.5f, __builtin_bit_cast(float, v[r & 3]));
      ++vk;
    }
    st.acc[J & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(st.A, st.B, st.acc[J & 3], 0, 0, 0);
#pragma unroll
    for (int e = J * NE / NM; e < (J + 1) * NE / NM; ++e) {
      st.y[vk & 7] = __builtin_fmaf(__builtin_amdgcn_exp2f(-__builtin_fabsf(st.y[(vk + 3) & 7])), 0.75f, st.y[vk & 7]);
      ++vk;
    }
#pragma unroll
    for (int v = J * kPlain / NM; v < (J + 1) * kPlain / NM; ++v) {
      st.y[vk & 7] = __builtin_fmaf(st.y[vk & 7], -0.5f, 0.25f);
      ++vk;
    }
    // each slot's loads are issued one slot ahead of their MFMA at most: the scheduler may not
    // hoist a whole body's reads to its top (that would need more registers than a wave has)
    if constexpr ((J & 1) == 1) __builtin_amdgcn_sched_barrier(0);
    if constexpr (J + 1 < NM) slot<J + 1>(st, smem, in, rbase, tbase, gbase);
  }
};

template <int NM, int NB, int NT, int NE, int NV, int NG>
__global__ void __launch_bounds__(kMixThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mix_kernel(const u32x4* __restrict__ in, float* __restrict__ out, int iters) {
  using M = Mix<NM, NB, NT, NE, NV, NG>;
  __shared__ __attribute__((aligned(16))) char smem[kMixLdsBytes];
  const int tid = threadIdx.x, l = tid & 63;
  const int blk = blockIdx.x & 63;
  for (int i = tid; i < kMixReadBytes / 16; i += kMixThreads)
    *reinterpret_cast<u32x4*>(smem + i * 16) = in[blk * (kMixReadBytes / 16) + i];
  __syncthreads();
  // b128 reads: lanes l and l + 32 on row l & 31 (256-byte rows); the 16 lanes of each quarter
  // wave on 16 different 16-byte chunks, so every read is free of bank conflicts
  const int rbase = (l & 31) * 256 + ((((l >> 5) + (l & 15)) & 15) << 4);
  // transpose reads: 512 contiguous bytes per wave
  const int tbase = l * 8;
  typename M::State st;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) st.y[k] = 0.125f * (float)(k + 1);
  st.A = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + rbase));
  st.B = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(smem + (rbase ^ 4096)));
  for (int it = 0; it < iters; ++it) {
    const int step = (it & 3) << 13;
    M::template slot<0>(st, smem, in, rbase + step, tbase + step, blk * 4096 + it * 64 + tid);
    // the staged loads land in the read region (a later iteration reads them back)
#pragma unroll
    for (int q = 0; q < NG; ++q)
      *reinterpret_cast<u32x4*>(smem + tid * 16 + (q & 7) * 2048 + 32768) = st.g[q];
  }
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += st.y[k];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += st.acc[j][e];
  out[blockIdx.x * kMixThreads + tid] = s;
}

// The mixes, counted in the compiled tile loops of the attention kernels on fully visible
// tiles (D = 128, two tiles of the forward, one of dK/dV, half a tile of dQ):
//   0 forward: 64 MFMAs, 64 b128 reads, 64 exponentials, 265 other VALU, 8 staged 16-byte loads;
//   1 dQ:      48 MFMAs, 16 b128 + 16 transpose reads, 32 exponentials, 107 other VALU, 4 loads;
//   2 dK/dV:   64 MFMAs, 80 b128 + 64 transpose reads, 32 exponentials, 124 other VALU, 8 loads.
// The compiled probe bodies hold the same counts: their VALU argument is below the target by the
// address arithmetic the compiler adds to each body (25, 14 and 26 instructions), except that the
// dK/dV body holds 138 other VALU instructions, not 124: every loaded word needs a consumer here
// (NV >= NB + NE), which puts the floor of that body at 112 + 26.  The dQ kernel
// runs one wave per SIMD (each fragment it reads feeds two MFMAs); the probe keeps two, so its
// rate is that of the mix with the latencies hidden.
constexpr int kMixMfmas[3] = {64, 48, 64};

}  // namespace

extern "C" {

// Bytes of random bf16 operands (device) the probe reads for `shape` (32 or 16), or 0.
size_t ul_probe_operand_bytes(int shape) {
  if (shape == 32) return (size_t)kBlocks * kThreads * 16 * 16;
  if (shape == 16) return (size_t)kBlocks * kThreads * 32 * 16;
  return 0;
}

// Bytes of the float output buffer (device) the probe writes.
size_t ul_probe_out_bytes(void) { return (size_t)kBlocks * kThreads * sizeof(float); }

// Flops of one launch: 2^20 per iteration and wave, kBlocks * 4 waves.
double ul_probe_flops_per_launch(int iters) { return (double)iters * 1048576.0 * kBlocks * 4; }

// Runs `launches` launches of the shape-`shape` kernel (32: v_mfma_f32_32x32x16_bf16, 16:
// v_mfma_f32_16x16x32_bf16) with `iters` iterations each (even, 2..2^20) on `stream`, after one
// untimed launch, and stores the elapsed milliseconds of the timed ones (hipEvents on that stream)
// in *ms.  `operands` and `out` are device buffers of at least ul_probe_operand_bytes(shape) and
// ul_probe_out_bytes().  Returns 0, or 1 for bad arguments (nothing launched), 2 for a HIP error.
int ul_probe_mfma_rate(int shape, int launches, int iters, const void* operands, size_t operand_bytes, void* out,
                       size_t out_bytes, float* ms, void* stream) {
  if ((shape != 32 && shape != 16) || launches < 1 || launches > 10000 || iters < 2 || iters > (1 << 20) ||
      (iters & 1) || operands == nullptr || out == nullptr || ms == nullptr ||
      operand_bytes < ul_probe_operand_bytes(shape) || out_bytes < ul_probe_out_bytes())
    return 1;
  hipStream_t s = (hipStream_t)stream;
  const bf16x8* in = static_cast<const bf16x8*>(operands);
  float* o = static_cast<float*>(out);
  auto launch = [&]() {
    if (shape == 32)
      hipLaunchKernelGGL(mfma32_kernel, dim3(kBlocks), dim3(kThreads), 0, s, in, o, iters);
    else
      hipLaunchKernelGGL(mfma16_kernel, dim3(kBlocks), dim3(kThreads), 0, s, in, o, iters);
  };
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 2;
  launch();
  (void)hipEventRecord(a, s);
  for (int r = 0; r < launches; ++r) launch();
  (void)hipEventRecord(b, s);
  hipError_t e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (e == hipSuccess) e = hipGetLastError();
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return e == hipSuccess ? 0 : 2;
}

// Bytes of the operand buffer (device, random bf16) and of the float output buffer the mix kernels use.
size_t ul_probe_mix_operand_bytes(void) { return (size_t)kMixInChunks * 16; }
size_t ul_probe_mix_out_bytes(void) { return (size_t)kMixBlocks * kMixThreads * sizeof(float); }

// MFMA flops of one launch of mix `kind` (0 forward, 1 dQ, 2 dK/dV) with `iters` iterations, or 0.
double ul_probe_mix_flops_per_launch(int kind, int iters) {
  if (kind < 0 || kind > 2) return 0.0;
  return (double)iters * kMixMfmas[kind] * 32768.0 * kMixBlocks * (kMixThreads / 64);
}

// Runs `launches` timed launches (after one untimed) of mix `kind` with `iters` iterations each
// (1..2^20) on `stream` and stores their elapsed milliseconds in *ms.  Returns 0, 1 for bad
// arguments (nothing launched), 2 for a HIP error.
int ul_probe_mix_rate(int kind, int launches, int iters, const void* operands, size_t operand_bytes, void* out,
                      size_t out_bytes, float* ms, void* stream) {
  if (kind < 0 || kind > 2 || launches < 1 || launches > 10000 || iters < 1 || iters > (1 << 20) ||
      operands == nullptr || out == nullptr || ms == nullptr || operand_bytes < ul_probe_mix_operand_bytes() ||
      out_bytes < ul_probe_mix_out_bytes())
    return 1;
  hipStream_t s = (hipStream_t)stream;
  const u32x4* in = static_cast<const u32x4*>(operands);
  float* o = static_cast<float*>(out);
  auto launch = [&]() {
    if (kind == 0)
      hipLaunchKernelGGL((mix_kernel<64, 64, 0, 64, 240, 8>), dim3(kMixBlocks), dim3(kMixThreads), 0, s, in, o, iters);
    else if (kind == 1)
      hipLaunchKernelGGL((mix_kernel<48, 16, 16, 32, 93, 4>), dim3(kMixBlocks), dim3(kMixThreads), 0, s, in, o, iters);
    else
      hipLaunchKernelGGL((mix_kernel<64, 80, 64, 32, 112, 8>), dim3(kMixBlocks), dim3(kMixThreads), 0, s, in, o, iters);
  };
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return 2;
  launch();
  (void)hipEventRecord(a, s);
  for (int r = 0; r < launches; ++r) launch();
  (void)hipEventRecord(b, s);
  hipError_t e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (e == hipSuccess) e = hipGetLastError();
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
