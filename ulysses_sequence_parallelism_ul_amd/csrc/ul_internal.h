// Internal declarations shared by the HIP translation units of libul.
// Nothing here is part of the C ABI (include/ul.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ul.h"

namespace ul {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Tokens per tile of the transposed (blocked) operand copies kept in the
// workspace: element (col, d) of a [cols][D] matrix lives at
// [col / kTB][d][col % kTB].
constexpr int kTB = 64;
// Tokens per block of the document-bounds scan.
constexpr int kScanBlock = 1024;
// Largest N of the allocation-free document bounds (its scan partials live in
// a fixed device array of 2 * N / kScanBlock int32, 512 KiB).
constexpr int64_t kNoAllocMaxN = UL_DOC_BOUNDS_NOALLOC_MAX_N;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte offsets of the workspace regions of ul_attn_fwd / ul_attn_bwd.
struct WsLayout {
  size_t doc_start = 0, doc_end = 0, scan = 0;  // int32 [N], int32 [N], int32 [2 * nblk]
  size_t vt = 0;     // bf16 fwd: V^T blocked [Hkv][NB][D][kTB]
  size_t delta = 0;  // bwd: float [Hkv][N*G] (query-column order)
  size_t order_col = 0;  // bf16: int32 launch order of the query-column blocks (forward, dQ)
  size_t order_key = 0;  // bf16 bwd: int32 launch order of the key blocks (dK/dV)
  size_t total = 0;
};

WsLayout ws_layout(int64_t N, int Hq, int Hkv, int D, ul_dtype dt, bool for_bwd);

// Optional per-kernel timing (ul_timing_enable): when on, launchers bracket
// each kernel with hipEvents recorded on the kernel's own stream.
bool timing_on();
void timing_begin(const char* name, hipStream_t s);
void timing_end(hipStream_t s);
struct TimedLaunch {
  hipStream_t s;
  bool on;
  TimedLaunch(const char* name, hipStream_t st) : s(st), on(timing_on()) {
    if (on) timing_begin(name, s);
  }
  ~TimedLaunch() {
    if (on) timing_end(s);
  }
};

// Work-group units of the bf16 attention kernels: query-column blocks of
// kColBlock columns against key tiles of kKeyTile keys (forward, dQ), and key
// blocks of kKeyBlock keys against query-column tiles of kColTile columns (dK/dV).
constexpr int kColBlock = 256, kKeyTile = 64, kKeyBlock = 128, kColTile = 64;
inline int64_t col_blocks(int64_t N, int G) { return (N * G + kColBlock - 1) / kColBlock; }
inline int64_t key_blocks(int64_t N) { return (N + kKeyBlock - 1) / kKeyBlock; }

// One launch order to compute: units 0 .. units-1 sorted by decreasing work.
struct OrderJob {
  int32_t* order;        // out: int32 [units], a permutation of 0 .. units-1
  const int32_t* bound;  // doc_end (key blocks) or doc_start (column blocks), int32 [N]
  int key_blocks;        // 1: key blocks of `unit` keys over column tiles of `tile`; 0: the transpose
  int units, unit, tile;
};
struct OrderJobs {
  OrderJob j[2];
};

// ---- launchers (enqueue only; arguments already validated) ----
hipError_t launch_order(const OrderJobs& jobs, int njobs, int N, int lgG, hipStream_t s);
hipError_t launch_relayout(const void* src, void* dst, int64_t N, int H, int D, int P, int rank,
                           int elem_bytes, bool seq_to_head, hipStream_t s);
hipError_t launch_doc_bounds(const int32_t* pos, int32_t* doc_start, int32_t* doc_end,
                             int32_t* scan_scratch, int N, hipStream_t s);
// Device address, on the device of `stream` (the current device for the null
// stream), of the fixed scan-partials array of the allocation-free document
// bounds (looked up once per device).
hipError_t noalloc_scan_scratch(hipStream_t stream, int32_t** out);
// [cols][D] bf16 view (column c -> token c >> lgG, head (hk << lgG) + (c & (G-1)) of a
// [N][H][D] tensor) -> blocked transpose [Hkv][ceil(ncols / kTB)][D][kTB], zero-padded.
hipError_t launch_transpose_blocked(const bf16* src, bf16* dst, int64_t ncols, int H, int Hkv, int lgG, int D,
                                    hipStream_t s);
// Projections (bf16 NT GEMM, fp32 accumulation): x [M][hidden] times w_qkv
// [(Hq + 2 Hkv) D][hidden] into the send blocks q_send [P][M][Hq/P][D],
// k_send / v_send [P][M][Hkv/P][D]; o_seq [M][HqD] times w_o [hidden][HqD]
// into y [M][hidden].  K (hidden, HqD) must be a multiple of 64.
hipError_t launch_qkv_proj_pack(const bf16* x, const bf16* w_qkv, bf16* q_send, bf16* k_send, bf16* v_send,
                                int64_t M, int hidden, int Hq, int Hkv, int D, int P, hipStream_t s);
hipError_t launch_out_proj(const bf16* o_seq, const bf16* w_o, bf16* y, int64_t M, int hidden, int HqD,
                           hipStream_t s);
// Loss of a sharded step: next-token targets, valid counts, per-row cross
// entropy (+ gradient when dlogits != nullptr) and the combination of ranks.
hipError_t launch_shift_labels(const int32_t* labels, const int32_t* pos, int32_t* out, int64_t N, int ign,
                               hipStream_t s);
hipError_t launch_count_valid(const int32_t* labels, int64_t T, int ign, int64_t* count, hipStream_t s);
hipError_t launch_cross_entropy(const void* logits, const int32_t* labels, float* loss_tok, double* loss_sum,
                                void* dlogits, const int64_t* total_count, float dloss, int64_t T, int V, int ign,
                                bool bf16_in, hipStream_t s);
hipError_t launch_loss_combine(const double* loss_sums, const int64_t* counts, int P, int64_t* total_out,
                               double* loss_out, hipStream_t s);
// Largest vocabulary whose rows the cross-entropy kernel keeps in registers.
int ce_max_resident_vocab(int elem_bytes);
// dst[i] += src[i] for n floats (n a multiple of 4, 16-byte aligned buffers).
hipError_t launch_add_f32(float* dst, const float* src, int64_t n, hipStream_t s);
hipError_t launch_attn_fwd_bf16(const bf16* q, const bf16* k, const bf16* v, const int32_t* doc_start,
                                bf16* o, float* lse, bf16* vt_ws, int32_t* order_ws, int N, int Hq, int Hkv,
                                int D, float scale, hipStream_t s);
hipError_t launch_attn_fwd_f32(const float* q, const float* k, const float* v, const int32_t* doc_start,
                               float* o, float* lse, int N, int Hq, int Hkv, int D, float scale,
                               hipStream_t s);
hipError_t launch_attn_bwd_bf16(const bf16* q, const bf16* k, const bf16* v, const bf16* o,
                                const bf16* dout, const float* lse, const int32_t* doc_start,
                                const int32_t* doc_end, float* dq, float* dk, float* dv, float* delta,
                                int32_t* order_col, int32_t* order_key, int N, int Hq, int Hkv, int D, float scale,
                                hipStream_t s);
hipError_t launch_attn_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                               const float* dout, const float* lse, const int32_t* doc_start,
                               const int32_t* doc_end, float* dq, float* dk, float* dv, float* delta,
                               int N, int Hq, int Hkv, int D, float scale, hipStream_t s);

}  // namespace ul
