/*
 * ul.h - C ABI of the per-rank hot path of Ulysses sequence parallelism on
 * one AMD Instinct MI355X (gfx950).
 *
 * The path has three steps (page "Hugging Face并行加速：10倍提升超长序列训练效率",
 * nmedialink.com, section "Ulysses的工作原理", steps 1-5; page "DeepSpeed
 * Ulysses 详解", explore.n1n.ai, section "DeepSpeed-Ulysses 的核心机制：
 * All-to-All 的艺术"):
 *   1. seq->head exchange: P sequence shards [N/P, H, D] become one rank's
 *      head slice [N, H/P, D]  (ul_seq_to_head);
 *   2. causal attention over the whole sequence for that rank's heads, with
 *      grouped-query heads and documents packed into one sequence, masked
 *      from position ids instead of a 4-D mask (page "Ulysses verteilt
 *      Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch, section
 *      "Integration in den Hugging-Face-Stack")  (ul_attn_fwd, ul_attn_bwd);
 *   3. head->seq exchange, the inverse of step 1  (ul_head_to_seq).
 * On one GPU the exchange is the local permutation that pack -> all-to-all
 * -> unpack delivers to one rank; no collective is issued.
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers to contiguous row-major memory,
 *    16-byte aligned (position_ids: 4-byte aligned).  The caller owns every
 *    buffer, including the workspace; the library never allocates, frees or
 *    keeps memory between calls.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *    work and return; results are ready when the stream is synchronised.
 *  - All argument checks run before anything is enqueued.  A failed check
 *    returns UL_ERR_ARG or UL_ERR_UNSUPPORTED, enqueues nothing and leaves
 *    every output untouched; ul_last_error() then describes it.  A failed
 *    kernel launch returns UL_ERR_HIP.  Device faults surface at the caller's
 *    next synchronisation, as for any HIP work.
 *  - Outputs never alias inputs.
 *  - Element types: UL_BF16 (bfloat16) or UL_F32 (float).
 */
#ifndef UL_H
#define UL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  UL_OK = 0,
  UL_ERR_ARG = 1,         /* invalid shape, pointer, alignment, rank or workspace size */
  UL_ERR_UNSUPPORTED = 2, /* valid but not implemented (head dim, dtype, group size) */
  UL_ERR_HIP = 3          /* a HIP runtime call or kernel launch failed */
} ul_status;

typedef enum { UL_F32 = 0, UL_BF16 = 1 } ul_dtype;

/* Largest N the fp32 attention calls accept.  Their kernels are small-case
 * checks (one thread per query row, visiting its keys one after another), so
 * their run time grows as N^2 with no MFMA; larger N is refused with
 * UL_ERR_UNSUPPORTED before anything is enqueued. */
#define UL_F32_MAX_N 65536

/*
 * Step 1, seq->head exchange of rank `rank` (pages: nmedialink.com
 * "Ulysses的工作原理" steps 1 and 3; explore.n1n.ai "核心机制" steps 1 and 3).
 *   x_seq  [N][H][D]   the P sequence shards stacked in shard order; shard i
 *                      holds tokens [i*N/P, (i+1)*N/P).  Read only.
 *   x_head [N][H/P][D] written: x_head[s][k][:] = x_seq[s][rank*H/P + k][:].
 * A bit-exact copy for any element bits.  Errors (UL_ERR_ARG): N < 1,
 * H < 1, D < 1, P < 1, N % P != 0 (sequence length must divide by the rank
 * count: dailytechsnack.ch "Integration in den Hugging-Face-Stack"),
 * H % P != 0 (the degree must divide the head count: explore.n1n.ai
 * "实践指南"), rank outside [0, P), null or misaligned pointer, overlapping
 * buffers.
 */
ul_status ul_seq_to_head(const void *x_seq, void *x_head, int64_t N, int32_t H, int32_t D,
                         int32_t P, int32_t rank, ul_dtype dt, void *stream);

/*
 * Step 3, head->seq exchange of rank `rank`, the inverse of step 1 (pages:
 * nmedialink.com "Ulysses的工作原理" step 5; explore.n1n.ai "核心机制" step 5).
 *   x_head [N][H/P][D] read only.
 *   x_seq  [N][H][D]   only the head columns [rank*H/P, (rank+1)*H/P) are
 *                      written; every other byte is left untouched, so the
 *                      P ranks' calls together fill the tensor.
 * Same errors as ul_seq_to_head.  The backward pass uses the same two calls:
 * dO goes seq->head, dQ/dK/dV go head->seq (the adjoint of an all-to-all is
 * the inverse all-to-all).
 */
ul_status ul_head_to_seq(const void *x_head, void *x_seq, int64_t N, int32_t H, int32_t D,
                         int32_t P, int32_t rank, ul_dtype dt, void *stream);

/*
 * Document bounds of a packed sequence (page dailytechsnack.ch "Integration
 * in den Hugging-Face-Stack": position ids replace the 4-D mask).  A token
 * whose position id is 0 starts a document; token 0 always starts one; no
 * other value starts one.
 *   position_ids [N] int32, or NULL for one document 0..N-1.
 *   doc_start [N], doc_end [N] int32, written: first and last token of the
 *   token's document (inclusive).
 *   ws / ws_bytes: device scratch of at least ul_doc_bounds_workspace_bytes(N)
 *   bytes (8 bytes per 1024 tokens).
 * Errors (UL_ERR_ARG): N < 1 or N >= 2^31, null or misaligned output or
 * workspace, workspace too small, overlapping buffers.
 */
size_t ul_doc_bounds_workspace_bytes(int64_t N);
ul_status ul_doc_bounds(const int32_t *position_ids, int32_t *doc_start, int32_t *doc_end,
                        int64_t N, void *ws, size_t ws_bytes, void *stream);

/*
 * ul_doc_bounds without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same inputs, outputs and results as ul_doc_bounds; the
 * scan partials live in a fixed device array of the library (512 KiB on every
 * GPU it runs on, held until the process ends), so N is limited to
 * UL_DOC_BOUNDS_NOALLOC_MAX_N.  The call allocates nothing.  Every call on
 * one GPU shares that GPU's array: calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and must not be issued.
 * The array used is that of the stream's device (the current device for the
 * null stream); the pointers must be on that device.  Errors: as ul_doc_bounds, and
 * UL_ERR_ARG for N > UL_DOC_BOUNDS_NOALLOC_MAX_N; UL_ERR_HIP if the array's
 * device address cannot be obtained.
 */
#define UL_DOC_BOUNDS_NOALLOC_MAX_N (1 << 26)
ul_status ul_doc_bounds_noalloc(const int32_t *position_ids, int32_t *doc_start, int32_t *doc_end,
                                int64_t N, void *stream);

/*
 * Workspace bytes ul_attn_fwd (for_bwd = 0) or ul_attn_bwd (for_bwd = 1)
 * needs for these shapes.  Linear in N (never N^2).  Returns 0 for shapes
 * the calls would reject.
 */
size_t ul_attn_workspace_bytes(int64_t N, int32_t Hq, int32_t Hkv, int32_t D, ul_dtype dt,
                               int32_t for_bwd);

/*
 * Step 2, forward: rank-local causal attention over the whole sequence for
 * Hq query heads and Hkv KV heads (pages: nmedialink.com "Ulysses的工作原理"
 * step 4; explore.n1n.ai "核心机制" step 4).  Query head h reads KV head
 * h / (Hq/Hkv).  Key j is visible to query i iff j <= i and both lie in the
 * same document of `position_ids` (dailytechsnack.ch "Integration in den
 * Hugging-Face-Stack").
 *   q [N][Hq][D], k/v [N][Hkv][D] of type dt, read only.
 *   position_ids [N] int32 or NULL (one document).
 *   o   [N][Hq][D] of type dt, written: softmax(scale q k^T + mask) v.
 *   lse [Hq][N] float, written: natural log of sum_j exp(scale q_i.k_j) over
 *       the visible keys (kept for the backward pass).
 *   scale: logit scale (pass 1/sqrt(D) for the usual attention).
 *   ws / ws_bytes: caller-owned device workspace of at least
 *       ul_attn_workspace_bytes(N, Hq, Hkv, D, dt, 0) bytes.
 * bf16 inputs are multiplied on MFMA with fp32 accumulation and fp32 softmax;
 * the probabilities are rounded to bf16 before the P.V product.
 * Errors: UL_ERR_ARG for N < 1, Hq < 1, Hkv < 1, Hq % Hkv != 0, null or
 * misaligned pointer, workspace too small, non-finite or non-positive scale,
 * an output or the workspace overlapping any other buffer (position_ids
 * included: the document bounds are computed into the workspace from it);
 * UL_ERR_UNSUPPORTED for D not in {64, 128}, dtype not in {UL_F32, UL_BF16},
 * (bf16) a group size Hq/Hkv that is not a power of two up to 16, or (fp32)
 * N > UL_F32_MAX_N.
 */
ul_status ul_attn_fwd(const void *q, const void *k, const void *v, const int32_t *position_ids,
                      void *o, float *lse, int64_t N, int32_t Hq, int32_t Hkv, int32_t D,
                      float scale, ul_dtype dt, void *ws, size_t ws_bytes, void *stream);

/*
 * Step 2, backward of L = sum(dO * O) for the forward above.  The pages do
 * not describe the backward; it is the chain rule with P recomputed from the
 * saved lse:  dP = dO V^T, dS = P * (dP - rowsum(dO * O)),
 * dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, with dK and dV summed over
 * the query heads of a group.
 *   q, k, v, position_ids, scale: as given to ul_attn_fwd.
 *   o [N][Hq][D] and lse [Hq][N]: the forward's outputs.
 *   dout [N][Hq][D] of type dt: gradient of L with respect to o.
 *   dq [N][Hq][D], dk/dv [N][Hkv][D]: float, fully overwritten.
 *   ws / ws_bytes: at least ul_attn_workspace_bytes(N, Hq, Hkv, D, dt, 1).
 * Deterministic: the same inputs give bit-identical outputs.
 * Errors: as ul_attn_fwd.
 */
ul_status ul_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                      const void *dout, const float *lse, const int32_t *position_ids, float *dq,
                      float *dk, float *dv, int64_t N, int32_t Hq, int32_t Hkv, int32_t D,
                      float scale, ul_dtype dt, void *ws, size_t ws_bytes, void *stream);

/*
 * The whole per-rank path in one call each way, optionally in head chunks.
 * Head chunking (the "UPipe" row of the comparison table on page
 * "Ulysses 序列並行：百萬 Token 上下文訓練", setupai.cc, section "競品分析":
 * attention split by heads to cut activation memory) runs the rank's Hq/P
 * query heads as `chunks` chunks of consecutive heads, so only one chunk's
 * head-layout buffers are live at a time.  Each chunk is the same three steps
 * as the separate calls above: seq->head of its Q (and K/V) columns,
 * attention, head->seq of its outputs.
 *   q_seq [N][Hq][D], k_seq / v_seq [N][Hkv][D] of type dt: the P sequence
 *     shards stacked (as ul_seq_to_head's x_seq), read only.
 *   position_ids [N] int32 or NULL, scale: as ul_attn_fwd.
 *   P, rank: the emulated rank count and this rank; Hq, Hkv and N must be
 *     multiples of P (no KV-head replication).
 *   chunks: divides Hq/P; a chunk's q heads either cover whole groups of
 *     G = Hq/Hkv heads (then its KV heads are chunked too) or divide one group
 *     (then consecutive chunks share their KV head and its dK / dV partials are
 *     summed in chunk order).  chunks = 1 is the unchunked path.
 *   ws / ws_bytes: at least ul_rank_workspace_bytes(...) bytes, caller-owned;
 *     it holds one chunk's head-layout buffers and the attention workspace.
 * ul_rank_attn_fwd writes rank `rank`'s columns of o_seq [N][Hq][D] (type dt;
 * other columns untouched) and lse [Hq/P][N] float (natural log, the rank's
 * heads in order).  ul_rank_attn_bwd takes o_seq and lse from it and
 * do_seq [N][Hq][D] (type dt), and writes the rank's columns of the float
 * gradients dq_seq [N][Hq][D], dk_seq and dv_seq [N][Hkv][D].  For one chunk
 * the results are bit-identical to ul_seq_to_head + ul_attn_fwd/bwd +
 * ul_head_to_seq; with chunks sharing a KV head, dK and dV differ by the
 * summation order only.
 * Errors: UL_ERR_ARG for the shape rules above, a chunking that fits neither
 * case, null, misaligned or overlapping outputs, a workspace too small;
 * UL_ERR_UNSUPPORTED as ul_attn_fwd (applied to one chunk's shapes).  All
 * checks run before anything is enqueued.
 */
size_t ul_rank_workspace_bytes(int64_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t chunks,
                               ul_dtype dt, int32_t for_bwd);
ul_status ul_rank_attn_fwd(const void *q_seq, const void *k_seq, const void *v_seq,
                           const int32_t *position_ids, void *o_seq, float *lse, int64_t N, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t P, int32_t rank, int32_t chunks, float scale,
                           ul_dtype dt, void *ws, size_t ws_bytes, void *stream);
ul_status ul_rank_attn_bwd(const void *q_seq, const void *k_seq, const void *v_seq, const void *o_seq,
                           const void *do_seq, const float *lse, const int32_t *position_ids,
                           float *dq_seq, float *dk_seq, float *dv_seq, int64_t N, int32_t Hq,
                           int32_t Hkv, int32_t D, int32_t P, int32_t rank, int32_t chunks, float scale,
                           ul_dtype dt, void *ws, size_t ws_bytes, void *stream);

/*
 * The projections on either side of the path, for one rank's own token shard
 * (page "Hugging Face并行加速", nmedialink.com, section "Ulysses的工作原理":
 * step 2, each GPU projects its shard into Q, K and V; step 6, the output
 * projection after the return exchange).  bf16 operands, fp32 accumulation on
 * MFMA, bf16 results; dt must be UL_BF16.
 * ul_qkv_proj_pack: x [M][hidden] (the shard's M tokens) times
 *   w_qkv [(Hq + 2 Hkv) D][hidden] (one row per output feature: rows
 *   [0, Hq D) project Q, the next Hkv D rows K, the last Hkv D rows V; head h
 *   of a tensor is its D consecutive features).  The results go straight into
 *   the all-to-all send blocks instead of [M][H][D]:
 *   q_send [P][M][Hq/P][D] and k_send / v_send [P][M][Hkv/P][D], block j
 *   holding heads [j H/P, (j+1) H/P) for rank j (the exchange then delivers
 *   rank j the blocks j of every shard, i.e. ul_seq_to_head's x_head).
 *   hidden must be a multiple of 64 (at most 2^22); Hq and Hkv multiples of P.
 * ul_out_proj: o_seq [M][HqD] (the attention output back in the sequence
 *   layout, read as is) times w_o [hidden][HqD] -> y [M][hidden];
 *   HqD must be a multiple of 64 (at most 2^22).
 * Errors: UL_ERR_ARG for the shape rules, null or misaligned pointers, outputs
 * overlapping anything; UL_ERR_UNSUPPORTED for dt != UL_BF16.  No workspace.
 */
ul_status ul_qkv_proj_pack(const void *x, const void *w_qkv, void *q_send, void *k_send, void *v_send,
                           int64_t M, int32_t hidden, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                           ul_dtype dt, void *stream);
ul_status ul_out_proj(const void *o_seq, const void *w_o, void *y, int64_t M, int32_t hidden, int32_t HqD,
                      ul_dtype dt, void *stream);

/*
 * Token-weighted loss of a sequence-sharded step.  The data loader shards the
 * sequence and every rank computes the loss of its own shard (page "Ulysses
 * 序列並行：百萬 Token 上下文訓練", setupai.cc, section "增強重點摘要"); the
 * ranks' losses are weighted by their numbers of valid tokens (page "Ulysses
 * verteilt Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch,
 * section "Integration in den Hugging-Face-Stack").  The loss is next-token
 * cross entropy.  On P GPUs the ranks' counts, and later their loss sums, are
 * all-reduced; ul_loss_combine is the arithmetic after that all-reduce, with
 * the P partials in one device array.  All pointers are device pointers.
 *
 * ul_shift_labels: labels [N] int32 of the whole packed sequence (a value equal
 *   to ignore_index marks a token that is not trained on) and position_ids [N]
 *   int32 or NULL (one document) -> shift_labels [N] int32 with
 *   shift_labels[t] = labels[t + 1] when t + 1 < N and position_ids[t + 1] != 0,
 *   else ignore_index.  Run it before sharding: the last target of a shard is
 *   the first label of the next shard.  shift_labels must not overlap the
 *   inputs.
 * ul_ce_count: count[0] (int64) = number of labels[0..T) != ignore_index; the
 *   global count is known from the labels alone, before any logits exist.
 * ul_loss_combine: counts [P] int64 and loss_sums [P] double (may be NULL) ->
 *   total_count[0] = sum of counts (if total_count is not NULL) and
 *   loss[0] = sum(loss_sums) / total_count, or 0 when no token is valid (if
 *   loss is not NULL; it needs loss_sums).  Fixed summation order.
 * ul_cross_entropy: one shard's logits [T][V] (dtype dt, row-major) and their
 *   targets labels [T] int32 (from ul_shift_labels) -> loss_tok [T] float,
 *   the natural-log cross entropy ln(sum_v exp(x_tv)) - x_t,y_t per token (0
 *   for ignored tokens, NaN for a label outside [0, V) that is not
 *   ignore_index), and loss_sum[0] (double) = sum of loss_tok, fixed order.
 *   When dlogits is not NULL it also writes, in dtype dt, the gradient of
 *   dloss * (token-weighted loss) with respect to this shard's logits:
 *   dloss / total_count[0] * (softmax(x_t)[v] - [v == y_t]) for valid tokens,
 *   0 for ignored tokens and when total_count[0] is 0.  total_count (int64,
 *   e.g. ul_loss_combine over the ranks' ul_ce_count) is required then.
 *   dlogits may equal logits (the gradient overwrites the logits in place);
 *   any other overlap is an error.  fp32 arithmetic; each row is read from
 *   HBM once when V <= 163840 (bf16) or 81920 (fp32), else twice.
 * Errors: UL_ERR_ARG for N, T, V or P < 1, T or V >= 2^31, null or misaligned
 * pointers (logits and dlogits 16 bytes, doubles and int64 8, others 4),
 * overlapping outputs, a non-finite dloss; UL_ERR_UNSUPPORTED for a dtype
 * other than UL_F32 / UL_BF16 or a row of V elements that is not a multiple
 * of 16 bytes (V % 8 for bf16, V % 4 for fp32).  All checks run before
 * anything is enqueued.
 */
ul_status ul_shift_labels(const int32_t *labels, const int32_t *position_ids, int32_t *shift_labels, int64_t N,
                          int32_t ignore_index, void *stream);
ul_status ul_ce_count(const int32_t *labels, int64_t T, int32_t ignore_index, int64_t *count, void *stream);
ul_status ul_loss_combine(const double *loss_sums, const int64_t *counts, int32_t P, int64_t *total_count,
                          double *loss, void *stream);
ul_status ul_cross_entropy(const void *logits, const int32_t *labels, float *loss_tok, double *loss_sum,
                           void *dlogits, const int64_t *total_count, float dloss, int64_t T, int32_t V,
                           int32_t ignore_index, ul_dtype dt, void *stream);

/*
 * Optional per-kernel timing for benchmarks.  While enabled, every kernel the
 * library launches is bracketed by two hipEvents recorded on the kernel's own
 * stream; elapsed times are summed per kernel name.  Off by default.
 *   ul_timing_enable(on): switch on (1) or off (0); returns the previous state.
 *   ul_timing_reset(): wait for pending events and clear the totals.
 *   ul_timing_read(index, name, name_len, total_ms, launches): waits for
 *     pending events; for index < 0 returns the number of kernel names; for
 *     0 <= index < count copies the index-th name (NUL-terminated, truncated
 *     to name_len) and its summed milliseconds and launch count, and returns
 *     the count; returns -1 for an index out of range or a HIP event error.
 * Host memory only; no device memory is allocated (events are HIP events).
 */
int32_t ul_timing_enable(int32_t on);
void ul_timing_reset(void);
int32_t ul_timing_read(int32_t index, char *name, size_t name_len, double *total_ms,
                       int64_t *launches);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char *ul_last_error(void);

/* Library version string. */
const char *ul_version(void);

#ifdef __cplusplus
}
#endif

#endif /* UL_H */
