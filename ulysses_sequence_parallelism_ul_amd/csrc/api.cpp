// C ABI of libul: argument validation, workspace layout and dispatch.
// Every check runs before anything is enqueued; on failure nothing is
// enqueued and ul_last_error() holds the reason.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "ul_internal.h"

namespace {

thread_local std::string g_err;

ul_status fail(ul_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ul_status ok() {
  g_err.clear();
  return UL_OK;
}

ul_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(UL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(ul_dtype dt) { return dt == UL_BF16 ? 2 : dt == UL_F32 ? 4 : 0; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

struct Buf {
  const void* p;
  size_t n;
  const char* name;
};

// Check non-null, alignment and pairwise non-overlap of device buffers.
ul_status check_bufs(const Buf* b, int count, uintptr_t align) {
  for (int i = 0; i < count; ++i) {
    if (b[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", b[i].name);
    if (!aligned(b[i].p, align)) return fail(UL_ERR_ARG, "%s is not %d-byte aligned", b[i].name, (int)align);
  }
  for (int i = 0; i < count; ++i)
    for (int j = i + 1; j < count; ++j)
      if (overlap(b[i].p, b[i].n, b[j].p, b[j].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", b[i].name, b[j].name);
  return UL_OK;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

// position_ids (N int32, optional) is read by the document-bounds kernels
// while they write the workspace, and must not alias that or any output.
ul_status check_position_ids(const int32_t* pos, int64_t N, const Buf* outs, int count) {
  if (pos == nullptr) return UL_OK;
  if (!aligned(pos, 4)) return fail(UL_ERR_ARG, "position_ids is not 4-byte aligned");
  for (int i = 0; i < count; ++i)
    if (overlap(pos, (size_t)N * 4, outs[i].p, outs[i].n))
      return fail(UL_ERR_ARG, "position_ids and %s overlap", outs[i].name);
  return UL_OK;
}

ul_status check_relayout(const void* src, void* dst, bool seq_to_head, int64_t N, int32_t H, int32_t D, int32_t P,
                         int32_t rank, ul_dtype dt) {
  if (dt != UL_BF16 && dt != UL_F32) return fail(UL_ERR_UNSUPPORTED, "dtype %d is not UL_F32 or UL_BF16", (int)dt);
  if (N < 1) return fail(UL_ERR_ARG, "N=%lld must be >= 1", (long long)N);
  if (H < 1 || D < 1) return fail(UL_ERR_ARG, "H=%d and D=%d must be >= 1", H, D);
  if (P < 1) return fail(UL_ERR_ARG, "P=%d must be >= 1", P);
  if (N % P != 0) return fail(UL_ERR_ARG, "sequence length N=%lld is not divisible by P=%d", (long long)N, P);
  if (H % P != 0) return fail(UL_ERR_ARG, "head count H=%d is not divisible by P=%d", H, P);
  if (rank < 0 || rank >= P) return fail(UL_ERR_ARG, "rank %d outside [0, %d)", rank, P);
  const size_t e = (size_t)elem_bytes(dt);
  const size_t full = (size_t)N * H * D * e, part = (size_t)N * (H / P) * D * e;
  Buf bufs[2] = {{src, seq_to_head ? full : part, seq_to_head ? "x_seq" : "x_head"},
                 {dst, seq_to_head ? part : full, seq_to_head ? "x_head" : "x_seq"}};
  return check_bufs(bufs, 2, 16);
}

ul_status check_attn_shapes(int64_t N, int32_t Hq, int32_t Hkv, int32_t D, float scale, ul_dtype dt) {
  if (dt != UL_BF16 && dt != UL_F32) return fail(UL_ERR_UNSUPPORTED, "dtype %d is not UL_F32 or UL_BF16", (int)dt);
  if (N < 1 || N > 0x7fffffffLL) return fail(UL_ERR_ARG, "N=%lld must be in [1, 2^31)", (long long)N);
  if (Hq < 1 || Hkv < 1) return fail(UL_ERR_ARG, "Hq=%d and Hkv=%d must be >= 1", Hq, Hkv);
  if (Hq % Hkv != 0) return fail(UL_ERR_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (D != 64 && D != 128) return fail(UL_ERR_UNSUPPORTED, "head dim D=%d is not 64 or 128", D);
  // the fp32 kernels are small-case checks (one thread per query row, keys in
  // series): their time grows as N^2, so large N is refused rather than run
  if (dt == UL_F32 && N > UL_F32_MAX_N)
    return fail(UL_ERR_UNSUPPORTED, "fp32 attention is limited to N <= %d, got N=%lld", UL_F32_MAX_N, (long long)N);
  if (dt == UL_BF16 && !(is_pow2(Hq / Hkv) && Hq / Hkv <= 16))
    return fail(UL_ERR_UNSUPPORTED, "bf16 attention needs a power-of-two group size <= 16, got %d", Hq / Hkv);
  if ((int64_t)N * (Hq / Hkv) > 0x7fffffffLL) return fail(UL_ERR_ARG, "N * Hq / Hkv must be < 2^31");
  if (!(scale > 0.0f) || !isfinite(scale)) return fail(UL_ERR_ARG, "scale must be finite and > 0");
  return UL_OK;
}

// ---- rank level: the whole per-rank path, optionally in head chunks ----

// How rank `rank`'s heads split into `chunks` chunks of consecutive q heads.
struct RankPlan {
  int hq = 0, hkv = 0, G = 0;  // the rank's q heads, KV heads and group size
  int C = 0, qc = 0, kc = 0;   // chunks, q heads and KV heads per chunk
  bool kv_shared = false;      // kc = 1 and qc < G: consecutive chunks share one KV head
  // first rank-local KV head of chunk c
  int kv0(int c) const { return kv_shared ? (c * qc) / G : c * kc; }
};

ul_status plan_rank(int64_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t rank, int32_t chunks,
                    float scale, ul_dtype dt, RankPlan* pl) {
  if (dt != UL_BF16 && dt != UL_F32) return fail(UL_ERR_UNSUPPORTED, "dtype %d is not UL_F32 or UL_BF16", (int)dt);
  if (P < 1) return fail(UL_ERR_ARG, "P=%d must be >= 1", P);
  if (rank < 0 || rank >= P) return fail(UL_ERR_ARG, "rank %d outside [0, %d)", rank, P);
  if (N < 1) return fail(UL_ERR_ARG, "N=%lld must be >= 1", (long long)N);
  if (N % P != 0) return fail(UL_ERR_ARG, "sequence length N=%lld is not divisible by P=%d", (long long)N, P);
  if (Hq < 1 || Hkv < 1 || Hq % P != 0 || Hkv % P != 0)
    return fail(UL_ERR_ARG, "Hq=%d and Hkv=%d must be positive multiples of P=%d", Hq, Hkv, P);
  RankPlan r;
  r.hq = Hq / P;
  r.hkv = Hkv / P;
  if (r.hq % r.hkv != 0) return fail(UL_ERR_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  r.G = r.hq / r.hkv;
  if (chunks < 1 || r.hq % chunks != 0)
    return fail(UL_ERR_ARG, "chunks=%d must divide the rank's %d query heads", chunks, r.hq);
  r.C = chunks;
  r.qc = r.hq / chunks;
  if (r.qc % r.G == 0) {
    r.kc = r.qc / r.G;
  } else if (r.G % r.qc == 0) {
    r.kc = 1;
    r.kv_shared = true;
  } else {
    return fail(UL_ERR_ARG, "a chunk of %d query heads neither covers whole groups of %d nor divides one", r.qc, r.G);
  }
  ul_status st = check_attn_shapes(N, r.qc, r.kc, D, scale, dt);
  if (st != UL_OK) return st;
  *pl = r;
  return UL_OK;
}

// Workspace of the rank-level calls: the per-chunk attention workspace first
// (its document bounds serve every chunk), then the chunk buffers.
struct RankWs {
  ul::WsLayout att;
  size_t qh = 0, kh = 0, vh = 0, oh = 0;           // head-layout chunks, input dtype
  size_t doh = 0, dqh = 0, dkh = 0, dvh = 0;       // bwd: dO chunk (input dtype); dQ, dK, dV chunks (fp32)
  size_t dkc = 0, dvc = 0;                         // bwd with a shared KV head: this chunk's dK, dV partials
  size_t total = 0;
};

RankWs rank_ws(int64_t N, int32_t D, ul_dtype dt, const RankPlan& r, bool for_bwd) {
  RankWs W;
  const size_t A = 256, e = (size_t)elem_bytes(dt);
  W.att = ul::ws_layout(N, r.qc, r.kc, D, dt, for_bwd);
  size_t off = ul::align_up(W.att.total, A);
  const size_t q_e = (size_t)N * r.qc * D * e, kv_e = (size_t)N * r.kc * D * e;
  W.qh = off; off = ul::align_up(off + q_e, A);
  W.kh = off; off = ul::align_up(off + kv_e, A);
  W.vh = off; off = ul::align_up(off + kv_e, A);
  W.oh = off; off = ul::align_up(off + q_e, A);
  if (for_bwd) {
    const size_t q_f = (size_t)N * r.qc * D * 4, kv_f = (size_t)N * r.kc * D * 4;
    W.doh = off; off = ul::align_up(off + q_e, A);
    W.dqh = off; off = ul::align_up(off + q_f, A);
    W.dkh = off; off = ul::align_up(off + kv_f, A);
    W.dvh = off; off = ul::align_up(off + kv_f, A);
    if (r.kv_shared && r.C > 1) {
      W.dkc = off; off = ul::align_up(off + kv_f, A);
      W.dvc = off; off = ul::align_up(off + kv_f, A);
    }
  }
  W.total = off;
  return W;
}

}  // namespace

namespace ul {

WsLayout ws_layout(int64_t N, int Hq, int Hkv, int D, ul_dtype dt, bool for_bwd) {
  WsLayout L;
  const size_t A = 256;
  const int64_t nblk = (N + kScanBlock - 1) / kScanBlock;
  const int64_t NB = (N + kTB - 1) / kTB;
  size_t off = 0;
  L.doc_start = off; off = align_up(off + (size_t)N * 4, A);
  L.doc_end = off;   off = align_up(off + (size_t)N * 4, A);
  L.scan = off;      off = align_up(off + (size_t)nblk * 8, A);
  if (dt == UL_BF16 && !for_bwd) {
    L.vt = off; off = align_up(off + (size_t)Hkv * NB * D * kTB * 2, A);
  }
  if (for_bwd) {
    L.delta = off; off = align_up(off + (size_t)Hq * N * 4, A);
  }
  if (dt == UL_BF16) {
    L.order_col = off; off = align_up(off + (size_t)col_blocks(N, Hq / Hkv) * 4, A);
    if (for_bwd) {
      L.order_key = off; off = align_up(off + (size_t)key_blocks(N) * 4, A);
    }
  }
  L.total = off;
  return L;
}

}  // namespace ul

extern "C" {

const char* ul_last_error(void) { return g_err.c_str(); }

const char* ul_version(void) { return "ulysses-mi355x 0.1 (gfx950)"; }

ul_status ul_seq_to_head(const void* x_seq, void* x_head, int64_t N, int32_t H, int32_t D, int32_t P, int32_t rank,
                         ul_dtype dt, void* stream) {
  ul_status st = check_relayout(x_seq, x_head, true, N, H, D, P, rank, dt);
  if (st != UL_OK) return st;
  return hip_status(ul::launch_relayout(x_seq, x_head, N, H, D, P, rank, elem_bytes(dt), true, (hipStream_t)stream),
                    "seq_to_head launch");
}

ul_status ul_head_to_seq(const void* x_head, void* x_seq, int64_t N, int32_t H, int32_t D, int32_t P, int32_t rank,
                         ul_dtype dt, void* stream) {
  ul_status st = check_relayout(x_head, x_seq, false, N, H, D, P, rank, dt);
  if (st != UL_OK) return st;
  return hip_status(ul::launch_relayout(x_head, x_seq, N, H, D, P, rank, elem_bytes(dt), false, (hipStream_t)stream),
                    "head_to_seq launch");
}

size_t ul_doc_bounds_workspace_bytes(int64_t N) {
  if (N < 1 || N > 0x7fffffffLL) return 0;
  return (size_t)((N + ul::kScanBlock - 1) / ul::kScanBlock) * 8;
}

ul_status ul_doc_bounds(const int32_t* position_ids, int32_t* doc_start, int32_t* doc_end, int64_t N, void* ws,
                        size_t ws_bytes, void* stream) {
  if (N < 1 || N > 0x7fffffffLL) return fail(UL_ERR_ARG, "N=%lld must be in [1, 2^31)", (long long)N);
  if (position_ids && !aligned(position_ids, 4)) return fail(UL_ERR_ARG, "position_ids is not 4-byte aligned");
  const size_t need = ul_doc_bounds_workspace_bytes(N);
  Buf bufs[3] = {{doc_start, (size_t)N * 4, "doc_start"}, {doc_end, (size_t)N * 4, "doc_end"}, {ws, need, "ws"}};
  ul_status st = check_bufs(bufs, 3, 4);
  if (st != UL_OK) return st;
  if (ws_bytes < need) return fail(UL_ERR_ARG, "workspace of %zu bytes is smaller than %zu", ws_bytes, need);
  if (position_ids && (overlap(position_ids, (size_t)N * 4, doc_start, (size_t)N * 4) ||
                       overlap(position_ids, (size_t)N * 4, doc_end, (size_t)N * 4)))
    return fail(UL_ERR_ARG, "position_ids overlaps an output");
  return hip_status(ul::launch_doc_bounds(position_ids, doc_start, doc_end, static_cast<int32_t*>(ws), (int)N,
                                          (hipStream_t)stream),
                    "doc_bounds launch");
}

ul_status ul_doc_bounds_noalloc(const int32_t* position_ids, int32_t* doc_start, int32_t* doc_end, int64_t N,
                                void* stream) {
  if (N < 1 || N > ul::kNoAllocMaxN)
    return fail(UL_ERR_ARG, "N=%lld must be in [1, %lld] for the allocation-free document bounds", (long long)N,
                (long long)ul::kNoAllocMaxN);
  if (position_ids && !aligned(position_ids, 4)) return fail(UL_ERR_ARG, "position_ids is not 4-byte aligned");
  Buf bufs[2] = {{doc_start, (size_t)N * 4, "doc_start"}, {doc_end, (size_t)N * 4, "doc_end"}};
  ul_status st = check_bufs(bufs, 2, 4);
  if (st != UL_OK) return st;
  st = check_position_ids(position_ids, N, bufs, 2);
  if (st != UL_OK) return st;
  int32_t* scan = nullptr;
  hipError_t e = ul::noalloc_scan_scratch((hipStream_t)stream, &scan);
  if (e != hipSuccess) return hip_status(e, "scratch address lookup");
  return hip_status(ul::launch_doc_bounds(position_ids, doc_start, doc_end, scan, (int)N, (hipStream_t)stream),
                    "doc_bounds launch");
}

size_t ul_attn_workspace_bytes(int64_t N, int32_t Hq, int32_t Hkv, int32_t D, ul_dtype dt, int32_t for_bwd) {
  std::string saved = g_err;
  ul_status st = check_attn_shapes(N, Hq, Hkv, D, 1.0f, dt);
  g_err = saved;
  if (st != UL_OK) return 0;
  return ul::ws_layout(N, Hq, Hkv, D, dt, for_bwd != 0).total;
}

ul_status ul_attn_fwd(const void* q, const void* k, const void* v, const int32_t* position_ids, void* o, float* lse,
                      int64_t N, int32_t Hq, int32_t Hkv, int32_t D, float scale, ul_dtype dt, void* ws,
                      size_t ws_bytes, void* stream) {
  ul_status st = check_attn_shapes(N, Hq, Hkv, D, scale, dt);
  if (st != UL_OK) return st;
  const size_t e = (size_t)elem_bytes(dt);
  const ul::WsLayout L = ul::ws_layout(N, Hq, Hkv, D, dt, false);
  const size_t nq = (size_t)N * Hq * D * e, nkv = (size_t)N * Hkv * D * e;
  Buf bufs[6] = {{q, nq, "q"}, {k, nkv, "k"}, {v, nkv, "v"}, {o, nq, "o"}, {lse, (size_t)Hq * N * 4, "lse"},
                 {ws, L.total, "ws"}};
  // q, k, v may alias each other (read only); outputs and workspace may not alias anything
  for (int i = 0; i < 6; ++i) {
    if (bufs[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", bufs[i].name);
    if (!aligned(bufs[i].p, 16)) return fail(UL_ERR_ARG, "%s is not 16-byte aligned", bufs[i].name);
  }
  for (int i = 3; i < 6; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", bufs[i].name, bufs[j].name);
  st = check_position_ids(position_ids, N, bufs + 3, 3);
  if (st != UL_OK) return st;
  if (ws_bytes < L.total) return fail(UL_ERR_ARG, "workspace of %zu bytes is smaller than %zu", ws_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  int32_t* ds = reinterpret_cast<int32_t*>(w + L.doc_start);
  int32_t* de = reinterpret_cast<int32_t*>(w + L.doc_end);
  hipError_t err = ul::launch_doc_bounds(position_ids, ds, de, reinterpret_cast<int32_t*>(w + L.scan), (int)N, s);
  if (err != hipSuccess) return hip_status(err, "doc_bounds launch");
  if (dt == UL_BF16)
    err = ul::launch_attn_fwd_bf16(static_cast<const ul::bf16*>(q), static_cast<const ul::bf16*>(k),
                                   static_cast<const ul::bf16*>(v), ds, static_cast<ul::bf16*>(o), lse,
                                   reinterpret_cast<ul::bf16*>(w + L.vt), reinterpret_cast<int32_t*>(w + L.order_col),
                                   (int)N, Hq, Hkv, D, scale, s);
  else
    err = ul::launch_attn_fwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                  static_cast<const float*>(v), ds, static_cast<float*>(o), lse, (int)N, Hq, Hkv, D,
                                  scale, s);
  return hip_status(err, "attn_fwd launch");
}

ul_status ul_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      const int32_t* position_ids, float* dq, float* dk, float* dv, int64_t N, int32_t Hq,
                      int32_t Hkv, int32_t D, float scale, ul_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  ul_status st = check_attn_shapes(N, Hq, Hkv, D, scale, dt);
  if (st != UL_OK) return st;
  const size_t e = (size_t)elem_bytes(dt);
  const ul::WsLayout L = ul::ws_layout(N, Hq, Hkv, D, dt, true);
  const size_t nq = (size_t)N * Hq * D * e, nkv = (size_t)N * Hkv * D * e;
  const size_t fq = (size_t)N * Hq * D * 4, fkv = (size_t)N * Hkv * D * 4;
  Buf bufs[10] = {{q, nq, "q"},   {k, nkv, "k"},   {v, nkv, "v"},   {o, nq, "o"},   {dout, nq, "dout"},
                  {lse, (size_t)Hq * N * 4, "lse"}, {dq, fq, "dq"}, {dk, fkv, "dk"}, {dv, fkv, "dv"},
                  {ws, L.total, "ws"}};
  for (int i = 0; i < 10; ++i) {
    if (bufs[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", bufs[i].name);
    if (!aligned(bufs[i].p, 16)) return fail(UL_ERR_ARG, "%s is not 16-byte aligned", bufs[i].name);
  }
  for (int i = 6; i < 10; ++i)
    for (int j = 0; j < 10; ++j)
      if (i != j && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", bufs[i].name, bufs[j].name);
  st = check_position_ids(position_ids, N, bufs + 6, 4);
  if (st != UL_OK) return st;
  if (ws_bytes < L.total) return fail(UL_ERR_ARG, "workspace of %zu bytes is smaller than %zu", ws_bytes, L.total);
  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  int32_t* ds = reinterpret_cast<int32_t*>(w + L.doc_start);
  int32_t* de = reinterpret_cast<int32_t*>(w + L.doc_end);
  hipError_t err = ul::launch_doc_bounds(position_ids, ds, de, reinterpret_cast<int32_t*>(w + L.scan), (int)N, s);
  if (err != hipSuccess) return hip_status(err, "doc_bounds launch");
  float* delta = reinterpret_cast<float*>(w + L.delta);
  if (dt == UL_BF16)
    err = ul::launch_attn_bwd_bf16(
        static_cast<const ul::bf16*>(q), static_cast<const ul::bf16*>(k), static_cast<const ul::bf16*>(v),
        static_cast<const ul::bf16*>(o), static_cast<const ul::bf16*>(dout), lse, ds, de, dq, dk, dv, delta,
        reinterpret_cast<int32_t*>(w + L.order_col), reinterpret_cast<int32_t*>(w + L.order_key), (int)N, Hq, Hkv, D,
        scale, s);
  else
    err = ul::launch_attn_bwd_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                                  static_cast<const float*>(v), static_cast<const float*>(o),
                                  static_cast<const float*>(dout), lse, ds, de, dq, dk, dv, delta, (int)N, Hq, Hkv,
                                  D, scale, s);
  if (err == hipErrorNotSupported) return fail(UL_ERR_UNSUPPORTED, "attn_bwd: this configuration is not built");
  return hip_status(err, "attn_bwd launch");
}

size_t ul_rank_workspace_bytes(int64_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, int32_t chunks, ul_dtype dt,
                               int32_t for_bwd) {
  std::string saved = g_err;
  RankPlan r;
  ul_status st = plan_rank(N, Hq, Hkv, D, P, 0, chunks, 1.0f, dt, &r);
  g_err = saved;
  if (st != UL_OK) return 0;
  return rank_ws(N, D, dt, r, for_bwd != 0).total;
}

ul_status ul_rank_attn_fwd(const void* q_seq, const void* k_seq, const void* v_seq, const int32_t* position_ids,
                           void* o_seq, float* lse, int64_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                           int32_t rank, int32_t chunks, float scale, ul_dtype dt, void* ws, size_t ws_bytes,
                           void* stream) {
  RankPlan r;
  ul_status st = plan_rank(N, Hq, Hkv, D, P, rank, chunks, scale, dt, &r);
  if (st != UL_OK) return st;
  const size_t e = (size_t)elem_bytes(dt);
  const RankWs W = rank_ws(N, D, dt, r, false);
  const size_t nq = (size_t)N * Hq * D * e, nkv = (size_t)N * Hkv * D * e;
  Buf bufs[6] = {{q_seq, nq, "q_seq"}, {k_seq, nkv, "k_seq"}, {v_seq, nkv, "v_seq"}, {o_seq, nq, "o_seq"},
                 {lse, (size_t)r.hq * N * 4, "lse"}, {ws, W.total, "ws"}};
  for (int i = 0; i < 6; ++i) {
    if (bufs[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", bufs[i].name);
    if (!aligned(bufs[i].p, 16)) return fail(UL_ERR_ARG, "%s is not 16-byte aligned", bufs[i].name);
  }
  for (int i = 3; i < 6; ++i)
    for (int j = 0; j < 6; ++j)
      if (i != j && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", bufs[i].name, bufs[j].name);
  st = check_position_ids(position_ids, N, bufs + 3, 3);
  if (st != UL_OK) return st;
  if (ws_bytes < W.total) return fail(UL_ERR_ARG, "workspace of %zu bytes is smaller than %zu", ws_bytes, W.total);

  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  int32_t* ds = reinterpret_cast<int32_t*>(w + W.att.doc_start);
  int32_t* de = reinterpret_cast<int32_t*>(w + W.att.doc_end);
  hipError_t err = ul::launch_doc_bounds(position_ids, ds, de, reinterpret_cast<int32_t*>(w + W.att.scan), (int)N, s);
  for (int c = 0; c < r.C && err == hipSuccess; ++c) {
    const int qpart = r.hq / r.qc * P, qidx = rank * r.C + c;  // chunk c = head block qidx of Hq / qc
    const int kvpart = Hkv / r.kc, kvidx = (rank * r.hkv + r.kv0(c)) / r.kc;
    if (c == 0 || r.kv0(c) != r.kv0(c - 1)) {
      err = ul::launch_relayout(k_seq, w + W.kh, N, Hkv, D, kvpart, kvidx, (int)e, true, s);
      if (err == hipSuccess) err = ul::launch_relayout(v_seq, w + W.vh, N, Hkv, D, kvpart, kvidx, (int)e, true, s);
    }
    if (err == hipSuccess) err = ul::launch_relayout(q_seq, w + W.qh, N, Hq, D, qpart, qidx, (int)e, true, s);
    float* lse_c = lse + (size_t)c * r.qc * N;
    if (err == hipSuccess) {
      if (dt == UL_BF16)
        err = ul::launch_attn_fwd_bf16(reinterpret_cast<const ul::bf16*>(w + W.qh),
                                       reinterpret_cast<const ul::bf16*>(w + W.kh),
                                       reinterpret_cast<const ul::bf16*>(w + W.vh), ds,
                                       reinterpret_cast<ul::bf16*>(w + W.oh), lse_c,
                                       reinterpret_cast<ul::bf16*>(w + W.att.vt),
                                       reinterpret_cast<int32_t*>(w + W.att.order_col), (int)N, r.qc, r.kc, D, scale,
                                       s);
      else
        err = ul::launch_attn_fwd_f32(reinterpret_cast<const float*>(w + W.qh),
                                      reinterpret_cast<const float*>(w + W.kh),
                                      reinterpret_cast<const float*>(w + W.vh), ds, reinterpret_cast<float*>(w + W.oh),
                                      lse_c, (int)N, r.qc, r.kc, D, scale, s);
    }
    if (err == hipSuccess) err = ul::launch_relayout(w + W.oh, o_seq, N, Hq, D, qpart, qidx, (int)e, false, s);
  }
  return hip_status(err, "rank_attn_fwd launch");
}

ul_status ul_rank_attn_bwd(const void* q_seq, const void* k_seq, const void* v_seq, const void* o_seq,
                           const void* do_seq, const float* lse, const int32_t* position_ids, float* dq_seq,
                           float* dk_seq, float* dv_seq, int64_t N, int32_t Hq, int32_t Hkv, int32_t D, int32_t P,
                           int32_t rank, int32_t chunks, float scale, ul_dtype dt, void* ws, size_t ws_bytes,
                           void* stream) {
  RankPlan r;
  ul_status st = plan_rank(N, Hq, Hkv, D, P, rank, chunks, scale, dt, &r);
  if (st != UL_OK) return st;
  const size_t e = (size_t)elem_bytes(dt);
  const RankWs W = rank_ws(N, D, dt, r, true);
  const size_t nq = (size_t)N * Hq * D * e, nkv = (size_t)N * Hkv * D * e;
  const size_t fq = (size_t)N * Hq * D * 4, fkv = (size_t)N * Hkv * D * 4;
  Buf bufs[10] = {{q_seq, nq, "q_seq"}, {k_seq, nkv, "k_seq"}, {v_seq, nkv, "v_seq"}, {o_seq, nq, "o_seq"},
                  {do_seq, nq, "do_seq"}, {lse, (size_t)r.hq * N * 4, "lse"}, {dq_seq, fq, "dq_seq"},
                  {dk_seq, fkv, "dk_seq"}, {dv_seq, fkv, "dv_seq"}, {ws, W.total, "ws"}};
  for (int i = 0; i < 10; ++i) {
    if (bufs[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", bufs[i].name);
    if (!aligned(bufs[i].p, 16)) return fail(UL_ERR_ARG, "%s is not 16-byte aligned", bufs[i].name);
  }
  for (int i = 6; i < 10; ++i)
    for (int j = 0; j < 10; ++j)
      if (i != j && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", bufs[i].name, bufs[j].name);
  st = check_position_ids(position_ids, N, bufs + 6, 4);
  if (st != UL_OK) return st;
  if (ws_bytes < W.total) return fail(UL_ERR_ARG, "workspace of %zu bytes is smaller than %zu", ws_bytes, W.total);

  hipStream_t s = (hipStream_t)stream;
  char* w = static_cast<char*>(ws);
  int32_t* ds = reinterpret_cast<int32_t*>(w + W.att.doc_start);
  int32_t* de = reinterpret_cast<int32_t*>(w + W.att.doc_end);
  float* delta = reinterpret_cast<float*>(w + W.att.delta);
  float* dqh = reinterpret_cast<float*>(w + W.dqh);
  float* dkh = reinterpret_cast<float*>(w + W.dkh);
  float* dvh = reinterpret_cast<float*>(w + W.dvh);
  const int64_t nkv_chunk = N * r.kc * D;
  hipError_t err = ul::launch_doc_bounds(position_ids, ds, de, reinterpret_cast<int32_t*>(w + W.att.scan), (int)N, s);
  for (int c = 0; c < r.C && err == hipSuccess; ++c) {
    const int qpart = r.hq / r.qc * P, qidx = rank * r.C + c;
    const int kvpart = Hkv / r.kc, kvidx = (rank * r.hkv + r.kv0(c)) / r.kc;
    const bool first_of_kv = c == 0 || r.kv0(c) != r.kv0(c - 1);
    const bool last_of_kv = c == r.C - 1 || r.kv0(c + 1) != r.kv0(c);
    if (first_of_kv) {
      err = ul::launch_relayout(k_seq, w + W.kh, N, Hkv, D, kvpart, kvidx, (int)e, true, s);
      if (err == hipSuccess) err = ul::launch_relayout(v_seq, w + W.vh, N, Hkv, D, kvpart, kvidx, (int)e, true, s);
    }
    if (err == hipSuccess) err = ul::launch_relayout(q_seq, w + W.qh, N, Hq, D, qpart, qidx, (int)e, true, s);
    if (err == hipSuccess) err = ul::launch_relayout(o_seq, w + W.oh, N, Hq, D, qpart, qidx, (int)e, true, s);
    if (err == hipSuccess) err = ul::launch_relayout(do_seq, w + W.doh, N, Hq, D, qpart, qidx, (int)e, true, s);
    // the first chunk of a KV head writes its dK / dV accumulators, later chunks their own partials
    float* dk_out = first_of_kv ? dkh : reinterpret_cast<float*>(w + W.dkc);
    float* dv_out = first_of_kv ? dvh : reinterpret_cast<float*>(w + W.dvc);
    const float* lse_c = lse + (size_t)c * r.qc * N;
    if (err == hipSuccess) {
      if (dt == UL_BF16)
        err = ul::launch_attn_bwd_bf16(
            reinterpret_cast<const ul::bf16*>(w + W.qh), reinterpret_cast<const ul::bf16*>(w + W.kh),
            reinterpret_cast<const ul::bf16*>(w + W.vh), reinterpret_cast<const ul::bf16*>(w + W.oh),
            reinterpret_cast<const ul::bf16*>(w + W.doh), lse_c, ds, de, dqh, dk_out, dv_out, delta,
            reinterpret_cast<int32_t*>(w + W.att.order_col), reinterpret_cast<int32_t*>(w + W.att.order_key), (int)N,
            r.qc, r.kc, D, scale, s);
      else
        err = ul::launch_attn_bwd_f32(
            reinterpret_cast<const float*>(w + W.qh), reinterpret_cast<const float*>(w + W.kh),
            reinterpret_cast<const float*>(w + W.vh), reinterpret_cast<const float*>(w + W.oh),
            reinterpret_cast<const float*>(w + W.doh), lse_c, ds, de, dqh, dk_out, dv_out, delta, (int)N, r.qc,
            r.kc, D, scale, s);
    }
    if (err == hipSuccess && !first_of_kv) {
      err = ul::launch_add_f32(dkh, dk_out, nkv_chunk, s);
      if (err == hipSuccess) err = ul::launch_add_f32(dvh, dv_out, nkv_chunk, s);
    }
    if (err == hipSuccess) err = ul::launch_relayout(dqh, dq_seq, N, Hq, D, qpart, qidx, 4, false, s);
    if (err == hipSuccess && last_of_kv) {
      err = ul::launch_relayout(dkh, dk_seq, N, Hkv, D, kvpart, kvidx, 4, false, s);
      if (err == hipSuccess) err = ul::launch_relayout(dvh, dv_seq, N, Hkv, D, kvpart, kvidx, 4, false, s);
    }
  }
  if (err == hipErrorNotSupported) return fail(UL_ERR_UNSUPPORTED, "rank_attn_bwd: this configuration is not built");
  return hip_status(err, "rank_attn_bwd launch");
}

ul_status ul_qkv_proj_pack(const void* x, const void* w_qkv, void* q_send, void* k_send, void* v_send, int64_t M,
                           int32_t hidden, int32_t Hq, int32_t Hkv, int32_t D, int32_t P, ul_dtype dt,
                           void* stream) {
  if (dt != UL_BF16) return fail(UL_ERR_UNSUPPORTED, "the projections take bf16 (dtype %d)", (int)dt);
  if (M < 1) return fail(UL_ERR_ARG, "M=%lld must be >= 1", (long long)M);
  if (hidden < 64 || hidden % 64 != 0 || hidden > (1 << 22))
    return fail(UL_ERR_ARG, "hidden=%d must be a positive multiple of 64, at most 2^22", hidden);
  if (D < 1 || P < 1 || Hq < 1 || Hkv < 1) return fail(UL_ERR_ARG, "D, P, Hq and Hkv must be >= 1");
  if (Hq % P != 0 || Hkv % P != 0)
    return fail(UL_ERR_ARG, "Hq=%d and Hkv=%d must be multiples of P=%d", Hq, Hkv, P);
  const int64_t width = (int64_t)(Hq + 2 * Hkv) * D;
  if (width > 0x7fffffffLL) return fail(UL_ERR_ARG, "(Hq + 2 Hkv) * D is too large");
  const size_t xq = (size_t)M * Hq * D * 2, xkv = (size_t)M * Hkv * D * 2;
  Buf bufs[5] = {{x, (size_t)M * hidden * 2, "x"}, {w_qkv, (size_t)width * hidden * 2, "w_qkv"},
                 {q_send, xq, "q_send"}, {k_send, xkv, "k_send"}, {v_send, xkv, "v_send"}};
  for (int i = 0; i < 5; ++i) {
    if (bufs[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", bufs[i].name);
    if (!aligned(bufs[i].p, 16)) return fail(UL_ERR_ARG, "%s is not 16-byte aligned", bufs[i].name);
  }
  for (int i = 2; i < 5; ++i)
    for (int j = 0; j < 5; ++j)
      if (i != j && overlap(bufs[i].p, bufs[i].n, bufs[j].p, bufs[j].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", bufs[i].name, bufs[j].name);
  return hip_status(ul::launch_qkv_proj_pack(static_cast<const ul::bf16*>(x), static_cast<const ul::bf16*>(w_qkv),
                                             static_cast<ul::bf16*>(q_send), static_cast<ul::bf16*>(k_send),
                                             static_cast<ul::bf16*>(v_send), M, hidden, Hq, Hkv, D, P,
                                             (hipStream_t)stream),
                    "qkv_proj_pack launch");
}

ul_status ul_out_proj(const void* o_seq, const void* w_o, void* y, int64_t M, int32_t hidden, int32_t HqD,
                      ul_dtype dt, void* stream) {
  if (dt != UL_BF16) return fail(UL_ERR_UNSUPPORTED, "the projections take bf16 (dtype %d)", (int)dt);
  if (M < 1) return fail(UL_ERR_ARG, "M=%lld must be >= 1", (long long)M);
  if (hidden < 1) return fail(UL_ERR_ARG, "hidden=%d must be >= 1", hidden);
  if (HqD < 64 || HqD % 64 != 0 || HqD > (1 << 22))
    return fail(UL_ERR_ARG, "Hq*D=%d must be a positive multiple of 64, at most 2^22", HqD);
  Buf bufs[3] = {{o_seq, (size_t)M * HqD * 2, "o_seq"}, {w_o, (size_t)hidden * HqD * 2, "w_o"},
                 {y, (size_t)M * hidden * 2, "y"}};
  for (int i = 0; i < 3; ++i) {
    if (bufs[i].p == nullptr) return fail(UL_ERR_ARG, "%s is NULL", bufs[i].name);
    if (!aligned(bufs[i].p, 16)) return fail(UL_ERR_ARG, "%s is not 16-byte aligned", bufs[i].name);
  }
  for (int j = 0; j < 2; ++j)
    if (overlap(bufs[2].p, bufs[2].n, bufs[j].p, bufs[j].n))
      return fail(UL_ERR_ARG, "y and %s overlap", bufs[j].name);
  return hip_status(ul::launch_out_proj(static_cast<const ul::bf16*>(o_seq), static_cast<const ul::bf16*>(w_o),
                                        static_cast<ul::bf16*>(y), M, hidden, HqD, (hipStream_t)stream),
                    "out_proj launch");
}

ul_status ul_shift_labels(const int32_t* labels, const int32_t* position_ids, int32_t* shift_labels, int64_t N,
                          int32_t ignore_index, void* stream) {
  if (N < 1) return fail(UL_ERR_ARG, "N=%lld must be >= 1", (long long)N);
  const size_t nb = (size_t)N * 4;
  Buf bufs[3] = {{shift_labels, nb, "shift_labels"}, {labels, nb, "labels"}, {position_ids, nb, "position_ids"}};
  const int count = position_ids != nullptr ? 3 : 2;
  ul_status st = check_bufs(bufs, count, 4);
  if (st != UL_OK) return st;
  return hip_status(ul::launch_shift_labels(labels, position_ids, shift_labels, N, ignore_index, (hipStream_t)stream),
                    "shift_labels launch");
}

ul_status ul_ce_count(const int32_t* labels, int64_t T, int32_t ignore_index, int64_t* count, void* stream) {
  if (T < 1) return fail(UL_ERR_ARG, "T=%lld must be >= 1", (long long)T);
  if (labels == nullptr || count == nullptr) return fail(UL_ERR_ARG, "labels and count must not be NULL");
  if (!aligned(labels, 4) || !aligned(count, 8)) return fail(UL_ERR_ARG, "labels (4) or count (8) misaligned");
  if (overlap(count, 8, labels, (size_t)T * 4)) return fail(UL_ERR_ARG, "count and labels overlap");
  return hip_status(ul::launch_count_valid(labels, T, ignore_index, count, (hipStream_t)stream), "ce_count launch");
}

ul_status ul_loss_combine(const double* loss_sums, const int64_t* counts, int32_t P, int64_t* total_count,
                          double* loss, void* stream) {
  if (P < 1) return fail(UL_ERR_ARG, "P=%d must be >= 1", P);
  if (counts == nullptr) return fail(UL_ERR_ARG, "counts is NULL");
  if (total_count == nullptr && loss == nullptr) return fail(UL_ERR_ARG, "total_count and loss are both NULL");
  if (loss != nullptr && loss_sums == nullptr) return fail(UL_ERR_ARG, "loss needs loss_sums");
  const void* ptrs[4] = {loss_sums, counts, total_count, loss};
  for (int i = 0; i < 4; ++i)
    if (ptrs[i] != nullptr && !aligned(ptrs[i], 8)) return fail(UL_ERR_ARG, "a loss_combine pointer is not 8-byte aligned");
  const size_t pb = (size_t)P * 8;
  const size_t in_n[2] = {loss_sums ? pb : 0, pb};
  const void* outs[2] = {total_count, loss};
  for (int o = 0; o < 2; ++o) {
    if (outs[o] == nullptr) continue;
    for (int i = 0; i < 2; ++i)
      if (ptrs[i] != nullptr && overlap(outs[o], 8, ptrs[i], in_n[i]))
        return fail(UL_ERR_ARG, "loss_combine outputs overlap its inputs");
  }
  if (total_count != nullptr && loss != nullptr && overlap(total_count, 8, loss, 8))
    return fail(UL_ERR_ARG, "total_count and loss overlap");
  return hip_status(ul::launch_loss_combine(loss_sums, counts, P, total_count, loss, (hipStream_t)stream),
                    "loss_combine launch");
}

ul_status ul_cross_entropy(const void* logits, const int32_t* labels, float* loss_tok, double* loss_sum,
                           void* dlogits, const int64_t* total_count, float dloss, int64_t T, int32_t V,
                           int32_t ignore_index, ul_dtype dt, void* stream) {
  if (dt != UL_BF16 && dt != UL_F32) return fail(UL_ERR_UNSUPPORTED, "dtype %d is not UL_F32 or UL_BF16", (int)dt);
  if (T < 1 || T > 0x7fffffffLL) return fail(UL_ERR_ARG, "T=%lld must be in [1, 2^31)", (long long)T);
  if (V < 1) return fail(UL_ERR_ARG, "V=%d must be >= 1", V);
  const int eb = elem_bytes(dt);
  if (((int64_t)V * eb) % 16 != 0)
    return fail(UL_ERR_UNSUPPORTED, "a logits row (V=%d elements of %d bytes) must be a multiple of 16 bytes", V, eb);
  if (!isfinite(dloss)) return fail(UL_ERR_ARG, "dloss must be finite");
  const size_t xb = (size_t)T * V * eb;
  if (logits == nullptr || labels == nullptr || loss_tok == nullptr || loss_sum == nullptr)
    return fail(UL_ERR_ARG, "logits, labels, loss_tok and loss_sum must not be NULL");
  if (!aligned(logits, 16)) return fail(UL_ERR_ARG, "logits is not 16-byte aligned");
  if (!aligned(labels, 4) || !aligned(loss_tok, 4) || !aligned(loss_sum, 8))
    return fail(UL_ERR_ARG, "labels (4), loss_tok (4) or loss_sum (8) misaligned");
  Buf outs[2] = {{loss_tok, (size_t)T * 4, "loss_tok"}, {loss_sum, 8, "loss_sum"}};
  Buf ins[4] = {{logits, xb, "logits"}, {labels, (size_t)T * 4, "labels"}, {total_count, 8, "total_count"},
                {dlogits, xb, "dlogits"}};
  int nin = 2;
  if (dlogits != nullptr) {
    if (total_count == nullptr) return fail(UL_ERR_ARG, "dlogits needs total_count");
    if (!aligned(dlogits, 16) || !aligned(total_count, 8))
      return fail(UL_ERR_ARG, "dlogits (16) or total_count (8) misaligned");
    if (dlogits != logits && overlap(dlogits, xb, logits, xb))
      return fail(UL_ERR_ARG, "dlogits overlaps logits without being equal to it");
    if (overlap(dlogits, xb, labels, (size_t)T * 4) || overlap(dlogits, xb, total_count, 8))
      return fail(UL_ERR_ARG, "dlogits overlaps labels or total_count");
    nin = 4;
  }
  if (overlap(loss_tok, (size_t)T * 4, loss_sum, 8)) return fail(UL_ERR_ARG, "loss_tok and loss_sum overlap");
  for (int o = 0; o < 2; ++o)
    for (int i = 0; i < nin; ++i)
      if (overlap(outs[o].p, outs[o].n, ins[i].p, ins[i].n))
        return fail(UL_ERR_ARG, "%s and %s overlap", outs[o].name, ins[i].name);
  return hip_status(ul::launch_cross_entropy(logits, labels, loss_tok, loss_sum, dlogits, total_count, dloss, T, V,
                                             ignore_index, dt == UL_BF16, (hipStream_t)stream),
                    "cross_entropy launch");
}

}  // extern "C"
