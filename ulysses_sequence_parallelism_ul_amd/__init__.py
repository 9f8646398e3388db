"""Python binding of libul, the MI355X (gfx950) per-rank hot path of Ulysses
sequence parallelism: the seq->head exchange, causal packed-document
grouped-query attention forward and backward, and the head->seq exchange.

This module only marshals arguments: it checks torch tensors, allocates
outputs and workspaces with torch on the tensors' device, and calls the C ABI
(include/ul.h) on torch's current HIP stream.  Every step of the path runs in
the library's HIP kernels; there is no CPU or PyTorch fallback, and a missing
library raises.
"""

import ctypes
import math
import os

import torch

__all__ = [
    "UlError",
    "load",
    "library_path",
    "version",
    "seq_to_head",
    "head_to_seq",
    "doc_bounds",
    "doc_bounds_noalloc",
    "attn_workspace_bytes",
    "attn_fwd",
    "attn_bwd",
    "rank_workspace_bytes",
    "rank_attn_fwd",
    "rank_attn_bwd",
    "qkv_proj_pack",
    "out_proj",
    "IGNORE_INDEX",
    "shift_labels",
    "ce_count",
    "loss_combine",
    "cross_entropy",
    "timing_enable",
    "timing_reset",
    "timing_read",
    "UL_OK",
    "UL_ERR_ARG",
    "UL_ERR_UNSUPPORTED",
    "UL_ERR_HIP",
    "UL_F32",
    "UL_BF16",
]

UL_OK, UL_ERR_ARG, UL_ERR_UNSUPPORTED, UL_ERR_HIP = 0, 1, 2, 3
UL_F32, UL_BF16 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
# UL_LIBRARY_PATH selects another build of the same library (e.g. the host-ASan one)
library_path = os.environ.get("UL_LIBRARY_PATH") or os.path.join(_HERE, "libul.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/ul.h
SIGNATURES = {
    "ul_seq_to_head": (_I32, [_P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P]),
    "ul_head_to_seq": (_I32, [_P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _P]),
    "ul_doc_bounds_workspace_bytes": (_SZ, [_I64]),
    "ul_doc_bounds": (_I32, [_P, _P, _P, _I64, _P, _SZ, _P]),
    "ul_doc_bounds_noalloc": (_I32, [_P, _P, _P, _I64, _P]),
    "ul_attn_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _I32]),
    "ul_attn_fwd": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _F, _I32, _P, _SZ, _P]),
    "ul_attn_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _F, _I32, _P, _SZ, _P]),
    "ul_rank_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "ul_rank_attn_fwd": (_I32, [_P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F, _I32, _P, _SZ,
                                _P]),
    "ul_rank_attn_bwd": (_I32, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _F,
                                _I32, _P, _SZ, _P]),
    "ul_qkv_proj_pack": (_I32, [_P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I32, _P]),
    "ul_out_proj": (_I32, [_P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "ul_shift_labels": (_I32, [_P, _P, _P, _I64, _I32, _P]),
    "ul_ce_count": (_I32, [_P, _I64, _I32, _P, _P]),
    "ul_loss_combine": (_I32, [_P, _P, _I32, _P, _P, _P]),
    "ul_cross_entropy": (_I32, [_P, _P, _P, _P, _P, _P, _F, _I64, _I32, _I32, _I32, _P]),
    "ul_timing_enable": (_I32, [_I32]),
    "ul_timing_reset": (None, []),
    "ul_timing_read": (_I32, [_I32, ctypes.c_char_p, _SZ, ctypes.POINTER(ctypes.c_double),
                              ctypes.POINTER(ctypes.c_int64)]),
    "ul_last_error": (ctypes.c_char_p, []),
    "ul_version": (ctypes.c_char_p, []),
}


def timing_enable(on=True):
    """Bracket every library kernel with hipEvents on its stream; returns the previous state."""
    return bool(load().ul_timing_enable(1 if on else 0))


def timing_reset():
    load().ul_timing_reset()


def timing_read():
    """{kernel name: (total milliseconds, launches)} accumulated since the last reset."""
    lib = load()
    n = lib.ul_timing_read(-1, None, 0, None, None)
    if n < 0:
        raise UlError(UL_ERR_HIP, "timing read failed")
    out = {}
    buf = ctypes.create_string_buffer(128)
    ms = ctypes.c_double()
    cnt = ctypes.c_int64()
    for i in range(n):
        if lib.ul_timing_read(i, buf, 128, ctypes.byref(ms), ctypes.byref(cnt)) < 0:
            raise UlError(UL_ERR_HIP, "timing read failed")
        out[buf.value.decode()] = (ms.value, cnt.value)
    return out


class UlError(RuntimeError):
    """A non-OK status from libul; ``status`` holds the ul_status code."""

    def __init__(self, status, message):
        super().__init__(f"libul status {status}: {message}")
        self.status = status


def load():
    """Load libul.so (built in-tree by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise RuntimeError(
                f"{library_path} is not built; run `python -m ulysses_sequence_parallelism_ul_amd.build` "
                "(there is no fallback path)")
        lib = ctypes.CDLL(library_path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def version():
    return load().ul_version().decode()


def _check(status):
    if status != UL_OK:
        raise UlError(status, load().ul_last_error().decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return UL_BF16
    if t.dtype == torch.float32:
        return UL_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _dev(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def seq_to_head(x_seq, P, rank, out=None):
    """[N, H, D] stacked sequence shards -> rank's head slice [N, H/P, D] (bit-exact)."""
    lib = load()
    N, H, D = x_seq.shape
    if out is None:
        if H % P:
            raise ValueError(f"H={H} is not divisible by P={P}")
        out = torch.empty((N, H // P, D), dtype=x_seq.dtype, device=x_seq.device)
    if out.dtype != x_seq.dtype:
        raise TypeError("out dtype differs from x_seq")
    _check(lib.ul_seq_to_head(_dev(x_seq, "x_seq"), _dev(out, "out"), N, H, D, P, rank, _dtype_code(x_seq),
                              _stream(x_seq.device)))
    return out


def head_to_seq(x_head, x_seq, P, rank):
    """Write rank's head slice [N, H/P, D] into columns of x_seq [N, H, D] in place; returns x_seq."""
    lib = load()
    N, H, D = x_seq.shape
    if x_head.dtype != x_seq.dtype:
        raise TypeError("x_head dtype differs from x_seq")
    if H % P or tuple(x_head.shape) != (N, H // P, D):
        raise ValueError(f"x_head shape {tuple(x_head.shape)} does not match [N, H/P, D] for x_seq {tuple(x_seq.shape)}")
    _check(lib.ul_head_to_seq(_dev(x_head, "x_head"), _dev(x_seq, "x_seq"), N, H, D, P, rank, _dtype_code(x_seq),
                              _stream(x_seq.device)))
    return x_seq


def doc_bounds(position_ids, N=None, device=None):
    """(doc_start, doc_end) int32 [N] from int32 position ids (None: one document of length N)."""
    lib = load()
    if position_ids is not None:
        if position_ids.dtype != torch.int32:
            raise TypeError("position_ids must be int32")
        N = position_ids.numel()
        device = position_ids.device
        pptr = _dev(position_ids, "position_ids")
    else:
        pptr = None
    ds = torch.empty(N, dtype=torch.int32, device=device)
    de = torch.empty(N, dtype=torch.int32, device=device)
    wsb = lib.ul_doc_bounds_workspace_bytes(N)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=device)
    _check(lib.ul_doc_bounds(pptr, ds.data_ptr(), de.data_ptr(), N, ws.data_ptr(), wsb, _stream(device)))
    return ds, de


def doc_bounds_noalloc(position_ids, doc_start, doc_end, N=None):
    """ul_doc_bounds_noalloc into caller-allocated int32 [N] outputs (nothing is allocated)."""
    lib = load()
    pptr = None
    if position_ids is not None:
        if position_ids.dtype != torch.int32:
            raise TypeError("position_ids must be int32")
        N = position_ids.numel()
        pptr = _dev(position_ids, "position_ids")
    for t, name in ((doc_start, "doc_start"), (doc_end, "doc_end")):
        if t.dtype != torch.int32 or t.numel() != N:
            raise ValueError(f"{name} must be int32 with N={N} elements")
    _check(lib.ul_doc_bounds_noalloc(pptr, _dev(doc_start, "doc_start"), _dev(doc_end, "doc_end"), N,
                                     _stream(doc_start.device)))
    return doc_start, doc_end


def attn_workspace_bytes(N, Hq, Hkv, D, dtype, for_bwd):
    code = UL_BF16 if dtype == torch.bfloat16 else UL_F32 if dtype == torch.float32 else -1
    return load().ul_attn_workspace_bytes(N, Hq, Hkv, D, code, 1 if for_bwd else 0)


def _workspace(nbytes, device, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)
    if workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace holds fewer than {nbytes} bytes")
    return workspace


def _pos_ptr(position_ids, N):
    if position_ids is None:
        return None
    if position_ids.dtype != torch.int32 or position_ids.numel() != N:
        raise ValueError("position_ids must be int32 with N elements")
    return _dev(position_ids, "position_ids")


def attn_fwd(q, k, v, position_ids=None, scale=None, out=None, lse=None, workspace=None):
    """Causal packed-document GQA attention forward. Returns (o [N,Hq,D], lse [Hq,N] fp32)."""
    lib = load()
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != N or k.shape[2] != D or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v shapes or dtypes disagree")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((Hq, N), dtype=torch.float32, device=q.device) if lse is None else lse
    wsb = lib.ul_attn_workspace_bytes(N, Hq, Hkv, D, _dtype_code(q), 0)
    ws = _workspace(wsb, q.device, workspace)
    _check(lib.ul_attn_fwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _pos_ptr(position_ids, N), _dev(out, "out"),
                           _dev(lse, "lse"), N, Hq, Hkv, D, scale, _dtype_code(q), ws.data_ptr(), wsb,
                           _stream(q.device)))
    return out, lse


def attn_bwd(q, k, v, o, dout, lse, position_ids=None, scale=None, dq=None, dk=None, dv=None, workspace=None):
    """Backward of attn_fwd. Returns fp32 (dq [N,Hq,D], dk [N,Hkv,D], dv [N,Hkv,D])."""
    lib = load()
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((N, Hq, D), **f32) if dq is None else dq
    dk = torch.empty((N, Hkv, D), **f32) if dk is None else dk
    dv = torch.empty((N, Hkv, D), **f32) if dv is None else dv
    wsb = lib.ul_attn_workspace_bytes(N, Hq, Hkv, D, _dtype_code(q), 1)
    ws = _workspace(wsb, q.device, workspace)
    _check(lib.ul_attn_bwd(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(dout, "dout"),
                           _dev(lse, "lse"), _pos_ptr(position_ids, N), _dev(dq, "dq"), _dev(dk, "dk"),
                           _dev(dv, "dv"), N, Hq, Hkv, D, scale, _dtype_code(q), ws.data_ptr(), wsb,
                           _stream(q.device)))
    return dq, dk, dv


def rank_workspace_bytes(N, Hq, Hkv, D, P, chunks, dtype, for_bwd):
    code = UL_BF16 if dtype == torch.bfloat16 else UL_F32 if dtype == torch.float32 else -1
    return load().ul_rank_workspace_bytes(N, Hq, Hkv, D, P, chunks, code, 1 if for_bwd else 0)


def rank_attn_fwd(q_seq, k_seq, v_seq, P, rank, position_ids=None, chunks=1, scale=None, o_seq=None, lse=None,
                  workspace=None):
    """Rank's whole forward path (seq->head, attention, head->seq) in `chunks` head chunks.

    Writes the rank's columns of o_seq [N, Hq, D] (allocated with zeros if None) and returns
    (o_seq, lse [Hq/P, N] fp32)."""
    lib = load()
    N, Hq, D = q_seq.shape
    Hkv = k_seq.shape[1]
    if k_seq.shape != v_seq.shape or k_seq.dtype != q_seq.dtype or v_seq.dtype != q_seq.dtype:
        raise ValueError("q_seq, k_seq, v_seq shapes or dtypes disagree")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    o_seq = torch.zeros_like(q_seq) if o_seq is None else o_seq
    if lse is None:
        lse = torch.empty((Hq // P if P > 0 and Hq % P == 0 else 1, N), dtype=torch.float32, device=q_seq.device)
    wsb = lib.ul_rank_workspace_bytes(N, Hq, Hkv, D, P, chunks, _dtype_code(q_seq), 0)
    ws = _workspace(wsb, q_seq.device, workspace)
    _check(lib.ul_rank_attn_fwd(_dev(q_seq, "q_seq"), _dev(k_seq, "k_seq"), _dev(v_seq, "v_seq"),
                                _pos_ptr(position_ids, N), _dev(o_seq, "o_seq"), _dev(lse, "lse"), N, Hq, Hkv, D, P,
                                rank, chunks, scale, _dtype_code(q_seq), ws.data_ptr(), wsb, _stream(q_seq.device)))
    return o_seq, lse


def rank_attn_bwd(q_seq, k_seq, v_seq, o_seq, do_seq, lse, P, rank, position_ids=None, chunks=1, scale=None,
                  dq_seq=None, dk_seq=None, dv_seq=None, workspace=None):
    """Rank's whole backward path in `chunks` head chunks; returns fp32 (dq_seq, dk_seq, dv_seq) in sequence
    layout with the rank's columns written (zero-filled if allocated here)."""
    lib = load()
    N, Hq, D = q_seq.shape
    Hkv = k_seq.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    f32 = dict(dtype=torch.float32, device=q_seq.device)
    dq_seq = torch.zeros((N, Hq, D), **f32) if dq_seq is None else dq_seq
    dk_seq = torch.zeros((N, Hkv, D), **f32) if dk_seq is None else dk_seq
    dv_seq = torch.zeros((N, Hkv, D), **f32) if dv_seq is None else dv_seq
    wsb = lib.ul_rank_workspace_bytes(N, Hq, Hkv, D, P, chunks, _dtype_code(q_seq), 1)
    ws = _workspace(wsb, q_seq.device, workspace)
    _check(lib.ul_rank_attn_bwd(_dev(q_seq, "q_seq"), _dev(k_seq, "k_seq"), _dev(v_seq, "v_seq"),
                                _dev(o_seq, "o_seq"), _dev(do_seq, "do_seq"), _dev(lse, "lse"),
                                _pos_ptr(position_ids, N), _dev(dq_seq, "dq_seq"), _dev(dk_seq, "dk_seq"),
                                _dev(dv_seq, "dv_seq"), N, Hq, Hkv, D, P, rank, chunks, scale, _dtype_code(q_seq),
                                ws.data_ptr(), wsb, _stream(q_seq.device)))
    return dq_seq, dk_seq, dv_seq


def qkv_proj_pack(x, w_qkv, Hq, Hkv, D, P, q_send=None, k_send=None, v_send=None):
    """Shard projection x [M, hidden] @ w_qkv^T into the send blocks (q_send [P, M, Hq/P, D], k_send and v_send
    [P, M, Hkv/P, D]); bf16."""
    lib = load()
    M, hidden = x.shape
    if tuple(w_qkv.shape) != ((Hq + 2 * Hkv) * D, hidden):
        raise ValueError(f"w_qkv shape {tuple(w_qkv.shape)} is not [(Hq + 2 Hkv) D, hidden]")
    opt = dict(dtype=x.dtype, device=x.device)
    if P < 1 or Hq % P or Hkv % P:
        raise ValueError(f"Hq={Hq} and Hkv={Hkv} must be multiples of P={P}")
    q_send = torch.empty((P, M, Hq // P, D), **opt) if q_send is None else q_send
    k_send = torch.empty((P, M, Hkv // P, D), **opt) if k_send is None else k_send
    v_send = torch.empty((P, M, Hkv // P, D), **opt) if v_send is None else v_send
    _check(lib.ul_qkv_proj_pack(_dev(x, "x"), _dev(w_qkv, "w_qkv"), _dev(q_send, "q_send"), _dev(k_send, "k_send"),
                                _dev(v_send, "v_send"), M, hidden, Hq, Hkv, D, P, _dtype_code(x), _stream(x.device)))
    return q_send, k_send, v_send


def out_proj(o_seq, w_o, y=None):
    """Output projection: o_seq [M, Hq*D] (or [M, Hq, D]) @ w_o^T -> y [M, hidden]; bf16."""
    lib = load()
    M = o_seq.shape[0]
    HqD = o_seq.numel() // M
    hidden = w_o.shape[0]
    if tuple(w_o.shape) != (hidden, HqD):
        raise ValueError(f"w_o shape {tuple(w_o.shape)} is not [hidden, Hq*D={HqD}]")
    y = torch.empty((M, hidden), dtype=o_seq.dtype, device=o_seq.device) if y is None else y
    _check(lib.ul_out_proj(_dev(o_seq, "o_seq"), _dev(w_o, "w_o"), _dev(y, "y"), M, hidden, HqD, _dtype_code(o_seq),
                           _stream(o_seq.device)))
    return y


IGNORE_INDEX = -100


def _i32(t, name, n=None):
    if t.dtype != torch.int32 or (n is not None and t.numel() != n):
        raise ValueError(f"{name} must be int32" + (f" with {n} elements" if n is not None else ""))
    return _dev(t, name)


def shift_labels(labels, position_ids=None, ignore_index=IGNORE_INDEX, out=None):
    """Next-token targets [N] int32 of the whole packed sequence (run before sharding)."""
    lib = load()
    N = labels.numel()
    out = torch.empty(N, dtype=torch.int32, device=labels.device) if out is None else out
    pptr = None if position_ids is None else _i32(position_ids, "position_ids", N)
    _check(lib.ul_shift_labels(_i32(labels, "labels"), pptr, _i32(out, "out", N), N, ignore_index,
                               _stream(labels.device)))
    return out


def ce_count(labels, ignore_index=IGNORE_INDEX, count=None):
    """Number of valid targets of a shard, as a device int64 tensor [1]."""
    lib = load()
    count = torch.empty(1, dtype=torch.int64, device=labels.device) if count is None else count
    _check(lib.ul_ce_count(_i32(labels, "labels"), labels.numel(), ignore_index, _dev(count, "count"),
                           _stream(labels.device)))
    return count


def loss_combine(counts, loss_sums=None, total_count=None, loss=None):
    """Token-weighted combination of P ranks' partials: (total_count int64 [1], loss float64 [1] or None)."""
    lib = load()
    P = counts.numel()
    if counts.dtype != torch.int64 or (loss_sums is not None and (loss_sums.dtype != torch.float64
                                                                  or loss_sums.numel() != P)):
        raise ValueError("counts must be int64 [P] and loss_sums float64 [P]")
    dev = counts.device
    total_count = torch.empty(1, dtype=torch.int64, device=dev) if total_count is None else total_count
    if loss_sums is not None and loss is None:
        loss = torch.empty(1, dtype=torch.float64, device=dev)
    _check(lib.ul_loss_combine(None if loss_sums is None else _dev(loss_sums, "loss_sums"), _dev(counts, "counts"), P,
                               _dev(total_count, "total_count"), None if loss is None else _dev(loss, "loss"),
                               _stream(dev)))
    return total_count, loss


def cross_entropy(logits, labels, total_count=None, dloss=1.0, ignore_index=IGNORE_INDEX, grad=False,
                  in_place=False, loss_tok=None, loss_sum=None, dlogits=None):
    """Per-token cross entropy of one shard's logits [T, V] (bf16 or fp32) against int32 targets [T].

    Returns (loss_tok float32 [T], loss_sum float64 [1], dlogits or None).  With grad=True, dlogits is the
    gradient of dloss * (token-weighted loss) for the global valid count total_count (device int64 [1]);
    in_place=True writes it over the logits."""
    lib = load()
    T, V = logits.shape
    dev = logits.device
    loss_tok = torch.empty(T, dtype=torch.float32, device=dev) if loss_tok is None else loss_tok
    loss_sum = torch.empty(1, dtype=torch.float64, device=dev) if loss_sum is None else loss_sum
    gptr = tcp = None
    if grad:
        if total_count is None:
            raise ValueError("grad=True needs total_count")
        if in_place:
            dlogits = logits
        elif dlogits is None:
            dlogits = torch.empty_like(logits)
        gptr = _dev(dlogits, "dlogits")
        tcp = _dev(total_count, "total_count")
    else:
        dlogits = None
    _check(lib.ul_cross_entropy(_dev(logits, "logits"), _i32(labels, "labels", T), _dev(loss_tok, "loss_tok"),
                                _dev(loss_sum, "loss_sum"), gptr, tcp, float(dloss), T, V, ignore_index,
                                _dtype_code(logits), _stream(dev)))
    return loss_tok, loss_sum, dlogits
