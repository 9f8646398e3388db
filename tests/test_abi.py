"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before enqueueing anything (the
pointers below are never dereferenced because every call fails a check first).
"""

import ctypes
import os
import re

import pytest

import ulysses_sequence_parallelism_ul_amd as ul

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ul.h")

# fake, 256-byte aligned, never dereferenced
A, B, C, D_, E, F, G_, H_, I_, J = (0x10000000 * (i + 1) for i in range(10))


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ul_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ul.load()
    syms = declared_symbols()
    assert len(syms) >= 9
    for s in syms:
        assert hasattr(lib, s), s
        assert s in ul.SIGNATURES, s
    assert set(ul.SIGNATURES) == set(syms)


def test_version_and_clean_error():
    assert "gfx950" in ul.version()


def _err():
    return ul.load().ul_last_error().decode()


def test_relayout_rejections():
    lib = ul.load()
    P = ctypes.c_void_p
    # N % P
    assert lib.ul_seq_to_head(A, B, 10, 8, 64, 4, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    assert "divisible" in _err()
    # H % P
    assert lib.ul_seq_to_head(A, B, 16, 6, 64, 4, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    # rank out of range
    assert lib.ul_head_to_seq(A, B, 16, 8, 64, 4, 4, ul.UL_BF16, None) == ul.UL_ERR_ARG
    assert lib.ul_head_to_seq(A, B, 16, 8, 64, 4, -1, ul.UL_BF16, None) == ul.UL_ERR_ARG
    # null and misaligned pointers
    assert lib.ul_seq_to_head(None, B, 16, 8, 64, 4, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    assert lib.ul_seq_to_head(A + 2, B, 16, 8, 64, 4, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    # overlapping buffers
    assert lib.ul_seq_to_head(A, A + 256, 16, 8, 64, 4, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    assert "overlap" in _err()
    # N < 1, P < 1, bad dtype
    assert lib.ul_seq_to_head(A, B, 0, 8, 64, 4, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    assert lib.ul_seq_to_head(A, B, 16, 8, 64, 0, 0, ul.UL_BF16, None) == ul.UL_ERR_ARG
    assert lib.ul_seq_to_head(A, B, 16, 8, 64, 4, 0, 7, None) == ul.UL_ERR_UNSUPPORTED


def test_doc_bounds_rejections():
    lib = ul.load()
    assert lib.ul_doc_bounds_workspace_bytes(1) == 8
    assert lib.ul_doc_bounds_workspace_bytes(1025) == 16
    assert lib.ul_doc_bounds(A, B, C, 0, D_, 8, None) == ul.UL_ERR_ARG
    assert lib.ul_doc_bounds(A, None, C, 16, D_, 8, None) == ul.UL_ERR_ARG
    assert lib.ul_doc_bounds(A, B, C, 16, D_, 4, None) == ul.UL_ERR_ARG  # workspace too small
    assert lib.ul_doc_bounds(A + 2, B, C, 16, D_, 8, None) == ul.UL_ERR_ARG  # misaligned ids
    assert lib.ul_doc_bounds(A, A, C, 16, D_, 8, None) == ul.UL_ERR_ARG  # ids overlap output


def test_workspace_is_linear_in_n():
    lib = ul.load()
    for dt, n in ((ul.UL_BF16, 1 << 16), (ul.UL_F32, 1 << 15)):
        for bwd in (0, 1):
            w1 = lib.ul_attn_workspace_bytes(n, 4, 1, 128, dt, bwd)
            w2 = lib.ul_attn_workspace_bytes(2 * n, 4, 1, 128, dt, bwd)
            assert w1 > 0 and abs(w2 - 2 * w1) <= 4096
    # rejected shapes report 0
    assert lib.ul_attn_workspace_bytes(1024, 6, 4, 128, ul.UL_BF16, 0) == 0
    assert lib.ul_attn_workspace_bytes(1024, 4, 1, 96, ul.UL_BF16, 0) == 0
    assert lib.ul_attn_workspace_bytes(0, 4, 1, 128, ul.UL_BF16, 0) == 0


def _fwd(lib, N=64, Hq=4, Hkv=1, D=128, scale=0.1, dt=ul.UL_BF16, ws=F, wsb=1 << 30, q=A, o=D_, pos=None):
    return lib.ul_attn_fwd(q, B, C, pos, o, E, N, Hq, Hkv, D, scale, dt, ws, wsb, None)


def test_attn_fwd_rejections():
    lib = ul.load()
    assert _fwd(lib, Hq=6, Hkv=4) == ul.UL_ERR_ARG
    assert "multiple" in _err()
    assert _fwd(lib, D=96) == ul.UL_ERR_UNSUPPORTED
    assert _fwd(lib, Hq=12, Hkv=4) == ul.UL_ERR_UNSUPPORTED  # bf16 group of 3
    assert _fwd(lib, Hq=64, Hkv=2) == ul.UL_ERR_UNSUPPORTED  # bf16 group of 32
    assert _fwd(lib, N=0) == ul.UL_ERR_ARG
    assert _fwd(lib, scale=0.0) == ul.UL_ERR_ARG
    assert _fwd(lib, scale=float("nan")) == ul.UL_ERR_ARG
    assert _fwd(lib, wsb=100) == ul.UL_ERR_ARG
    assert "workspace" in _err()
    assert _fwd(lib, q=None) == ul.UL_ERR_ARG
    assert _fwd(lib, q=A + 8) == ul.UL_ERR_ARG
    assert _fwd(lib, o=A) == ul.UL_ERR_ARG  # output aliases q
    assert _fwd(lib, pos=G_ + 2) == ul.UL_ERR_ARG
    assert _fwd(lib, dt=5) == ul.UL_ERR_UNSUPPORTED


def test_attn_bwd_rejections():
    lib = ul.load()

    def bwd(N=64, Hq=4, Hkv=1, D=128, wsb=1 << 30, dq=G_, dk=H_):
        return lib.ul_attn_bwd(A, B, C, D_, E, F, None, dq, dk, I_, N, Hq, Hkv, D, 0.1, ul.UL_BF16, J, wsb, None)

    assert bwd(Hq=5, Hkv=2) == ul.UL_ERR_ARG
    assert bwd(D=32) == ul.UL_ERR_UNSUPPORTED
    assert bwd(wsb=16) == ul.UL_ERR_ARG
    assert bwd(dq=None) == ul.UL_ERR_ARG
    assert bwd(dk=G_) == ul.UL_ERR_ARG  # dk overlaps dq


def test_rank_workspace_and_rejections():
    lib = ul.load()
    # valid: the million-token training share at 1, 2 and 4 head chunks; linear in N
    for chunks in (1, 2, 4):
        for bwd in (0, 1):
            w1 = lib.ul_rank_workspace_bytes(1 << 16, 32, 8, 128, 8, chunks, ul.UL_BF16, bwd)
            w2 = lib.ul_rank_workspace_bytes(1 << 17, 32, 8, 128, 8, chunks, ul.UL_BF16, bwd)
            assert w1 > 0 and abs(w2 - 2 * w1) <= 8192
    # fewer heads per chunk, smaller workspace
    assert (lib.ul_rank_workspace_bytes(1 << 16, 32, 8, 128, 8, 4, ul.UL_BF16, 0)
            < lib.ul_rank_workspace_bytes(1 << 16, 32, 8, 128, 8, 1, ul.UL_BF16, 0))
    bad = [
        (1024, 32, 8, 128, 8, 3),    # 3 chunks do not divide 4 query heads
        (1024, 24, 6, 128, 2, 2),    # 6 query heads per chunk vs groups of 4: neither divides
        (1024, 32, 4, 128, 8, 1),    # 4 KV heads over 8 ranks (replication)
        (1020, 32, 8, 128, 8, 1),    # N not a multiple of P
        (1024, 32, 8, 96, 8, 1),     # head dim
        (1024, 32, 8, 128, 0, 1),    # P
        (1024, 32, 8, 128, 8, 0),    # chunks
    ]
    for N, Hq, Hkv, D, P, chunks in bad:
        assert lib.ul_rank_workspace_bytes(N, Hq, Hkv, D, P, chunks, ul.UL_F32, 0) == 0, (Hq, Hkv, P, chunks)

    def fwd(N=64, Hq=32, Hkv=8, P=8, rank=0, chunks=1, wsb=1 << 30, q=A, o=D_, lse=E):
        return lib.ul_rank_attn_fwd(q, B, C, None, o, lse, N, Hq, Hkv, 128, P, rank, chunks, 0.1, ul.UL_BF16, F, wsb,
                                    None)

    assert fwd(chunks=3) == ul.UL_ERR_ARG and "chunks" in _err()
    assert fwd(rank=8) == ul.UL_ERR_ARG and "rank" in _err()
    assert fwd(N=60) == ul.UL_ERR_ARG
    assert fwd(wsb=1024) == ul.UL_ERR_ARG and "workspace" in _err()
    assert fwd(q=None) == ul.UL_ERR_ARG
    assert fwd(o=A) == ul.UL_ERR_ARG  # output overlaps q_seq
    assert fwd(lse=A + 8) == ul.UL_ERR_ARG

    def bwd(chunks=1, dq=G_, dk=H_, wsb=1 << 30):
        return lib.ul_rank_attn_bwd(A, B, C, D_, E, F, None, dq, dk, I_, 64, 32, 8, 128, 8, 0, chunks, 0.1,
                                    ul.UL_BF16, J, wsb, None)

    assert bwd(chunks=8) == ul.UL_ERR_ARG
    assert bwd(dk=G_) == ul.UL_ERR_ARG  # dk overlaps dq
    assert bwd(wsb=64) == ul.UL_ERR_ARG


def test_projection_rejections_cpu():
    lib = ul.load()

    def qkv(M=16, hidden=128, Hq=4, Hkv=2, D=64, P=2, dt=ul.UL_BF16, x=A, q=C):
        return lib.ul_qkv_proj_pack(x, B, q, D_, E, M, hidden, Hq, Hkv, D, P, dt, None)

    assert qkv(hidden=100) == ul.UL_ERR_ARG
    assert qkv(hidden=(1 << 22) + 64) == ul.UL_ERR_ARG   # above the 2^22 limit
    assert qkv(Hkv=3) == ul.UL_ERR_ARG      # not a multiple of P
    assert qkv(M=0) == ul.UL_ERR_ARG
    assert qkv(dt=ul.UL_F32) == ul.UL_ERR_UNSUPPORTED
    assert qkv(x=None) == ul.UL_ERR_ARG
    assert qkv(q=A) == ul.UL_ERR_ARG        # q_send overlaps x
    assert lib.ul_out_proj(A, B, C, 16, 64, 96, ul.UL_BF16, None) == ul.UL_ERR_ARG   # HqD % 64
    assert lib.ul_out_proj(A, B, C, 16, 64, (1 << 22) + 64, ul.UL_BF16, None) == ul.UL_ERR_ARG  # above 2^22
    assert lib.ul_out_proj(A, B, A, 16, 64, 128, ul.UL_BF16, None) == ul.UL_ERR_ARG  # y overlaps o_seq
    assert lib.ul_out_proj(A, B, C, 16, 64, 128, ul.UL_F32, None) == ul.UL_ERR_UNSUPPORTED


def test_loss_rejections_cpu():
    lib = ul.load()
    ign = ul.IGNORE_INDEX
    # shift labels: N, NULL, overlap, alignment
    assert lib.ul_shift_labels(A, None, B, 0, ign, None) == ul.UL_ERR_ARG
    assert lib.ul_shift_labels(None, None, B, 16, ign, None) == ul.UL_ERR_ARG
    assert lib.ul_shift_labels(A, None, A + 8, 16, ign, None) == ul.UL_ERR_ARG     # out overlaps labels
    assert lib.ul_shift_labels(A, C, C, 16, ign, None) == ul.UL_ERR_ARG            # out overlaps position_ids
    assert lib.ul_shift_labels(A, None, B + 2, 16, ign, None) == ul.UL_ERR_ARG     # misaligned
    # counts
    assert lib.ul_ce_count(A, 0, ign, B, None) == ul.UL_ERR_ARG
    assert lib.ul_ce_count(A, 16, ign, A + 8, None) == ul.UL_ERR_ARG              # count overlaps labels
    assert lib.ul_ce_count(A, 16, ign, B + 4, None) == ul.UL_ERR_ARG              # count misaligned
    # combine
    assert lib.ul_loss_combine(A, B, 0, C, D_, None) == ul.UL_ERR_ARG
    assert lib.ul_loss_combine(A, None, 4, C, D_, None) == ul.UL_ERR_ARG
    assert lib.ul_loss_combine(A, B, 4, None, None, None) == ul.UL_ERR_ARG          # nothing to write
    assert lib.ul_loss_combine(None, B, 4, C, D_, None) == ul.UL_ERR_ARG            # loss needs loss_sums
    assert lib.ul_loss_combine(A, B, 4, B + 8, D_, None) == ul.UL_ERR_ARG           # output overlaps counts
    assert lib.ul_loss_combine(A, B, 4, C, C, None) == ul.UL_ERR_ARG                # outputs overlap

    # cross entropy
    def ce(logits=A, labels=B, lt=C, ls=D_, dl=None, tc=None, dloss=1.0, T=8, V=64, dt=ul.UL_BF16):
        return lib.ul_cross_entropy(logits, labels, lt, ls, dl, tc, dloss, T, V, ign, dt, None)

    assert ce(V=60) == ul.UL_ERR_UNSUPPORTED                  # 120-byte rows
    assert ce(V=62, dt=ul.UL_F32) == ul.UL_ERR_UNSUPPORTED    # 248-byte rows
    assert ce(dt=7) == ul.UL_ERR_UNSUPPORTED
    assert ce(T=0) == ul.UL_ERR_ARG
    assert ce(T=1 << 31) == ul.UL_ERR_ARG
    assert ce(V=0) == ul.UL_ERR_ARG
    assert ce(logits=A + 8) == ul.UL_ERR_ARG                   # logits misaligned
    assert ce(ls=D_ + 4) == ul.UL_ERR_ARG                      # loss_sum misaligned
    assert ce(lt=None) == ul.UL_ERR_ARG
    assert ce(lt=A + 16) == ul.UL_ERR_ARG                      # loss_tok overlaps logits
    assert ce(ls=C + 8) == ul.UL_ERR_ARG                       # loss_sum overlaps loss_tok
    assert ce(dl=E) == ul.UL_ERR_ARG                           # gradient without total_count
    assert ce(dl=A + 16, tc=F) == ul.UL_ERR_ARG                # partial overlap with logits
    assert ce(dl=E, tc=F, dloss=float("inf")) == ul.UL_ERR_ARG
    assert ce(dl=E, tc=E + 64) == ul.UL_ERR_ARG                # total_count inside dlogits
    assert ce(dl=C, tc=F) == ul.UL_ERR_ARG                     # dlogits overlaps loss_tok


UL_F32_MAX_N = 65536  # include/ul.h


def test_header_states_the_fp32_limit():
    text = open(HEADER).read()
    assert re.search(r"#define\s+UL_F32_MAX_N\s+%d\b" % UL_F32_MAX_N, text)


def test_fp32_attention_refuses_large_n_before_enqueueing():
    """The fp32 kernels visit keys one after another per query row; a large N
    is refused up front (pointers are fake: a refusal enqueues nothing)."""
    lib = ul.load()
    big = UL_F32_MAX_N + 64
    assert lib.ul_attn_workspace_bytes(UL_F32_MAX_N, 8, 8, 64, ul.UL_F32, 0) > 0
    assert lib.ul_attn_workspace_bytes(big, 8, 8, 64, ul.UL_F32, 0) == 0
    assert lib.ul_attn_workspace_bytes(big, 8, 8, 64, ul.UL_BF16, 0) > 0
    assert _fwd(lib, N=big, dt=ul.UL_F32) == ul.UL_ERR_UNSUPPORTED
    assert "fp32" in _err() and str(UL_F32_MAX_N) in _err()
    assert lib.ul_attn_bwd(A, B, C, D_, E, F, None, G_, H_, I_, big, 4, 1, 128, 0.1, ul.UL_F32, J, 1 << 40,
                           None) == ul.UL_ERR_UNSUPPORTED
    big_r = 8 * (UL_F32_MAX_N // 8 + 8)
    assert lib.ul_rank_attn_fwd(A, B, C, None, D_, E, big_r, 32, 8, 128, 8, 0, 1, 0.1, ul.UL_F32, F, 1 << 40,
                                None) == ul.UL_ERR_UNSUPPORTED
    assert lib.ul_rank_attn_bwd(A, B, C, D_, E, F, None, G_, H_, I_, big_r, 32, 8, 128, 8, 0, 1, 0.1, ul.UL_F32,
                                J, 1 << 40, None) == ul.UL_ERR_UNSUPPORTED
    assert lib.ul_rank_workspace_bytes(big_r, 32, 8, 128, 8, 1, ul.UL_F32, 1) == 0


def test_position_ids_may_not_alias_outputs_or_workspace():
    """The document-bounds kernels read position_ids while writing the
    workspace; an alias with the workspace or an output is refused."""
    lib = ul.load()
    N = 64
    # forward: workspace F, outputs o = D_, lse = E
    for pos, what in ((F, "ws"), (F + 128, "ws"), (D_, "o"), (E + 64, "lse")):
        assert _fwd(lib, pos=pos) == ul.UL_ERR_ARG, what
        assert "position_ids" in _err() and what in _err()
    assert _fwd(lib, pos=A) != ul.UL_ERR_ARG or "position_ids" not in _err()  # reading an input is fine

    def bwd(pos):
        return lib.ul_attn_bwd(A, B, C, D_, E, F, pos, G_, H_, I_, N, 4, 1, 128, 0.1, ul.UL_BF16, J, 1 << 30, None)

    for pos, what in ((J, "ws"), (G_ + 256, "dq"), (H_, "dk"), (I_ + 4, "dv")):
        assert bwd(pos) == ul.UL_ERR_ARG, what
        assert "position_ids" in _err() and what in _err()

    def rfwd(pos):
        return lib.ul_rank_attn_fwd(A, B, C, pos, D_, E, N, 32, 8, 128, 8, 0, 1, 0.1, ul.UL_BF16, F, 1 << 30, None)

    for pos, what in ((F, "ws"), (D_ + 16, "o_seq"), (E, "lse")):
        assert rfwd(pos) == ul.UL_ERR_ARG, what
        assert "position_ids" in _err() and what in _err()

    def rbwd(pos):
        return lib.ul_rank_attn_bwd(A, B, C, D_, E, F, pos, G_, H_, I_, N, 32, 8, 128, 8, 0, 1, 0.1, ul.UL_BF16,
                                    J, 1 << 30, None)

    for pos, what in ((J + 512, "ws"), (G_, "dq_seq"), (H_, "dk_seq"), (I_, "dv_seq")):
        assert rbwd(pos) == ul.UL_ERR_ARG, what
        assert "position_ids" in _err() and what in _err()
