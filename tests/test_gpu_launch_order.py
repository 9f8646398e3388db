"""The launch order of the bf16 attention work-groups (heaviest first).

The order does not change any output (each work-group writes only its own
rows); these tests check the order itself.  The attention workspace ends with
the order of the query-column blocks (forward, dQ) and, for the backward, the
order of the key blocks (dK/dV), each int32 and padded to 256 bytes.  A unit's
work is the number of tiles its loop visits; units are bucketed into 2048
equal-width work buckets (width (max work + 1) / 2048), heaviest bucket first,
and within a bucket kept in the order in which work grows inside a document:
key blocks ascending, column blocks descending.
"""

import numpy as np
import pytest
import torch

import synth
import ulysses_sequence_parallelism_ul_amd as ul
from gpu_helpers import log, require_gpu

pytestmark = pytest.mark.gpu

COL_BLOCK, KEY_TILE, KEY_BLOCK, COL_TILE, BUCKETS = 256, 64, 128, 64, 2048


def _pad(n):
    return (n * 4 + 255) // 256 * 256


def _bounds(pos):
    N = len(pos)
    starts = np.flatnonzero((np.asarray(pos) == 0) | (np.arange(N) == 0))
    lengths = np.diff(np.r_[starts, N])
    return np.repeat(starts, lengths), np.repeat(np.r_[starts[1:], N] - 1, lengths)


def _expected(work, ascending):
    b = np.minimum(work.astype(np.int64) * BUCKETS // (work.max() + 1), BUCKETS - 1)
    idx = np.arange(len(work))
    tie = idx if ascending else -idx
    return np.lexsort((tie, -b))


def _key_work(doc_end, N, G):
    k0 = np.arange((N + KEY_BLOCK - 1) // KEY_BLOCK, dtype=np.int64) * KEY_BLOCK
    kl = np.minimum(N - 1, k0 + KEY_BLOCK - 1)
    return ((doc_end[kl] + 1) * G - 1) // COL_TILE - (k0 * G) // COL_TILE + 1


def _col_work(doc_start, N, G):
    c0 = np.arange((N * G + COL_BLOCK - 1) // COL_BLOCK, dtype=np.int64) * COL_BLOCK
    rf = c0 // G
    rl = np.minimum(N - 1, (c0 + COL_BLOCK - 1) // G)
    return rl // KEY_TILE - doc_start[rf] // KEY_TILE + 1


@pytest.mark.parametrize("case", ["one_document", "train_packed", "random", "lone_tokens", "small", "one_token"])
def test_orders_are_heaviest_first_permutations(case):
    require_gpu()
    Hq, Hkv, D = 4, 1, 128
    G = Hq // Hkv
    if case == "train_packed":
        pos = synth.workload_positions("train_packed")
    elif case == "random":
        pos = synth.random_positions(50_000, 5, max_docs=40)
    elif case == "lone_tokens":
        pos = np.zeros(3000, dtype=np.int32)
    elif case == "small":  # fewer units than waves in the order kernel
        pos = synth.random_positions(1000, 3, max_docs=4)
    elif case == "one_token":
        pos = np.zeros(1, dtype=np.int32)
    else:
        pos = np.arange(70_000, dtype=np.int32)
    N = len(pos)
    log(f"launch order {case} N={N}")
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(N)
    q = torch.randn((N, Hq, D), device=dev, generator=g).to(torch.bfloat16)
    k = torch.randn((N, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    v = torch.randn((N, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    pd = torch.from_numpy(np.asarray(pos, dtype=np.int32)).to(dev)
    total = ul.attn_workspace_bytes(N, Hq, Hkv, D, torch.bfloat16, True)
    ws = torch.full((total,), 0xFF, dtype=torch.uint8, device=dev)
    o, lse = ul.attn_fwd(q, k, v, pd)
    ul.attn_bwd(q, k, v, o, o, lse, pd, workspace=ws)
    torch.cuda.synchronize()
    nkb = (N + KEY_BLOCK - 1) // KEY_BLOCK
    ncb = (N * G + COL_BLOCK - 1) // COL_BLOCK
    host = ws.cpu().numpy()
    key_at = total - _pad(nkb)
    col_at = key_at - _pad(ncb)
    order_key = host[key_at:key_at + 4 * nkb].view(np.int32)
    order_col = host[col_at:col_at + 4 * ncb].view(np.int32)
    assert np.array_equal(np.sort(order_key), np.arange(nkb))
    assert np.array_equal(np.sort(order_col), np.arange(ncb))
    doc_start, doc_end = _bounds(pos)
    assert np.array_equal(order_key, _expected(_key_work(doc_end, N, G), True))
    assert np.array_equal(order_col, _expected(_col_work(doc_start, N, G), False))
    if case == "one_document":
        # work grows with the column block and shrinks with the key block
        assert np.array_equal(order_key, np.arange(nkb))
        assert np.array_equal(order_col, np.arange(ncb)[::-1])
