"""Pins of the oracle's backward attention (CPU only).

Pinned by central finite differences of L = sum(dO * O), by a library
autograd routine (torch CPU float64 SDPA) on single documents, by closed
forms (Q = 0), and by invariants: softmax-gradient rows sum to zero (so
per-document sums of dK vanish), per-document sums of dV equal those of dO,
the first row of each document gets dQ = 0, grouped-query equals replicated
multi-head with group sums, packing equals separate documents, and the per-
rank computation equals the unsharded one.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _rand(shape, seed, scale=1.0):
    return scale * np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _loss(q, k, v, do, pos, sc):
    o, _ = oracle.attn_fwd(q, k, v, pos, sc)
    return float((o * do).sum())


@pytest.mark.parametrize("Hq,Hkv,seed", [(2, 1, 0), (2, 2, 1), (4, 2, 2)])
def test_finite_differences(Hq, Hkv, seed):
    N, D, sc = 10, 3, 0.45
    q, k, v = _rand((N, Hq, D), seed), _rand((N, Hkv, D), seed + 1), _rand((N, Hkv, D), seed + 2)
    do = _rand((N, Hq, D), seed + 3)
    pos = synth.position_ids_from_lengths([4, 1, 5])
    r = oracle.attn_bwd(q, k, v, do, pos, sc, block=3)
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp = x.copy()
            xm = x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name[1]] = xp
            args_m[name[1]] = xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], do, pos, sc)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], do, pos, sc)) / (2 * eps)
        err = np.abs(num - r[name]).max() / max(1.0, np.abs(num).max())
        assert err < 1e-6, (name, err)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1)])
def test_single_document_matches_torch_autograd(Hq, Hkv):
    N, D = 70, 8
    q, k, v = _rand((N, Hq, D), 40), _rand((N, Hkv, D), 41), _rand((N, Hkv, D), 42)
    do = _rand((N, Hq, D), 43)
    r = oracle.attn_bwd(q, k, v, do, block=25)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2).clone().requires_grad_()
    tk = torch.from_numpy(k).permute(1, 0, 2).clone().requires_grad_()
    tv = torch.from_numpy(v).permute(1, 0, 2).clone().requires_grad_()
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=0), tv.repeat_interleave(G, dim=0), is_causal=True)
    o.backward(torch.from_numpy(do).permute(1, 0, 2))
    np.testing.assert_allclose(r["dq"], tq.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["dk"], tk.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["dv"], tv.grad.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-11)


def _case(seed=50):
    N, Hq, Hkv, D = 90, 4, 2, 6
    lengths = [1, 30, 2, 40, 17]
    return (_rand((N, Hq, D), seed), _rand((N, Hkv, D), seed + 1), _rand((N, Hkv, D), seed + 2),
            _rand((N, Hq, D), seed + 3), synth.position_ids_from_lengths(lengths), lengths)


def test_delta_two_routes_agree():
    q, k, v, do, pos, _ = _case()
    r = oracle.attn_bwd(q, k, v, do, pos)
    np.testing.assert_allclose(r["delta"], (r["o"] * do).sum(axis=2).T, rtol=1e-12, atol=1e-12)


def test_per_document_gradient_sums():
    q, k, v, do, pos, lengths = _case()
    r = oracle.attn_bwd(q, k, v, do, pos)
    G = q.shape[1] // k.shape[1]
    s = 0
    for L in lengths:
        dk_sum = r["dk"][s:s + L].sum(axis=0)
        np.testing.assert_allclose(dk_sum, 0.0, rtol=0, atol=1e-12)
        dv_sum = r["dv"][s:s + L].sum(axis=0)
        do_sum = do[s:s + L].sum(axis=0).reshape(k.shape[1], G, -1).sum(axis=1)
        np.testing.assert_allclose(dv_sum, do_sum, rtol=1e-12, atol=1e-12)
        assert np.all(r["dq"][s] == 0)
        s += L


def test_zero_queries_closed_forms():
    q, k, v, do, pos, _ = _case(60)
    q = np.zeros_like(q)
    sc = 1.0 / math.sqrt(q.shape[2])
    r = oracle.attn_bwd(q, k, v, do, pos)
    start, end = oracle.doc_bounds(pos)
    N, Hq, D = q.shape
    G = Hq // k.shape[1]
    np.testing.assert_allclose(r["dk"], 0.0, rtol=0, atol=1e-14)
    for j in range(N):
        for g in range(k.shape[1]):
            expect = sum(do[i, h] / (i - start[i] + 1) for h in range(g * G, (g + 1) * G)
                         for i in range(j, end[j] + 1))
            np.testing.assert_allclose(r["dv"][j, g], expect, rtol=1e-12, atol=1e-12)
    for i in range(N):
        s = start[i]
        n = i - s + 1
        for h in range(Hq):
            g = h // G
            kk, vv = k[s:i + 1, g], v[s:i + 1, g]
            dlt = do[i, h] @ vv.mean(axis=0)
            expect = (sc / n) * (do[i, h] @ (vv.T @ kk) - dlt * kk.sum(axis=0))
            np.testing.assert_allclose(r["dq"][i, h], expect, rtol=1e-11, atol=1e-12)


def test_gqa_equals_mha_replicated_then_group_summed():
    q, k, v, do, pos, _ = _case(70)
    G = q.shape[1] // k.shape[1]
    a = oracle.attn_bwd(q, k, v, do, pos)
    b = oracle.attn_bwd(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), do, pos)
    np.testing.assert_allclose(a["dq"], b["dq"], rtol=1e-12, atol=1e-12)
    N, _, D = k.shape
    np.testing.assert_allclose(a["dk"], b["dk"].reshape(N, -1, G, D).sum(axis=2), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["dv"], b["dv"].reshape(N, -1, G, D).sum(axis=2), rtol=1e-12, atol=1e-12)


def test_packed_backward_equals_documents_run_separately():
    q, k, v, do, pos, lengths = _case(80)
    a = oracle.attn_bwd(q, k, v, do, pos, block=16)
    s = 0
    for L in lengths:
        b = oracle.attn_bwd(q[s:s + L], k[s:s + L], v[s:s + L], do[s:s + L])
        for name in ("dq", "dk", "dv"):
            np.testing.assert_allclose(a[name][s:s + L], b[name], rtol=1e-12, atol=1e-12)
        s += L
    c = oracle.attn_bwd_per_document(q, k, v, do, pos)
    for name in ("dq", "dk", "dv", "o", "lse", "delta"):
        np.testing.assert_allclose(a[name], c[name], rtol=1e-12, atol=1e-12)


def test_per_rank_backward_equals_unsharded():
    P = 2
    q, k, v, do, pos, _ = _case(90)
    full = oracle.attn_bwd(q, k, v, do, pos)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(P):
        rr = oracle.attn_bwd(*(oracle.seq_to_head(x, P, r) for x in (q, k, v, do)), pos)
        dq = oracle.head_to_seq(rr["dq"], dq, P, r)
        dk = oracle.head_to_seq(rr["dk"], dk, P, r)
        dv = oracle.head_to_seq(rr["dv"], dv, P, r)
    for name, x in (("dq", dq), ("dk", dk), ("dv", dv)):
        np.testing.assert_allclose(x, full[name], rtol=1e-12, atol=1e-12)


def test_sampled_row_gradients_equal_full():
    q, k, v, do, pos, lengths = _case(100)
    full = oracle.attn_bwd(q, k, v, do, pos)
    rows = [0, 1, 2, 30, 31, 33, 60, 72, 88, 89]
    r, dq, dlt = oracle.attn_bwd_dq_rows(q, k, v, do, pos, rows, batch=4)
    np.testing.assert_allclose(dq, full["dq"][rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dlt, full["delta"][:, rows], rtol=1e-12, atol=1e-12)
    kv_rows = [0, 29, 30, 32, 70, 73, 80, 89]
    r, dk, dv = oracle.attn_bwd_dkdv_rows(q, k, v, do, pos, kv_rows, batch=5)
    np.testing.assert_allclose(dk, full["dk"][kv_rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dv, full["dv"][kv_rows], rtol=1e-12, atol=1e-12)
    o, lse = oracle.attn_fwd_per_document(q, k, v, pos)
    np.testing.assert_allclose(o, full["o"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, full["lse"], rtol=1e-12, atol=1e-12)
