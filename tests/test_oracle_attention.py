"""Pins of the oracle's forward attention (CPU only).

Nothing on the pages prints a numeric result, so the oracle is pinned by:
brute-force scalar loops, a hand-derived worked example (tests/golden),
closed forms (Q = 0, first row of a document, constant V), invariants the
pages fix (heads independent -> sharded equals unsharded; packing equals
documents run separately; softmax rows sum to 1), and a library routine
(torch CPU scaled_dot_product_attention in float64) on single documents.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return scale * np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


def _brute_fwd(q, k, v, pos, scale):
    """Scalar loops straight from the definition (tiny N only)."""
    N, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    # document of each token by walking from the start
    doc = []
    d = 0
    for t in range(N):
        if t > 0 and pos[t] == 0:
            d += 1
        doc.append(d)
    o = np.zeros((N, Hq, D))
    lse = np.zeros((Hq, N))
    for h in range(Hq):
        g = h // G
        for i in range(N):
            js = [j for j in range(N) if j <= i and doc[j] == doc[i]]
            logits = [scale * sum(q[i, h, x] * k[j, g, x] for x in range(D)) for j in js]
            mx = max(logits)
            w = [math.exp(s - mx) for s in logits]
            tot = sum(w)
            for x in range(D):
                o[i, h, x] = sum(w[a] * v[js[a], g, x] for a in range(len(js))) / tot
            lse[h, i] = mx + math.log(tot)
    return o, lse


@pytest.mark.parametrize("N,Hq,Hkv,D,seed", [(1, 1, 1, 3, 0), (7, 2, 1, 4, 1), (13, 4, 2, 3, 2), (24, 4, 1, 5, 3)])
def test_forward_matches_brute_force(N, Hq, Hkv, D, seed):
    q, k, v = _rand((N, Hq, D), seed), _rand((N, Hkv, D), seed + 10), _rand((N, Hkv, D), seed + 20)
    pos = synth.random_positions(N, seed)
    sc = 0.37
    o, lse = oracle.attn_fwd(q, k, v, pos, sc, block=5)
    bo, bl = _brute_fwd(q, k, v, pos, sc)
    np.testing.assert_allclose(o, bo, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def _golden_value(x):
    if isinstance(x, str):
        sign = -1.0 if x.startswith("-") else 1.0
        body = x.lstrip("-")
        coef, _, fn = body.partition("ln")
        c = float(coef) if coef else 1.0
        return sign * c * math.log(float(fn))
    return float(x)


@pytest.mark.parametrize("case", ["one_document", "two_documents"])
def test_golden_two_tokens(case):
    with open(os.path.join(GOLDEN, "attn_two_tokens.json")) as f:
        g = json.load(f)
    c = g[case]
    q = np.array([g["q0"], math.log(3.0)]).reshape(2, 1, 1)
    k = np.array([0.0, 1.0]).reshape(2, 1, 1)
    v = np.array([4.0, 8.0]).reshape(2, 1, 1)
    do = np.ones((2, 1, 1))
    o, lse = oracle.attn_fwd(q, k, v, c["position_ids"], 1.0)
    np.testing.assert_allclose(o[:, 0, 0], [_golden_value(x) for x in c["o"]], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(lse[0], [_golden_value(x) for x in c["lse"]], rtol=1e-14, atol=1e-14)
    r = oracle.attn_bwd(q, k, v, do, c["position_ids"], 1.0)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r[name][:, 0, 0], [_golden_value(x) for x in c[name]], rtol=1e-14, atol=1e-14)


def test_packed_equals_documents_run_separately():
    N, Hq, Hkv, D = 200, 4, 2, 8
    q, k, v = _rand((N, Hq, D), 1), _rand((N, Hkv, D), 2), _rand((N, Hkv, D), 3)
    pos = synth.position_ids_from_lengths([37, 1, 64, 90, 8])
    o, lse = oracle.attn_fwd(q, k, v, pos, block=33)
    s = 0
    for L in [37, 1, 64, 90, 8]:
        od, ld = oracle.attn_fwd(q[s:s + L], k[s:s + L], v[s:s + L])
        np.testing.assert_allclose(o[s:s + L], od, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[:, s:s + L], ld, rtol=1e-12, atol=1e-12)
        s += L


@pytest.mark.parametrize("P", [1, 2, 4])
def test_sharded_per_rank_equals_unsharded(P):
    N, Hq, Hkv, D = 64, 8, 4, 6
    q, k, v = _rand((N, Hq, D), 4), _rand((N, Hkv, D), 5), _rand((N, Hkv, D), 6)
    pos = synth.random_positions(N, 9)
    o_full, lse_full = oracle.attn_fwd(q, k, v, pos)
    o_seq = np.zeros_like(q)
    for r in range(P):
        o_r, lse_r = oracle.attn_fwd(oracle.seq_to_head(q, P, r), oracle.seq_to_head(k, P, r),
                                     oracle.seq_to_head(v, P, r), pos)
        o_seq = oracle.head_to_seq(o_r, o_seq, P, r)
        np.testing.assert_allclose(lse_r, lse_full[r * Hq // P:(r + 1) * Hq // P], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o_seq, o_full, rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one_and_respect_mask():
    N, D = 40, 4
    q, k = _rand((N, 2, D), 7), _rand((N, 1, D), 8)
    pos = synth.position_ids_from_lengths([10, 25, 5])
    start, _ = oracle.doc_bounds(pos)
    for h in range(2):
        P = oracle.attn_probs(q, k, pos, head=h)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        for i in range(N):
            assert np.all(P[i, :start[i]] == 0) and np.all(P[i, i + 1:] == 0)
            assert np.all(P[i, start[i]:i + 1] > 0)


def _brute_probs(q, k, pos, scale, h, G):
    """P[i, j] of query head h from scalar loops: exp of the scaled logit over
    the sum of exp over the keys visible to i (tiny N only)."""
    N, _, D = q.shape
    doc, d = [], 0
    for t in range(N):
        if t > 0 and pos[t] == 0:
            d += 1
        doc.append(d)
    P = np.zeros((N, N))
    for i in range(N):
        js = [j for j in range(N) if j <= i and doc[j] == doc[i]]
        w = {j: math.exp(scale * sum(q[i, h, x] * k[j, h // G, x] for x in range(D))) for j in js}
        tot = sum(w.values())
        for j in js:
            P[i, j] = w[j] / tot
    return P


def test_attn_probs_values():
    """Every element of P against scalar loops, at a group size where h // G
    and h % Hkv pick different KV heads and with a non-default scale; then
    P V and the diagonal's log-probability against the forward's O and LSE
    (log P_ii = scale q_i.k_i - LSE_i)."""
    N, Hq, Hkv, D, sc = 23, 4, 2, 3, 0.37
    q, k, v = _rand((N, Hq, D), 40, 1.5), _rand((N, Hkv, D), 41, 1.5), _rand((N, Hkv, D), 42)
    pos = synth.position_ids_from_lengths([6, 1, 9, 7])
    o, lse = oracle.attn_fwd(q, k, v, pos, sc, block=5)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        P = oracle.attn_probs(q, k, pos, sc, head=h)
        np.testing.assert_allclose(P, _brute_probs(q, k, pos, sc, h, Hq // Hkv), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(P @ v[:, g, :], o[:, h, :], rtol=1e-12, atol=1e-13)
        diag = sc * np.einsum("nd,nd->n", q[:, h, :], k[:, g, :]) - np.log(np.diag(P))
        np.testing.assert_allclose(diag, lse[h], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", ["one_document", "two_documents"])
def test_attn_probs_golden_two_tokens(case):
    """The hand-derived probabilities of the two-token example: one document
    gives P_1 = [1/4, 3/4], two documents the identity."""
    with open(os.path.join(GOLDEN, "attn_two_tokens.json")) as f:
        g = json.load(f)
    q = np.array([g["q0"], math.log(3.0)]).reshape(2, 1, 1)
    k = np.array([0.0, 1.0]).reshape(2, 1, 1)
    P = oracle.attn_probs(q, k, g[case]["position_ids"], 1.0)
    np.testing.assert_allclose(P, np.array(g[case]["p"]), rtol=1e-15, atol=1e-15)


def test_first_row_of_every_document_returns_its_v_row():
    N, Hq, Hkv, D = 50, 4, 2, 5
    q, k, v = _rand((N, Hq, D), 10), _rand((N, Hkv, D), 11), _rand((N, Hkv, D), 12)
    lengths = [1, 20, 3, 26]
    pos = synth.position_ids_from_lengths(lengths)
    o, lse = oracle.attn_fwd(q, k, v, pos)
    starts = np.cumsum([0] + lengths[:-1])
    for s in starts:
        for h in range(Hq):
            g = h // 2
            assert np.array_equal(o[s, h], v[s, g])
            assert lse[h, s] == pytest.approx(np.dot(q[s, h], k[s, g]) / math.sqrt(D), rel=1e-14, abs=1e-14)


def test_zero_queries_closed_form():
    N, Hq, Hkv, D = 60, 2, 1, 3
    q = np.zeros((N, Hq, D))
    k, v = _rand((N, Hkv, D), 13), _rand((N, Hkv, D), 14)
    pos = synth.position_ids_from_lengths([17, 30, 13])
    start, _ = oracle.doc_bounds(pos)
    o, lse = oracle.attn_fwd(q, k, v, pos)
    for i in range(N):
        n = i - start[i] + 1
        for h in range(Hq):
            np.testing.assert_allclose(o[i, h], v[start[i]:i + 1, 0].mean(axis=0), rtol=1e-13, atol=1e-13)
            assert lse[h, i] == pytest.approx(math.log(n), rel=1e-14, abs=1e-14)


def test_constant_v_gives_constant_output():
    N, D = 33, 4
    q, k = _rand((N, 2, D), 15), _rand((N, 2, D), 16)
    v = np.full((N, 2, D), -2.5)
    o, _ = oracle.attn_fwd(q, k, v, synth.random_positions(N, 3))
    np.testing.assert_allclose(o, -2.5, rtol=0, atol=1e-14)


def test_large_logits_are_stable():
    N, D = 48, 8
    q, k, v = _rand((N, 1, D), 17, 30.0), _rand((N, 1, D), 18, 30.0), _rand((N, 1, D), 19)
    o, lse = oracle.attn_fwd(q, k, v)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # rows are convex combinations of V rows
    assert np.all(np.abs(o) <= np.abs(v).max() + 1e-12)


def test_scale_defaults_to_inverse_sqrt_d():
    N, D = 20, 9
    q, k, v = _rand((N, 1, D), 20), _rand((N, 1, D), 21), _rand((N, 1, D), 22)
    a, la = oracle.attn_fwd(q, k, v)
    b, lb = oracle.attn_fwd(q, k, v, None, 1.0 / 3.0)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (8, 2)])
def test_single_document_matches_torch_sdpa(Hq, Hkv):
    N, D = 96, 16
    q, k, v = _rand((N, Hq, D), 23), _rand((N, Hkv, D), 24), _rand((N, Hkv, D), 25)
    o, _ = oracle.attn_fwd(q, k, v, block=40)
    G = Hq // Hkv
    tq = torch.from_numpy(q).permute(1, 0, 2)
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, dim=0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, dim=0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_replicated_kv():
    N, Hq, Hkv, D = 30, 6, 2, 4
    q, k, v = _rand((N, Hq, D), 26), _rand((N, Hkv, D), 27), _rand((N, Hkv, D), 28)
    pos = synth.random_positions(N, 4)
    G = Hq // Hkv
    krep = np.repeat(k, G, axis=1)
    vrep = np.repeat(v, G, axis=1)
    a, la = oracle.attn_fwd(q, k, v, pos)
    b, lb = oracle.attn_fwd(q, krep, vrep, pos)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-13, atol=1e-13)
    # and head h really reads KV head h // G (not h % Hkv)
    assert not np.allclose(b, oracle.attn_fwd(q, np.tile(k, (1, G, 1)), np.tile(v, (1, G, 1)), pos)[0])


def test_sampled_rows_equal_full_forward():
    N, Hq, Hkv, D = 300, 4, 1, 8
    q, k, v = _rand((N, Hq, D), 29), _rand((N, Hkv, D), 30), _rand((N, Hkv, D), 31)
    pos = synth.position_ids_from_lengths([100, 7, 150, 43])
    o, lse = oracle.attn_fwd(q, k, v, pos)
    rows = [0, 1, 99, 100, 106, 107, 200, 256, 257, 299]
    r, orow, lrow = oracle.attn_fwd_rows(q, k, v, pos, rows, batch=3)
    np.testing.assert_array_equal(r, rows)
    np.testing.assert_allclose(orow, o[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lrow, lse[:, rows], rtol=1e-12, atol=1e-12)
