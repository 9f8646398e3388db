"""Pins of the projection oracle (CPU): per-element sums written out, one-hot
weights, and the link between the send blocks of every shard and the
exchange oracle (the first all-to-all delivers to rank r exactly block r of
every shard's projection)."""

import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def test_linear_is_the_per_element_sum():
    r = _rng(0)
    x, w = r.standard_normal((5, 7)), r.standard_normal((3, 7))
    y = oracle.linear(x, w)
    for m in range(5):
        for n in range(3):
            assert y[m, n] == pytest.approx(sum(x[m, k] * w[n, k] for k in range(7)), abs=1e-12)


def test_qkv_send_blocks_by_index():
    r = _rng(1)
    Hq, Hkv, D, P, M, hidden = 4, 2, 3, 2, 6, 5
    x = r.standard_normal((M, hidden))
    w = r.standard_normal(((Hq + 2 * Hkv) * D, hidden))
    q, k, v = oracle.qkv_proj_pack(x, w, Hq, Hkv, D, P)
    assert q.shape == (P, M, Hq // P, D) and k.shape == (P, M, Hkv // P, D) and v.shape == k.shape
    for j in range(P):
        for m in range(M):
            for hl in range(Hq // P):
                for d in range(D):
                    row = (j * (Hq // P) + hl) * D + d
                    assert q[j, m, hl, d] == pytest.approx(x[m] @ w[row], abs=1e-12)
            for hl in range(Hkv // P):
                for d in range(D):
                    rk = Hq * D + (j * (Hkv // P) + hl) * D + d
                    rv = (Hq + Hkv) * D + (j * (Hkv // P) + hl) * D + d
                    assert k[j, m, hl, d] == pytest.approx(x[m] @ w[rk], abs=1e-12)
                    assert v[j, m, hl, d] == pytest.approx(x[m] @ w[rv], abs=1e-12)


def test_one_hot_weights_route_input_features():
    Hq, Hkv, D, P, M = 4, 2, 2, 2, 3
    width = (Hq + 2 * Hkv) * D
    x = np.arange(M * width, dtype=np.float64).reshape(M, width)
    w = np.eye(width)[::-1].copy()      # feature n of the output = input feature width-1-n
    q, k, v = oracle.qkv_proj_pack(x, w, Hq, Hkv, D, P)
    # q head 3 (block 1, local head 1), d = 1 is output feature 7 = input feature width - 8
    assert q[1, 2, 1, 1] == x[2, width - 1 - 7]
    # v head 0 (block 0), d = 0 is output feature (Hq + Hkv) * D = 12 -> input feature width - 13
    assert v[0, 1, 0, 0] == x[1, width - 1 - 12]


@pytest.mark.parametrize("P", [1, 2, 4])
def test_send_blocks_of_all_shards_are_the_first_exchange(P):
    r = _rng(2 + P)
    Hq, Hkv, D, hidden, Ns = 8, 4, 3, 5, 4          # Ns tokens per shard
    w = r.standard_normal(((Hq + 2 * Hkv) * D, hidden))
    shards = [r.standard_normal((Ns, hidden)) for _ in range(P)]
    packs = [oracle.qkv_proj_pack(x, w, Hq, Hkv, D, P) for x in shards]
    q_seq = np.concatenate([oracle.split_heads(oracle.linear(x, w)[:, :Hq * D], Hq, D) for x in shards])
    for rank in range(P):
        recv = np.concatenate([packs[i][0][rank] for i in range(P)])
        np.testing.assert_allclose(recv, oracle.seq_to_head(q_seq, P, rank), atol=0, rtol=0)


def test_out_proj_accepts_split_heads_and_matches_sum():
    r = _rng(9)
    o = r.standard_normal((4, 3, 2))
    w = r.standard_normal((5, 6))
    y = oracle.out_proj(o, w)
    for m in range(4):
        for n in range(5):
            assert y[m, n] == pytest.approx(sum(o.reshape(4, 6)[m, f] * w[n, f] for f in range(6)), abs=1e-12)


def test_send_blocks_rejects_indivisible_heads():
    with pytest.raises(ValueError):
        oracle.send_blocks(np.zeros((2, 6, 1)), 4)
