"""Pins of the loss oracle (oracle/loss.py) against closed forms, direct
per-element sums, torch's CPU cross entropy, finite differences and the
invariance of the token-weighted loss to how the sequence is sharded."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth

IGN = oracle.IGNORE_INDEX


def _logits(T, V, seed, scale=3.0):
    return synth.normal_f32((T, V), seed, 40).astype(np.float64) * scale


def _labels(T, V, seed, frac_ignored=0.3):
    rng = np.random.Generator(np.random.PCG64([seed, 41]))
    y = rng.integers(0, V, size=T)
    y[rng.random(T) < frac_ignored] = IGN
    return y


def test_uniform_logits_give_log_vocab():
    T, V = 7, 13
    x = np.full((T, V), 2.5)
    y = np.array([0, 3, IGN, 12, 5, IGN, 1])
    loss, lse = oracle.token_ce(x, y)
    valid = y != IGN
    assert np.allclose(loss[valid], math.log(V), rtol=0, atol=1e-14)
    assert np.all(loss[~valid] == 0.0)
    assert np.allclose(lse, 2.5 + math.log(V), rtol=0, atol=1e-14)


def test_two_classes_is_softplus_of_the_margin():
    for a, b in [(0.0, 0.0), (1.5, -2.0), (-3.0, 4.0), (30.0, -30.0)]:
        loss, _ = oracle.token_ce(np.array([[a, b]]), np.array([0]))
        assert loss[0] == pytest.approx(math.log1p(math.exp(b - a)) if b - a < 30 else b - a, rel=1e-11, abs=1e-14)
        loss1, _ = oracle.token_ce(np.array([[a, b]]), np.array([1]))
        assert loss1[0] == pytest.approx(math.log1p(math.exp(a - b)) if a - b < 30 else a - b, rel=1e-11, abs=1e-14)


def test_matches_minus_log_probability_elementwise():
    T, V = 5, 9
    x = _logits(T, V, 1, scale=1.0)
    y = _labels(T, V, 1, frac_ignored=0.0)
    loss, _ = oracle.token_ce(x, y)
    for t in range(T):
        den = sum(math.exp(x[t, v]) for v in range(V))
        assert loss[t] == pytest.approx(-math.log(math.exp(x[t, y[t]]) / den), rel=1e-12)


def test_adding_a_constant_to_a_row_changes_nothing():
    T, V = 6, 11
    x = _logits(T, V, 2)
    y = _labels(T, V, 2)
    shift = np.arange(T)[:, None] * 17.25 - 40.0
    a, _ = oracle.token_ce(x, y)
    b, _ = oracle.token_ce(x + shift, y)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_torch_cross_entropy_sum_mean_and_gradient():
    T, V = 37, 29
    x = _logits(T, V, 3)
    y = _labels(T, V, 3)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y, dtype=torch.int64)
    s, n = oracle.shard_partial(x, y)
    ref_sum = torch.nn.functional.cross_entropy(xt, yt, ignore_index=IGN, reduction="sum").item()
    assert s == pytest.approx(ref_sum, rel=1e-13)
    assert n == int((y != IGN).sum())
    mean = torch.nn.functional.cross_entropy(xt, yt, ignore_index=IGN, reduction="mean")
    assert oracle.sp_loss(x, y, 1) == pytest.approx(mean.item(), rel=1e-13)
    (2.0 * mean).backward()
    g = oracle.ce_grad(x, y, n, dloss=2.0)
    assert np.allclose(g, xt.grad.numpy(), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_token_weighted_loss_is_the_unsharded_mean(P):
    N, V = 64, 17
    x = _logits(N, V, 4)
    y = _labels(N, V, 4, frac_ignored=0.0)
    first = np.arange(N // 2)
    y[first[first % 4 != 0]] = IGN  # the first half has a quarter of the valid tokens of the second
    ref = torch.nn.functional.cross_entropy(torch.tensor(x), torch.tensor(y), ignore_index=IGN, reduction="mean").item()
    assert oracle.sp_loss(x, y, P) == pytest.approx(ref, rel=1e-13)
    if P > 1:
        # the plain mean of the ranks' own means is a different number here
        T = N // P
        means = [oracle.shard_partial(x[r * T:(r + 1) * T], y[r * T:(r + 1) * T]) for r in range(P)]
        naive = np.mean([s / c for s, c in means if c > 0])
        assert abs(naive - ref) > 1e-3


def test_combine_of_nothing_is_zero():
    assert oracle.combine([0.0, 0.0], [0, 0]) == (0.0, 0)
    x = _logits(4, 5, 5)
    y = np.full(4, IGN)
    assert np.all(oracle.ce_grad(x, y, 0) == 0.0)
    assert oracle.sp_loss(x, y, 2) == 0.0


def test_gradient_by_central_differences_across_shards():
    N, V, P = 8, 5, 2
    x = _logits(N, V, 6, scale=1.0)
    y = _labels(N, V, 6, frac_ignored=0.25)
    total = oracle.valid_count(y)
    assert total > 0
    T = N // P
    g = np.concatenate([oracle.ce_grad(x[r * T:(r + 1) * T], y[r * T:(r + 1) * T], total) for r in range(P)])
    h = 1e-6
    for t in range(N):
        for v in range(V):
            xp = x.copy(); xp[t, v] += h
            xm = x.copy(); xm[t, v] -= h
            fd = (oracle.sp_loss(xp, y, P) - oracle.sp_loss(xm, y, P)) / (2 * h)
            assert g[t, v] == pytest.approx(fd, rel=1e-6, abs=1e-9)


def test_gradient_rows_sum_to_zero_and_ignored_rows_vanish():
    T, V = 20, 31
    x = _logits(T, V, 7)
    y = _labels(T, V, 7, frac_ignored=0.4)
    g = oracle.ce_grad(x, y, 50, dloss=1.5)
    assert np.allclose(g.sum(axis=1), 0.0, atol=1e-15)
    assert np.all(g[y == IGN] == 0.0)
    valid = np.nonzero(y != IGN)[0]
    assert np.all(g[valid, y[valid]] < 0)


def _shift_by_loops(labels, position_ids, ign):
    N = len(labels)
    out = []
    for t in range(N):
        if t + 1 >= N:
            out.append(ign)
        elif position_ids is not None and position_ids[t + 1] == 0:
            out.append(ign)
        else:
            out.append(int(labels[t + 1]))
    return out


@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_shift_labels_against_loops(seed):
    N = 50
    rng = np.random.Generator(np.random.PCG64([seed, 42]))
    labels = rng.integers(0, 1000, size=N)
    labels[rng.random(N) < 0.2] = IGN
    pos = synth.random_positions(N, seed)
    assert oracle.shift_labels(labels, pos).tolist() == _shift_by_loops(labels, pos, IGN)
    assert oracle.shift_labels(labels, None).tolist() == _shift_by_loops(labels, None, IGN)
    assert oracle.shift_labels(labels, pos, ignore_index=-1).tolist() == _shift_by_loops(labels, pos, -1)


def test_shift_labels_special_cases():
    lab = np.arange(10, 20)
    # one-token documents: nothing to predict anywhere
    assert np.all(oracle.shift_labels(lab, np.zeros(10, dtype=np.int32)) == IGN)
    # one token
    assert oracle.shift_labels([5]).tolist() == [IGN]
    # the last token of a shard takes the first token of the next shard when the document continues
    out = oracle.shift_labels(lab, np.arange(10, dtype=np.int32))
    assert out[4] == lab[5] and out[9] == IGN
    # a document that starts at token 6: token 5 has no target
    pos = np.array([0, 1, 2, 3, 4, 5, 0, 1, 2, 3], dtype=np.int32)
    out = oracle.shift_labels(lab, pos)
    assert out[5] == IGN and out[4] == lab[5] and out[6] == lab[7]
    # a position id that decreases without reaching 0 does not start a document
    pos2 = np.array([0, 1, 2, 3, 1, 2, 3, 4, 5, 6], dtype=np.int32)
    assert oracle.shift_labels(lab, pos2)[3] == lab[4]


def test_out_of_range_label_is_rejected():
    with pytest.raises(ValueError):
        oracle.token_ce(np.zeros((2, 4)), np.array([1, 4]))
    with pytest.raises(ValueError):
        oracle.ce_grad(np.zeros((2, 4)), np.array([-5, 0]), 2)
