"""Pins of the oracle's exchanges (CPU only).

The pages fix what the two all-to-alls deliver (sharding into contiguous
token ranges, then whole sequence for a head subset, then back); these tests
check the index formula against the literal pack / exchange / unpack, the
round trip, the hand-written fixture and the divisibility rules.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


@pytest.mark.parametrize("P,N,H,D", [(1, 6, 3, 2), (2, 8, 4, 3), (4, 16, 8, 5), (8, 64, 32, 4), (4, 12, 4, 1)])
def test_index_formula_equals_literal_all_to_all(P, N, H, D):
    x = _rand((N, H, D), P * 100 + N)
    shards = [x[i * N // P:(i + 1) * N // P] for i in range(P)]
    literal = oracle.all_to_all_seq_to_head(shards)
    for r in range(P):
        np.testing.assert_array_equal(oracle.seq_to_head(x, P, r), literal[r])
    back = oracle.all_to_all_head_to_seq(literal)
    for i in range(P):
        np.testing.assert_array_equal(back[i], shards[i])


@pytest.mark.parametrize("P,N,H,D", [(2, 8, 4, 3), (4, 16, 8, 5), (8, 32, 8, 2)])
def test_round_trip_over_all_ranks_is_identity(P, N, H, D):
    x = _rand((N, H, D), 7)
    y = np.full_like(x, np.nan)
    for r in range(P):
        y = oracle.head_to_seq(oracle.seq_to_head(x, P, r), y, P, r)
    np.testing.assert_array_equal(y, x)


def test_head_to_seq_touches_only_its_columns():
    x = _rand((8, 4, 2), 3)
    y = oracle.head_to_seq(np.zeros((8, 2, 2)), x, 2, 1)
    np.testing.assert_array_equal(y[:, :2], x[:, :2])
    assert np.all(y[:, 2:] == 0)


def test_golden_fixture_p2_h4():
    with open(os.path.join(GOLDEN, "relayout_p2_h4.json")) as f:
        g = json.load(f)
    shards = [np.array(s, dtype=np.float64)[:, :, None] for s in g["shards"]]
    x = np.concatenate(shards, axis=0)
    for r in range(g["P"]):
        expect = np.array(g["head_slices"][r], dtype=np.float64)[:, :, None]
        np.testing.assert_array_equal(oracle.seq_to_head(x, g["P"], r), expect)
        np.testing.assert_array_equal(oracle.all_to_all_seq_to_head(shards)[r], expect)


def test_divisibility_rules():
    x = np.zeros((6, 4, 2))
    with pytest.raises(ValueError):
        oracle.seq_to_head(x, 4, 0)  # N % P != 0
    with pytest.raises(ValueError):
        oracle.seq_to_head(np.zeros((8, 6, 2)), 4, 0)  # H % P != 0
    with pytest.raises(ValueError):
        oracle.seq_to_head(np.zeros((8, 4, 2)), 2, 2)  # rank out of range
    with pytest.raises(ValueError):
        oracle.seq_to_head(np.zeros((8, 4, 2)), 2, -1)


def test_bytes_moved():
    N, H, D, P = 64, 32, 128, 8
    x = np.zeros((N, H, D), dtype=np.uint16)
    out = oracle.seq_to_head(x, P, 3)
    assert oracle.relayout_bytes(N, H, D, P, 2) == 2 * out.nbytes == 2 * N * (H // P) * D * 2
