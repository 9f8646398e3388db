"""Pins of the oracle's document bounds (CPU only): brute force and special cases."""

import numpy as np
import pytest

import oracle
import synth


def _brute(pos):
    """Walk left and right from every token until a document start (pos == 0 or t == 0)."""
    N = len(pos)
    start, end = [], []
    for i in range(N):
        s = i
        while s > 0 and pos[s] != 0:
            s -= 1
        e = i
        while e + 1 < N and pos[e + 1] != 0:
            e += 1
        start.append(s)
        end.append(e)
    return np.array(start), np.array(end)


@pytest.mark.parametrize("seed", range(20))
def test_bounds_match_brute_force(seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    N = int(rng.integers(1, 60))
    pos = synth.random_positions(N, seed)
    # sprinkle non-zero decreases that must not start a document
    s, e = oracle.doc_bounds(pos)
    bs, be = _brute(pos)
    np.testing.assert_array_equal(s, bs)
    np.testing.assert_array_equal(e, be)


def test_all_zero_positions_give_single_token_documents():
    pos = np.zeros(7, dtype=np.int32)
    s, e = oracle.doc_bounds(pos)
    np.testing.assert_array_equal(s, np.arange(7))
    np.testing.assert_array_equal(e, np.arange(7))
    np.testing.assert_array_equal(oracle.doc_ids(pos), np.arange(7))


def test_arange_is_one_document():
    s, e = oracle.doc_bounds(np.arange(9))
    assert np.all(s == 0) and np.all(e == 8)


def test_first_token_starts_a_document_even_if_nonzero():
    pos = np.array([5, 6, 7, 0, 1])
    s, e = oracle.doc_bounds(pos)
    np.testing.assert_array_equal(s, [0, 0, 0, 3, 3])
    np.testing.assert_array_equal(e, [2, 2, 2, 4, 4])


def test_decrease_without_zero_does_not_split():
    pos = np.array([0, 1, 2, 1, 2, 0, 1])
    np.testing.assert_array_equal(oracle.doc_ids(pos), [0, 0, 0, 0, 0, 1, 1])


def test_generator_lengths_cover_n():
    lengths = synth.doc_lengths(131072, 2)
    assert sum(lengths) == 131072
    assert all(1 <= L < 32768 for L in lengths)
    assert all(L >= 512 for L in lengths[:-1])
    pos = synth.position_ids_from_lengths(lengths)
    assert int((pos == 0).sum()) == len(lengths)
