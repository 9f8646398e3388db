"""GPU document bounds against the oracle: exact integers."""

import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_ul_amd as ul
from gpu_helpers import log, require_gpu

pytestmark = pytest.mark.gpu


def _check(pos_np):
    pos = torch.from_numpy(np.asarray(pos_np, dtype=np.int32)).to("cuda:0")
    ds, de = ul.doc_bounds(pos)
    torch.cuda.synchronize()
    s, e = oracle.doc_bounds(pos_np)
    np.testing.assert_array_equal(ds.cpu().numpy(), s)
    np.testing.assert_array_equal(de.cpu().numpy(), e)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("N", [1, 2, 63, 1023, 1024, 1025, 3000, 5000])
def test_random_packings(N, seed):
    require_gpu()
    _check(synth.random_positions(N, seed, max_docs=12))


def test_special_cases():
    require_gpu()
    _check(np.zeros(3000, dtype=np.int32))            # every token its own document
    _check(np.arange(4097, dtype=np.int32))           # one document
    _check(np.array([5, 6, 7, 0, 1], dtype=np.int32))  # first token not 0
    _check(np.r_[np.arange(2048), np.arange(3000) + 7].astype(np.int32))  # decrease without 0


def test_null_positions_is_one_document():
    require_gpu()
    ds, de = ul.doc_bounds(None, N=2500, device="cuda:0")
    torch.cuda.synchronize()
    assert torch.all(ds == 0) and torch.all(de == 2499)


@pytest.mark.parametrize("name", ["llama8b_packed", "train_packed"])
def test_workload_packings(name):
    require_gpu()
    log(f"doc bounds {name}")
    _check(synth.workload_positions(name))


def test_million_tokens_packed():
    require_gpu()
    _check(synth.position_ids_from_lengths(synth.doc_lengths(1 << 20, 11)))
