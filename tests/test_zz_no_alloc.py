"""The allocation-free document bounds (ul_doc_bounds_noalloc) against the
workspace entry point (ul_doc_bounds), through the C ABI: exact integers, two
calls in a row with the second on a smaller input (the shared scan array keeps
the first call's partials), and the size limit."""

import ctypes

import numpy as np
import pytest
import torch

import synth
import ulysses_sequence_parallelism_ul_amd as ul
from gpu_helpers import log, require_gpu

pytestmark = pytest.mark.gpu


def _with_workspace(lib, pos, N, stream):
    ds = torch.empty(N, dtype=torch.int32, device="cuda:0")
    de = torch.empty(N, dtype=torch.int32, device="cuda:0")
    wsb = lib.ul_doc_bounds_workspace_bytes(N)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    pptr = None if pos is None else pos.data_ptr()
    assert lib.ul_doc_bounds(pptr, ds.data_ptr(), de.data_ptr(), N, ws.data_ptr(), wsb, stream) == ul.UL_OK
    return ds, de


def _no_alloc(lib, pos, N, ds, de, stream):
    pptr = None if pos is None else pos.data_ptr()
    st = lib.ul_doc_bounds_noalloc(pptr, ds.data_ptr(), de.data_ptr(), N, stream)
    assert st == ul.UL_OK, lib.ul_last_error().decode()


def test_no_alloc_matches_workspace_entry_point_on_two_calls():
    require_gpu()
    lib = ul.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # outputs sized for the larger call, allocated before either call
    N1, N2 = 3_000_001, 70_003
    out_s = torch.full((N1,), -7, dtype=torch.int32, device="cuda:0")
    out_e = torch.full((N1,), -7, dtype=torch.int32, device="cuda:0")
    for N, seed in ((N1, 11), (N2, 12)):
        log(f"no-alloc doc bounds N={N} seed={seed}")
        pos = torch.from_numpy(synth.random_positions(N, seed, max_docs=400)).to("cuda:0")
        ref_s, ref_e = _with_workspace(lib, pos, N, stream)
        ds, de = out_s[:N], out_e[:N]
        _no_alloc(lib, pos, N, ds, de, stream)
        torch.cuda.synchronize()
        assert torch.equal(ds, ref_s) and torch.equal(de, ref_e)
        # one document (no position ids) into the same outputs
        ref_s1, ref_e1 = _with_workspace(lib, None, N, stream)
        _no_alloc(lib, None, N, ds, de, stream)
        torch.cuda.synchronize()
        assert torch.equal(ds, ref_s1) and torch.equal(de, ref_e1)
        assert int(ds.max().item()) == 0 and int(de.min().item()) == N - 1


def test_no_alloc_refuses_sizes_beyond_its_array():
    require_gpu()
    lib = ul.load()
    N = (1 << 26) + 1
    assert lib.ul_doc_bounds_noalloc(None, 0x10000000, 0x40000000, N, None) == ul.UL_ERR_ARG
    assert "allocation-free" in lib.ul_last_error().decode()


def test_no_alloc_on_a_created_stream():
    """A stream other than the null stream: the array is that of the stream's device."""
    require_gpu()
    lib = ul.load()
    N = 200_001
    pos = torch.from_numpy(synth.random_positions(N, 13, max_docs=50)).to("cuda:0")
    ref_s, ref_e = _with_workspace(lib, pos, N, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    ds = torch.empty(N, dtype=torch.int32, device="cuda:0")
    de = torch.empty(N, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        _no_alloc(lib, pos, N, ds, de, ctypes.c_void_p(st.cuda_stream))
    st.synchronize()
    assert torch.equal(ds, ref_s) and torch.equal(de, ref_e)
