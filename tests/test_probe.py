"""The MFMA-rate calibration probe (libul_probe.so, used by bench.py --mfma-ceiling)."""

import ctypes
import math
import os

import pytest

from ulysses_sequence_parallelism_ul_amd import build as B


def _lib():
    if not os.path.exists(B.PROBE_LIB):
        pytest.skip("libul_probe.so is not built")
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.ul_probe_operand_bytes.restype = ctypes.c_size_t
    lib.ul_probe_operand_bytes.argtypes = [ctypes.c_int]
    lib.ul_probe_out_bytes.restype = ctypes.c_size_t
    lib.ul_probe_flops_per_launch.restype = ctypes.c_double
    lib.ul_probe_flops_per_launch.argtypes = [ctypes.c_int]
    lib.ul_probe_mfma_rate.restype = ctypes.c_int
    lib.ul_probe_mfma_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_float),
                                       ctypes.c_void_p]
    return lib


def test_probe_sizes_and_rejections_cpu():
    lib = _lib()
    assert lib.ul_probe_operand_bytes(32) == 1024 * 256 * 16 * 16
    assert lib.ul_probe_operand_bytes(16) == 2 * lib.ul_probe_operand_bytes(32)
    assert lib.ul_probe_operand_bytes(8) == 0
    assert lib.ul_probe_flops_per_launch(2) == 2 * 2 ** 20 * 1024 * 4
    ms = ctypes.c_float(0)
    big = lib.ul_probe_operand_bytes(16)
    fake = 0x10000000  # never dereferenced: every call below fails a check first
    out_b = lib.ul_probe_out_bytes()
    assert lib.ul_probe_mfma_rate(8, 1, 2, fake, big, fake, out_b, ctypes.byref(ms), None) == 1   # shape
    assert lib.ul_probe_mfma_rate(32, 1, 3, fake, big, fake, out_b, ctypes.byref(ms), None) == 1  # odd iters
    assert lib.ul_probe_mfma_rate(32, 0, 2, fake, big, fake, out_b, ctypes.byref(ms), None) == 1  # launches
    assert lib.ul_probe_mfma_rate(16, 1, 2, fake, big - 16, fake, out_b, ctypes.byref(ms), None) == 1  # too small
    assert lib.ul_probe_mfma_rate(32, 1, 2, None, big, fake, out_b, ctypes.byref(ms), None) == 1
    assert lib.ul_probe_mfma_rate(32, 1, 2, fake, big, fake, out_b - 4, ctypes.byref(ms), None) == 1
    assert lib.ul_probe_mfma_rate(32, 1, 2, fake, big, fake, out_b, None, None) == 1


def _mix_lib():
    lib = _lib()
    lib.ul_probe_mix_operand_bytes.restype = ctypes.c_size_t
    lib.ul_probe_mix_out_bytes.restype = ctypes.c_size_t
    lib.ul_probe_mix_flops_per_launch.restype = ctypes.c_double
    lib.ul_probe_mix_flops_per_launch.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.ul_probe_mix_rate.restype = ctypes.c_int
    lib.ul_probe_mix_rate.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                                      ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_float),
                                      ctypes.c_void_p]
    return lib


def test_mix_sizes_cpu():
    lib = _mix_lib()
    # 1024 work-groups of 8 waves; bodies of 64 (forward, dK/dV) or 48 (dQ) MFMAs of 32768 flops
    assert lib.ul_probe_mix_flops_per_launch(0, 10) == 10 * 64 * 32768.0 * 1024 * 8
    assert lib.ul_probe_mix_flops_per_launch(1, 10) == 10 * 48 * 32768.0 * 1024 * 8
    assert lib.ul_probe_mix_flops_per_launch(2, 1) == 64 * 32768.0 * 1024 * 8
    assert lib.ul_probe_mix_flops_per_launch(3, 1) == 0.0
    assert lib.ul_probe_mix_flops_per_launch(-1, 1) == 0.0
    assert lib.ul_probe_mix_out_bytes() == 1024 * 512 * 4
    assert lib.ul_probe_mix_operand_bytes() == 4 << 20


@pytest.mark.parametrize("kind,launches,iters,shrink,null_ms", [
    (-1, 1, 2, 0, False), (3, 1, 2, 0, False), (0, 0, 2, 0, False), (0, 10001, 2, 0, False),
    (0, 1, 0, 0, False), (0, 1, (1 << 20) + 1, 0, False), (1, 1, 2, 16, False), (2, 1, 2, 0, True),
])
def test_mix_rate_rejects_bad_arguments_cpu(kind, launches, iters, shrink, null_ms):
    lib = _mix_lib()
    ms = ctypes.c_float(-1.0)
    fake = 0x10000000  # never dereferenced: every case fails a check before a launch
    st = lib.ul_probe_mix_rate(kind, launches, iters, fake, lib.ul_probe_mix_operand_bytes() - shrink, fake,
                               lib.ul_probe_mix_out_bytes(), None if null_ms else ctypes.byref(ms), None)
    assert st == 1
    assert ms.value == -1.0


@pytest.mark.gpu
def test_probe_runs_on_gpu():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    lib = _lib()
    dev = torch.device("cuda:0")
    nbytes = lib.ul_probe_operand_bytes(16)
    operands = (torch.rand(nbytes // 2, device=dev) - 0.5).to(torch.bfloat16)
    out = torch.empty(lib.ul_probe_out_bytes() // 4, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    for shape in (32, 16):
        ms = ctypes.c_float(0)
        out.fill_(float("nan"))
        st = lib.ul_probe_mfma_rate(shape, 2, 16, operands.data_ptr(), nbytes, out.data_ptr(), out.numel() * 4,
                                    ctypes.byref(ms), ctypes.c_void_p(stream))
        assert st == 0
        assert ms.value > 0.0
        vals = out.cpu()
        assert torch.isfinite(vals).all()
        assert float(vals.abs().sum()) > 0.0
        print(f"probe shape {shape}: {lib.ul_probe_flops_per_launch(16) * 2 / (ms.value * 1e-3) / 1e12:.0f} TFLOP/s "
              f"(short run)", flush=True)
        assert not math.isnan(ms.value)
    lib = _mix_lib()
    mb = lib.ul_probe_mix_operand_bytes()
    mops = torch.randn(mb // 2, device=dev, dtype=torch.float32).to(torch.bfloat16)
    mout = torch.empty(lib.ul_probe_mix_out_bytes() // 4, device=dev)
    for kind in (0, 1, 2):
        ms = ctypes.c_float(0)
        mout.fill_(float("nan"))
        st = lib.ul_probe_mix_rate(kind, 2, 32, mops.data_ptr(), mb, mout.data_ptr(), mout.numel() * 4,
                                   ctypes.byref(ms), ctypes.c_void_p(stream))
        assert st == 0
        assert ms.value > 0.0
        assert torch.isfinite(mout.cpu()).all()
        print(f"mix {kind}: {lib.ul_probe_mix_flops_per_launch(kind, 32) * 2 / (ms.value * 1e-3) / 1e12:.0f} "
              f"TFLOP/s (short run)", flush=True)
