"""Shared helpers for the GPU parity tests (import only from tests)."""

import numpy as np
import pytest
import torch

# tolerances: bf16 inputs, fp32 accumulation, bf16 O
TOL_OUT = 2e-2
TOL_LSE = 1e-3


def grad_bar(ref):
    """Gradient bar: 2e-2 absolute while |ref| <= 8 (the regime of the 4 q / 1 KV
    workloads), then the same relative error (2e-2 / 8 = 2.5e-3, about one bf16
    half-ulp of the probabilities) for larger gradients, which arise with larger
    query groups summing into one KV head."""
    return TOL_OUT * max(1.0, float(np.abs(ref).max()) / 8.0)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")


def np64(t):
    """Exact decode of a device tensor to float64 numpy."""
    return t.detach().to("cpu").double().numpy()


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def dev_inputs(N, Hq, Hkv, D, seed, dtype, with_do=False):
    """Host-drawn seeded inputs (synth) moved to cuda:0."""
    import synth

    host = synth.host_qkv(N, Hq, Hkv, D, seed, "bf16" if dtype == torch.bfloat16 else "f32", with_do)
    return {k: v.to("cuda:0") for k, v in host.items()}, host


def log(msg):
    print(msg, flush=True)
