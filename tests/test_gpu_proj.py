"""GPU parity of the projections (bf16 MFMA GEMM, fp32 accumulation) against
the fp64 oracle.

Bar: the kernel rounds an fp32 sum to bf16 once, so every element must lie
within half a bf16 ulp of the exact value: |got - ref| <= 2^-8 |ref| + 1e-4
(the 1e-4 covers fp32 accumulation over K <= 4096 terms of size ~1/sqrt(K)).
Small shapes are checked in full; the million-token shard (131072 tokens of
a 4096-wide model projecting 32 q / 8 KV heads of 128) on sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_ul_amd as ul
from gpu_helpers import log, np64, require_gpu

pytestmark = pytest.mark.gpu


def _bar_ok(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return bool(np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4))


def _host(shape, seed, stream, scale=1.0):
    x = synth.normal_f32(shape, seed, stream) * np.float32(scale)
    return synth.to_bf16_torch(x)


QKV_CASES = [
    # M, hidden, Hq, Hkv, D, P
    (1, 64, 2, 2, 64, 1),
    (37, 192, 4, 2, 64, 2),
    (256, 256, 8, 2, 128, 2),
    (300, 512, 8, 8, 64, 8),
    (513, 1024, 32, 8, 128, 8),
    (600, 320, 6, 3, 40, 3),     # several row and column tiles, both ragged
    (40, 128, 4, 2, 12, 2),      # D not a multiple of 8: element-wise stores
]


@pytest.mark.parametrize("M,hidden,Hq,Hkv,D,P", QKV_CASES)
def test_qkv_proj_pack_small(M, hidden, Hq, Hkv, D, P):
    require_gpu()
    log(f"qkv_proj_pack M={M} hidden={hidden} Hq={Hq} Hkv={Hkv} D={D} P={P}")
    seed = M + hidden
    x = _host((M, hidden), seed, 1)
    w = _host(((Hq + 2 * Hkv) * D, hidden), seed, 2, 1.0 / np.sqrt(hidden))
    q, k, v = ul.qkv_proj_pack(x.cuda(), w.cuda(), Hq, Hkv, D, P)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.qkv_proj_pack(x.double().numpy(), w.double().numpy(), Hq, Hkv, D, P)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("v", v, rv)):
        assert got.shape == ref.shape, name
        assert _bar_ok(np64(got), ref), name


@pytest.mark.parametrize("M,hidden,HqD", [(1, 64, 64), (77, 200, 128), (256, 4096, 256), (700, 512, 4096),
                                          (50, 100, 64), (300, 1000, 256)])
def test_out_proj_small(M, hidden, HqD):
    require_gpu()
    log(f"out_proj M={M} hidden={hidden} HqD={HqD}")
    seed = 3 * M + HqD
    o = _host((M, HqD), seed, 3)
    w = _host((hidden, HqD), seed, 4, 1.0 / np.sqrt(HqD))
    y = ul.out_proj(o.cuda(), w.cuda())
    torch.cuda.synchronize()
    assert _bar_ok(np64(y), oracle.out_proj(o.double().numpy(), w.double().numpy()))


def test_projections_million_shard_sampled():
    """The million-token share: one shard of N/P = 131072 tokens, hidden 4096, 32 q / 8 KV heads of 128 over
    8 ranks; 96 sampled tokens (first, last, and seeded random ones) against the oracle."""
    require_gpu()
    M, hidden, Hq, Hkv, D, P = 131072, 4096, 32, 8, 128, 8
    dev = torch.device("cuda:0")
    x = synth.device_normal((M, hidden), 41, 1, dev, torch.bfloat16)
    w = (synth.device_normal(((Hq + 2 * Hkv) * D, hidden), 41, 2, dev, torch.float32) / 64.0).to(torch.bfloat16)
    wo = (synth.device_normal((hidden, Hq * D), 41, 3, dev, torch.float32) / 64.0).to(torch.bfloat16)
    log("projections million shard: qkv")
    q, k, v = ul.qkv_proj_pack(x, w, Hq, Hkv, D, P)
    log("projections million shard: out (reading q_send's unpacked equivalent as o)")
    o = x[:, :Hq * D].contiguous()
    y = ul.out_proj(o, wo)
    torch.cuda.synchronize()
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(7).integers(0, M, 94)])
    xs = x[rows].double().cpu().numpy()
    rq, rk, rv = oracle.qkv_proj_pack(xs, w.double().cpu().numpy(), Hq, Hkv, D, P)
    ridx = torch.from_numpy(rows).to(dev)
    assert _bar_ok(np64(q[:, ridx]), rq)
    assert _bar_ok(np64(k[:, ridx]), rk)
    assert _bar_ok(np64(v[:, ridx]), rv)
    ry = oracle.out_proj(o[ridx].double().cpu().numpy(), wo.double().cpu().numpy())
    assert _bar_ok(np64(y[ridx]), ry)


def test_projection_rejections():
    require_gpu()
    x = torch.zeros((8, 100), dtype=torch.bfloat16, device="cuda:0")  # hidden not a multiple of 64
    w = torch.zeros((3 * 64, 100), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ul.UlError):
        ul.qkv_proj_pack(x, w, 1, 1, 64, 1)
    with pytest.raises(ul.UlError):
        ul.out_proj(torch.zeros((8, 96), dtype=torch.bfloat16, device="cuda:0"),
                    torch.zeros((4, 96), dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises((ul.UlError, TypeError)):
        ul.out_proj(torch.zeros((8, 64), dtype=torch.float32, device="cuda:0"),
                    torch.zeros((4, 64), dtype=torch.float32, device="cuda:0"))
