"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and lays out test workloads; it holds none of
the method's arithmetic (no exchange, no mask, no softmax).  Both the oracle
and the HIP path receive exactly the arrays made here.

Workloads (the pages name no dataset; these stand in for long-context
fine-tuning of a Llama-3-8B-shaped model with document packing):

* ``tiny_fp32``      - N=1024, 8 q heads = 8 KV heads, D=64, P=4, fp32, one document.
* ``llama8b_1doc``   - N=32768, rank share 4 q / 1 KV heads, D=128, bf16, one document.
* ``llama8b_packed`` - N=131072, same share, packed documents.
* ``train_packed``   - N=262144, shards [32768, 32|8, 128] x 8, packed, with dO.
* ``million``        - N=1048576, one document, shards x 8, with dO.

Document lengths are log-uniform in [512, 32768): L = floor(exp(u)),
u ~ U[ln 512, ln 32768), drawn until they cover N, the last one truncated to
fill N.  Position ids restart at 0 at every document.  Q, K, V and dO are
N(0, 1) draws in fp32, rounded to bf16 (round to nearest even) where the
workload is bf16.  Workload k uses seed k.
"""

import math

import numpy as np

WORKLOADS = {
    "tiny_fp32": dict(index=0, N=1024, Hq=8, Hkv=8, D=64, P=4, dtype="f32", packed=False, bwd=False),
    "llama8b_1doc": dict(index=1, N=32768, Hq=32, Hkv=8, D=128, P=8, dtype="bf16", packed=False, bwd=False),
    "llama8b_packed": dict(index=2, N=131072, Hq=32, Hkv=8, D=128, P=8, dtype="bf16", packed=True, bwd=False),
    "train_packed": dict(index=3, N=262144, Hq=32, Hkv=8, D=128, P=8, dtype="bf16", packed=True, bwd=True),
    "million": dict(index=4, N=1048576, Hq=32, Hkv=8, D=128, P=8, dtype="bf16", packed=False, bwd=True),
}


def doc_lengths(N, seed, lo=512, hi=32768):
    """Log-uniform document lengths covering exactly N tokens (last one truncated)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = []
    total = 0
    while total < N:
        u = rng.uniform(math.log(lo), math.log(hi))
        L = int(math.floor(math.exp(u)))
        L = min(L, N - total)
        lengths.append(L)
        total += L
    return lengths


def position_ids_from_lengths(lengths):
    """Concatenate 0..L-1 for every document length L (int32)."""
    return np.concatenate([np.arange(L, dtype=np.int32) for L in lengths])


def single_document_positions(N):
    return np.arange(N, dtype=np.int32)


def normal_f32(shape, seed, stream=0):
    """fp32 N(0,1) array from a PCG64 stream keyed by (seed, stream)."""
    rng = np.random.Generator(np.random.PCG64([seed, stream]))
    return rng.standard_normal(size=shape, dtype=np.float32)


def to_bf16_torch(x_f32):
    """fp32 numpy -> torch bfloat16 CPU tensor (round to nearest even)."""
    import torch

    return torch.from_numpy(np.ascontiguousarray(x_f32)).to(torch.bfloat16)


def host_qkv(N, Hq, Hkv, D, seed, dtype="bf16", with_do=False):
    """Q [N,Hq,D], K/V [N,Hkv,D] (and dO [N,Hq,D]) as torch CPU tensors of ``dtype``."""
    import torch

    arrays = {
        "q": normal_f32((N, Hq, D), seed, 1),
        "k": normal_f32((N, Hkv, D), seed, 2),
        "v": normal_f32((N, Hkv, D), seed, 3),
    }
    if with_do:
        arrays["do"] = normal_f32((N, Hq, D), seed, 4)
    out = {}
    for name, a in arrays.items():
        out[name] = to_bf16_torch(a) if dtype == "bf16" else torch.from_numpy(a)
    return out


def device_normal(shape, seed, stream, device, dtype):
    """N(0,1) draws made on the device with a seeded torch generator (large workloads)."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + stream)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x.to(dtype)


def workload_positions(name, N=None):
    """Position ids of a named workload (optionally at a reduced N with the same recipe)."""
    w = WORKLOADS[name]
    n = w["N"] if N is None else N
    if w["packed"]:
        return position_ids_from_lengths(doc_lengths(n, w["index"]))
    return single_document_positions(n)


def random_positions(N, seed, max_docs=8, min_len=1):
    """Small random packings for edge-case tests: random cut points, ids restart at 0."""
    rng = np.random.Generator(np.random.PCG64([seed, 99]))
    ndocs = int(rng.integers(1, max_docs + 1))
    cuts = np.sort(rng.choice(np.arange(1, N), size=min(ndocs - 1, max(N - 1, 0)), replace=False)) if N > 1 else []
    bounds = [0] + [int(c) for c in cuts] + [N]
    lengths = [b - a for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
    return position_ids_from_lengths(lengths)


def token_labels(N, V, seed, frac_ignored=0.1, ignore_index=-100):
    """int32 token ids uniform in [0, V) with a fraction set to the ignore index (untrained tokens)."""
    rng = np.random.Generator(np.random.PCG64([seed, 50]))
    y = rng.integers(0, V, size=N, dtype=np.int64)
    y[rng.random(N) < frac_ignored] = ignore_index
    return y.astype(np.int32)


def device_logits(T, V, seed, device, dtype, std=3.0, rows_per_draw=2048):
    """Logits [T, V] ~ N(0, std^2), drawn on the device in row blocks (no fp32 copy of the whole tensor)."""
    import torch

    out = torch.empty((T, V), dtype=dtype, device=device)
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000003 + 60)
    for r0 in range(0, T, rows_per_draw):
        r1 = min(T, r0 + rows_per_draw)
        blk = torch.randn((r1 - r0, V), generator=g, device=device, dtype=torch.float32)
        out[r0:r1] = (blk * std).to(dtype)
    return out
