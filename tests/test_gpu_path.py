"""The whole per-rank path at full size: seq->head, attention forward and
backward, head->seq, for the packed training share (N=262144) and the
million-token share (N=1048576), bf16, 8 emulated ranks, rank 0.

Checks: exchanges bit-exact on full tensors against a torch slice (an
independent library routine) and on sampled rows against the oracle; forward
and dQ on sampled rows against the oracle; dK/dV on the last 64 keys of each
of the first three documents against the oracle; per-document dK/dV sums; the
Q = 0 and K = 0 closed forms at N = 1M (the latter on whole dK / dV tensors);
a ragged N = 1,000,008 packed case on the last rank;
determinism; and, for the training share, every
document's O, LSE, dQ, dK and dV on whole tensors against the oracle run per
document.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_ul_amd as ul
from gpu_helpers import TOL_LSE, TOL_OUT, log, max_abs, np64, require_gpu

pytestmark = pytest.mark.gpu

P, RANK = 8, 0


def _run(name, zero_q=False):
    w = synth.WORKLOADS[name]
    N, D = w["N"], w["D"]
    dev = torch.device("cuda:0")
    seed = w["index"]
    q_seq = synth.device_normal((N, w["Hq"], D), seed, 1, dev, torch.bfloat16)
    k_seq = synth.device_normal((N, w["Hkv"], D), seed, 2, dev, torch.bfloat16)
    v_seq = synth.device_normal((N, w["Hkv"], D), seed, 3, dev, torch.bfloat16)
    do_seq = synth.device_normal((N, w["Hq"], D), seed, 4, dev, torch.bfloat16)
    if zero_q:
        q_seq.zero_()
    pos_np = synth.workload_positions(name)
    pos = torch.from_numpy(pos_np).to(dev)
    q, k, v, do = (ul.seq_to_head(x, P, RANK) for x in (q_seq, k_seq, v_seq, do_seq))
    o, lse = ul.attn_fwd(q, k, v, pos)
    dq, dk, dv = ul.attn_bwd(q, k, v, o, do, lse, pos)
    o_seq = torch.zeros_like(q_seq)
    dq_seq = torch.zeros(q_seq.shape, dtype=torch.float32, device=dev)
    dk_seq = torch.zeros(k_seq.shape, dtype=torch.float32, device=dev)
    dv_seq = torch.zeros(k_seq.shape, dtype=torch.float32, device=dev)
    ul.head_to_seq(o, o_seq, P, RANK)
    ul.head_to_seq(dq, dq_seq, P, RANK)
    ul.head_to_seq(dk, dk_seq, P, RANK)
    ul.head_to_seq(dv, dv_seq, P, RANK)
    torch.cuda.synchronize()
    return dict(N=N, D=D, pos=pos_np, q_seq=q_seq, k_seq=k_seq, v_seq=v_seq, do_seq=do_seq, q=q, k=k, v=v, do=do,
                o=o, lse=lse, dq=dq, dk=dk, dv=dv, o_seq=o_seq, dq_seq=dq_seq, dk_seq=dk_seq, dv_seq=dv_seq)


def _check_exchanges(r):
    hq = r["q"].shape[1]
    hkv = r["k"].shape[1]
    for full, part, hp in ((r["q_seq"], r["q"], hq), (r["k_seq"], r["k"], hkv), (r["v_seq"], r["v"], hkv),
                           (r["do_seq"], r["do"], hq)):
        assert torch.equal(part.view(torch.int16), full[:, RANK * hp:(RANK + 1) * hp].contiguous().view(torch.int16))
    for full, part, hp in ((r["o_seq"], r["o"], hq), (r["dq_seq"], r["dq"], hq), (r["dk_seq"], r["dk"], hkv),
                           (r["dv_seq"], r["dv"], hkv)):
        assert torch.equal(full[:, RANK * hp:(RANK + 1) * hp], part)
        assert torch.count_nonzero(full[:, (RANK + 1) * hp:]) == 0
    # oracle on a row sample of the raw bits
    rows = torch.arange(0, 64, device="cuda:0")
    bits = r["q_seq"][rows].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(r["q"][rows].view(torch.int16).cpu().numpy(), oracle.seq_to_head(bits, P, RANK))


def _host(r):
    return (r["q"].float().cpu().numpy(), r["k"].double().cpu().numpy(), r["v"].double().cpu().numpy(),
            r["do"].float().cpu().numpy())


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", ["train_packed", "million"])
def test_full_path(name):
    require_gpu()
    log(f"path {name}")
    r = _run(name)
    _check_exchanges(r)
    N, pos = r["N"], r["pos"]
    pos_o = None if name == "million" else pos  # million: one document (ids 0..N-1)
    qf, k64, v64, dof = _host(r)
    rng = np.random.Generator(np.random.PCG64(11))
    # first and last 64 rows, rows on both sides of key-tile (64), work-group (64 tokens at 4 heads) and
    # larger power-of-two boundaries, and 112 random rows (about 256 in all)
    edges = [b + d for b in (64, 128, 4096, 65536, N // 2) for d in (-1, 0, 1) if 0 <= b + d < N]
    rows = np.unique(np.r_[0:64, N - 64:N, edges, rng.integers(0, N, 112)])
    log(f"path {name}: oracle forward rows")
    rr, eo, el = oracle.attn_fwd_rows(qf, k64, v64, pos_o, rows)
    ri = torch.from_numpy(rr).to("cuda:0")
    assert max_abs(np64(r["o"][ri]), eo) <= TOL_OUT
    assert max_abs(np64(r["lse"][:, ri]), el) <= TOL_LSE
    log(f"path {name}: oracle dQ rows")
    rr, edq, _ = oracle.attn_bwd_dq_rows(qf, k64, v64, dof, pos_o, rows)
    assert max_abs(np64(r["dq"][torch.from_numpy(rr).to("cuda:0")]), edq) <= TOL_OUT
    log(f"path {name}: oracle dK/dV rows")
    _, end = oracle.doc_bounds(pos)
    ends = np.unique(end)[:3]
    kv_rows = np.unique(np.concatenate([np.arange(max(0, e - 63), e + 1) for e in ends]))
    rr, edk, edv = oracle.attn_bwd_dkdv_rows(qf, k64, v64, dof, pos_o, kv_rows)
    ri = torch.from_numpy(rr).to("cuda:0")
    assert max_abs(np64(r["dk"][ri]), edk) <= TOL_OUT
    assert max_abs(np64(r["dv"][ri]), edv) <= TOL_OUT
    # per-document sums of dK and dV over the whole tensor
    dk64, dv64 = np64(r["dk"]), np64(r["dv"])
    do_sum = r["do"].double().reshape(N, r["k"].shape[1], -1, r["D"]).sum(dim=2)
    start, _ = oracle.doc_bounds(pos)
    for s in np.unique(start)[:8]:
        e = int(end[s]) + 1
        L = e - s
        assert np.abs(dk64[s:e].sum(axis=0)).max() <= TOL_OUT * np.sqrt(L)
        assert np.abs(dv64[s:e].sum(axis=0) - np64(do_sum[s:e].sum(dim=0))).max() <= TOL_OUT * np.sqrt(L)


@pytest.mark.timeout(900)
def test_training_share_full_tensor_per_document():
    """The packed training share (N=262144, 39 documents, 4 q / 1 KV heads, D=128, bf16) on whole
    tensors: O, LSE, dQ, dK and dV of every document against the explicit-mask oracle run on that
    document alone (a packed sequence equals its documents run separately, pinned by the oracle tests)."""
    require_gpu()
    log("path train_packed: full tensors per document")
    r = _run("train_packed")
    N, pos = r["N"], r["pos"]
    q64, k64, v64, do64 = (np64(r[x]) for x in ("q", "k", "v", "do"))
    gpu = {x: np64(r[x]) for x in ("o", "dq", "dk", "dv")}
    lse64 = np64(r["lse"])
    starts = np.flatnonzero(pos == 0)
    ends = np.r_[starts[1:], N]
    assert starts[0] == 0 and len(starts) == len(np.unique(oracle.doc_bounds(pos)[0]))
    worst = dict.fromkeys(("o", "lse", "dq", "dk", "dv"), 0.0)
    for s, e in zip(starts, ends):
        ref = oracle.attn_bwd(q64[s:e], k64[s:e], v64[s:e], do64[s:e], None)
        for x in ("o", "dq", "dk", "dv"):
            worst[x] = max(worst[x], max_abs(gpu[x][s:e], ref[x]))
        worst["lse"] = max(worst["lse"], max_abs(lse64[:, s:e], ref["lse"]))
        log(f"path train_packed document [{s}, {e}): worst so far " + ", ".join(f"{x} {v:.3e}" for x, v in worst.items()))
    for x in ("o", "dq", "dk", "dv"):
        assert worst[x] <= TOL_OUT, (x, worst[x])
    assert worst["lse"] <= TOL_LSE


@pytest.mark.timeout(300)
def test_million_zero_queries_closed_forms():
    """Q = 0 over one 1M-token document: O_i = mean(V[0..i]), LSE_i = ln(i+1), dK = 0,
    dV_j = sum_{i>=j} (sum over the group of dO_i) / (i+1)."""
    require_gpu()
    log("path million Q=0")
    r = _run("million", zero_q=True)
    N, D = r["N"], r["D"]
    v = r["v"].double()[:, 0]
    idx = torch.arange(1, N + 1, device="cuda:0", dtype=torch.float64)
    mean = torch.cumsum(v, dim=0) / idx[:, None]
    for h in range(r["q"].shape[1]):
        assert float((r["o"][:, h].double() - mean).abs().max()) <= TOL_OUT
        assert float((r["lse"][h].double() - torch.log(idx)).abs().max()) <= TOL_LSE
    assert float(r["dk"].abs().max()) <= TOL_OUT
    g = r["do"].double().sum(dim=1) / idx[:, None]          # group sum of dO_i / (i+1)
    dv_ref = torch.flip(torch.cumsum(torch.flip(g, [0]), dim=0), [0])
    assert float((r["dv"][:, 0].double() - dv_ref).abs().max()) <= TOL_OUT


def _zero_keys_closed_forms(N, Hq, D, rows, seed):
    """K = 0 over one N-token document (one KV head) with dO non-zero only on
    the rows R, scaled by (i+1)/16 so that every such row adds O(0.1) to the
    gradient of every key before it.  Then P_ij = 1/(i+1) and, with n_i = i+1
    and O_i = mean(V[0..i]):
      dQ = 0,  dV_j = sum_{i in R, i >= j} sum_h dO_ih / n_i,
      dK_j = scale sum_{i in R, i >= j} sum_h ((dO_ih . V_j) - dO_ih . O_i) Q_ih / n_i,
    so dK (with non-zero Q) and dV are checked on whole tensors, including the
    query rows far above each key's own window of query tiles."""
    dev = torch.device("cuda:0")
    scale = 1.0 / D ** 0.5
    q = synth.device_normal((N, Hq, D), seed, 1, dev, torch.bfloat16)
    v = synth.device_normal((N, 1, D), seed, 3, dev, torch.bfloat16)
    k = torch.zeros((N, 1, D), dtype=torch.bfloat16, device=dev)
    R = torch.tensor(rows, device=dev)
    n_r = (R + 1).double()
    do = torch.zeros((N, Hq, D), dtype=torch.bfloat16, device=dev)
    do[R] = (synth.device_normal((len(rows), Hq, D), seed, 4, dev, torch.float32) * (n_r / 16.0)[:, None, None].float()
             ).to(torch.bfloat16)
    o, lse = ul.attn_fwd(q, k, v, None)
    dq, dk, dv = ul.attn_bwd(q, k, v, o, do, lse, None)
    torch.cuda.synchronize()
    idx = torch.arange(1, N + 1, device=dev, dtype=torch.float64)
    mean = torch.cumsum(v[:, 0].double(), dim=0) / idx[:, None]
    for h in range(Hq):
        assert float((o[:, h].double() - mean).abs().max()) <= TOL_OUT
        assert float((lse[h].double() - torch.log(idx)).abs().max()) <= TOL_LSE
    assert float(dq.abs().max()) == 0.0
    # per row i of R: A = sum_h dO_ih Q_ih^T / n_i (so V_j A = sum_h (dO_ih . V_j) Q_ih / n_i),
    # b = sum_h (dO_ih . O_i) Q_ih / n_i, g = sum_h dO_ih / n_i
    qr, dor = q[R].double(), do[R].double()
    A = torch.stack([dor[i].t().contiguous() @ qr[i] for i in range(len(rows))]) / n_r[:, None, None]
    delta = (dor * mean[R][:, None, :]).sum(dim=2)
    b = (delta[:, :, None] * qr).sum(dim=1) / n_r[:, None]
    g = dor.sum(dim=1) / n_r[:, None]
    # suffix sums over R; keys in (r_{k-1}, r_k] see rows r_k, r_{k+1}, ...
    A_s = torch.flip(torch.cumsum(torch.flip(A, [0]), 0), [0])
    b_s = torch.flip(torch.cumsum(torch.flip(b, [0]), 0), [0])
    g_s = torch.flip(torch.cumsum(torch.flip(g, [0]), 0), [0])
    dk_err = dv_err = 0.0
    lo = 0
    for kk, r in enumerate(rows):
        vj = v[lo:r + 1, 0].double()
        dk_ref = scale * (vj @ A_s[kk] - b_s[kk])
        dk_err = max(dk_err, float((dk[lo:r + 1, 0].double() - dk_ref).abs().max()))
        dv_err = max(dv_err, float((dv[lo:r + 1, 0].double() - g_s[kk]).abs().max()))
        lo = r + 1
    if lo < N:
        dk_err = max(dk_err, float(dk[lo:].abs().max()))
        dv_err = max(dv_err, float(dv[lo:].abs().max()))
    log(f"  K=0 N={N} Hq={Hq} D={D}: max|dK - closed form| {dk_err:.3e}, max|dV - closed form| {dv_err:.3e}, "
        f"max|dK| {float(dk.abs().max()):.3f}, max|dV| {float(dv.abs().max()):.3f}")
    assert dk_err <= TOL_OUT and dv_err <= TOL_OUT


@pytest.mark.timeout(300)
def test_million_zero_keys_closed_forms():
    """The K = 0 closed forms over the million-token document (4 q / 1 KV heads,
    D = 128): 32 rows of R spread over the sequence."""
    require_gpu()
    log("path million K=0, sparse dO")
    rows = sorted({0, 5, 1000, 32767, 32768, 40000, 65535, 65536, 100000, 131071, 262143, 262144, 300001,
                   500000, 524288, 640000, 777777, 900000, 1000000, 1048575}
                  | set(np.random.Generator(np.random.PCG64(9)).integers(0, 1 << 20, 12).tolist()))
    _zero_keys_closed_forms(1 << 20, 4, 128, rows, 9)


@pytest.mark.timeout(300)
def test_split_key_blocks_zero_keys_closed_forms():
    """The K = 0 closed forms where a window of 2048 query tiles is only 8192
    tokens (16 query heads on one KV head, D = 64): the 24576-token document
    spans three windows, so its first 64 key blocks are split."""
    require_gpu()
    log("K=0 split key blocks, 16 q / 1 KV heads")
    rows = [0, 3, 700, 4095, 8191, 8192, 9000, 12000, 16383, 16384, 17000, 20000, 24000, 24575]
    _zero_keys_closed_forms(24576, 16, 64, rows, 12)


@pytest.mark.timeout(300)
def test_training_share_deterministic():
    require_gpu()
    a = _run("train_packed")
    b = _run("train_packed")
    for name in ("o", "lse", "dq", "dk", "dv", "o_seq", "dq_seq"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.timeout(400)
def test_ragged_million_packed_last_rank():
    """N = 1,000,008 (a multiple of the 8 ranks but of no tile size: 8 tokens past the last full 64-token tile),
    three documents of 300,001, 7 and 700,000 tokens (the long ones split into query-tile windows, the short one
    inside one key block), rank 7 of 8: exchanges bit-exact on whole tensors, forward and dQ on sampled rows
    (the ragged tail included), dK/dV on the last 64 keys of every document, against the oracle."""
    require_gpu()
    N, HqA, HkvA, D, rank = 1_000_008, 32, 8, 128, 7
    lengths = [300_001, 7, 700_000]
    assert sum(lengths) == N and N % P == 0
    log(f"ragged path N={N} docs={lengths} rank={rank}")
    dev = torch.device("cuda:0")
    seed = 41
    q_seq = synth.device_normal((N, HqA, D), seed, 1, dev, torch.bfloat16)
    k_seq = synth.device_normal((N, HkvA, D), seed, 2, dev, torch.bfloat16)
    v_seq = synth.device_normal((N, HkvA, D), seed, 3, dev, torch.bfloat16)
    do_seq = synth.device_normal((N, HqA, D), seed, 4, dev, torch.bfloat16)
    pos_np = synth.position_ids_from_lengths(lengths)
    pos = torch.from_numpy(pos_np).to(dev)
    q, k, v, do = (ul.seq_to_head(x, P, rank) for x in (q_seq, k_seq, v_seq, do_seq))
    o, lse = ul.attn_fwd(q, k, v, pos)
    dq, dk, dv = ul.attn_bwd(q, k, v, o, do, lse, pos)
    outs = {}
    for name, t, hp in (("o", o, HqA // P), ("dq", dq, HqA // P), ("dk", dk, HkvA // P), ("dv", dv, HkvA // P)):
        full = torch.zeros((N, hp * P, D), dtype=t.dtype, device=dev)
        ul.head_to_seq(t, full, P, rank)
        outs[name] = (full, hp)
    torch.cuda.synchronize()
    log("ragged path: exchanges")
    for full, part, hp in ((q_seq, q, HqA // P), (k_seq, k, HkvA // P), (v_seq, v, HkvA // P), (do_seq, do, HqA // P)):
        assert torch.equal(part.view(torch.int16), full[:, rank * hp:(rank + 1) * hp].contiguous().view(torch.int16))
    for name, part in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        full, hp = outs[name]
        assert torch.equal(full[:, rank * hp:(rank + 1) * hp], part)
        assert torch.count_nonzero(full[:, :rank * hp]) == 0
    del outs, q_seq, k_seq, v_seq, do_seq
    log("ragged path: oracle forward and dQ rows")
    qf, k64, v64, dof = (q.float().cpu().numpy(), k.double().cpu().numpy(), v.double().cpu().numpy(),
                         do.float().cpu().numpy())
    rng = np.random.Generator(np.random.PCG64(41))
    starts = np.cumsum([0] + lengths[:-1])
    edges = [b + d for b in list(starts) + [N - 8, N // 2, 65536] for d in (-1, 0, 1) if 0 <= b + d < N]
    rows = np.unique(np.r_[0:32, N - 72:N, edges, rng.integers(0, N, 64)])
    rr, eo, el = oracle.attn_fwd_rows(qf, k64, v64, pos_np, rows)
    ri = torch.from_numpy(rr).to(dev)
    assert max_abs(np64(o[ri]), eo) <= TOL_OUT
    assert max_abs(np64(lse[:, ri]), el) <= TOL_LSE
    rr, edq, _ = oracle.attn_bwd_dq_rows(qf, k64, v64, dof, pos_np, rows)
    assert max_abs(np64(dq[torch.from_numpy(rr).to(dev)]), edq) <= TOL_OUT
    log("ragged path: oracle dK/dV on the last keys of every document")
    ends = starts + np.array(lengths) - 1
    kv_rows = np.unique(np.concatenate([np.arange(max(s, e - 63), e + 1) for s, e in zip(starts, ends)]))
    rr, edk, edv = oracle.attn_bwd_dkdv_rows(qf, k64, v64, dof, pos_np, kv_rows)
    ri = torch.from_numpy(rr).to(dev)
    assert max_abs(np64(dk[ri]), edk) <= TOL_OUT
    assert max_abs(np64(dv[ri]), edv) <= TOL_OUT
