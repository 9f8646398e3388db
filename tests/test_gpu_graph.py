"""The whole rank path (seq->head, attention forward and backward, head->seq) captured once in a
HIP graph through torch.cuda.graph and replayed: no call of the path allocates, synchronizes or
clears memory with a memset, so a captured step must reproduce the eager one bit for bit on every
replay (the kernels are deterministic).  Each replay is followed by unrelated eager work and a
synchronization before its outputs are checked."""

import pytest
import torch

import synth
import ulysses_sequence_parallelism_ul_amd as ul

from gpu_helpers import log, require_gpu


@pytest.mark.gpu
@pytest.mark.parametrize("packed", [False, True])
def test_rank_path_graph_replays_match_eager(packed):
    require_gpu()
    dev = torch.device("cuda:0")
    N, Hq_all, Hkv_all, D, P, rank = 4096, 32, 8, 128, 8, 5
    log(f"graph capture of the rank path N={N} packed={packed}")
    host = synth.host_qkv(N, Hq_all, Hkv_all, D, 77, "bf16", with_do=True)
    x = {k: v.to(dev) for k, v in host.items()}
    pos = synth.position_ids_from_lengths([1000, 3, 1500, 1593]) if packed else synth.position_ids_from_lengths([N])
    pos_d = torch.from_numpy(pos).to(dev)
    Hq, Hkv = Hq_all // P, Hkv_all // P
    q, do_ = (torch.empty(N, Hq, D, dtype=torch.bfloat16, device=dev) for _ in range(2))
    k, v = (torch.empty(N, Hkv, D, dtype=torch.bfloat16, device=dev) for _ in range(2))
    o_seq = torch.zeros_like(x["q"])
    dq_seq = torch.zeros(N, Hq_all, D, dtype=torch.float32, device=dev)
    dk_seq = torch.zeros(N, Hkv_all, D, dtype=torch.float32, device=dev)
    dv_seq = torch.zeros_like(dk_seq)

    def step():
        ul.seq_to_head(x["q"], P, rank, q)
        ul.seq_to_head(x["k"], P, rank, k)
        ul.seq_to_head(x["v"], P, rank, v)
        ul.seq_to_head(x["do"], P, rank, do_)
        o, lse = ul.attn_fwd(q, k, v, pos_d)
        dq, dk, dv = ul.attn_bwd(q, k, v, o, do_, lse, pos_d)
        ul.head_to_seq(o, o_seq, P, rank)
        ul.head_to_seq(dq, dq_seq, P, rank)
        ul.head_to_seq(dk, dk_seq, P, rank)
        ul.head_to_seq(dv, dv_seq, P, rank)
        return lse

    lse_eager = step().clone()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o_seq, dq_seq, dk_seq, dv_seq, lse_eager)]

    # warm up on a side stream, as torch recommends before capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    for t in (o_seq, dq_seq, dk_seq, dv_seq):
        t.zero_()
    with torch.cuda.graph(g):
        lse_g = step()
    for rep in range(3):
        for t in (o_seq, dq_seq, dk_seq, dv_seq, lse_g):
            t.fill_(float("nan"))  # the replay must rewrite the rank's columns and the lse
        g.replay()
        scratch = torch.randn(1 << 20, device=dev).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        got = (o_seq, dq_seq, dk_seq, dv_seq, lse_g)
        for name, a, b in zip(("o", "dq", "dk", "dv", "lse"), got, ref):
            # head->seq writes only the rank's columns; compare those
            if name != "lse":
                H = a.shape[1]
                cols = slice(rank * H // P, (rank + 1) * H // P)
                a, b = a[:, cols], b[:, cols]
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        log(f"replay {rep} bit-identical")


@pytest.mark.gpu
def test_rank_calls_graph_replays_match_eager():
    """The same check for the one-call rank path (ul_rank_attn_fwd / ul_rank_attn_bwd) in two head chunks,
    with caller-provided workspaces."""
    require_gpu()
    dev = torch.device("cuda:0")
    N, Hq_all, Hkv_all, D, P, rank, chunks = 4096, 32, 8, 128, 4, 2, 2
    log(f"graph capture of the rank calls N={N} P={P} chunks={chunks}")
    host = synth.host_qkv(N, Hq_all, Hkv_all, D, 78, "bf16", with_do=True)
    x = {k: v.to(dev) for k, v in host.items()}
    pos_d = torch.from_numpy(synth.position_ids_from_lengths([2048, 17, 2031])).to(dev)
    ws_f = torch.empty(ul.rank_workspace_bytes(N, Hq_all, Hkv_all, D, P, chunks, torch.bfloat16, False),
                       dtype=torch.uint8, device=dev)
    ws_b = torch.empty(ul.rank_workspace_bytes(N, Hq_all, Hkv_all, D, P, chunks, torch.bfloat16, True),
                       dtype=torch.uint8, device=dev)
    o_seq = torch.zeros_like(x["q"])
    lse = torch.empty(Hq_all // P, N, dtype=torch.float32, device=dev)
    dq_seq = torch.zeros(N, Hq_all, D, dtype=torch.float32, device=dev)
    dk_seq = torch.zeros(N, Hkv_all, D, dtype=torch.float32, device=dev)
    dv_seq = torch.zeros_like(dk_seq)
    outs = (o_seq, lse, dq_seq, dk_seq, dv_seq)

    def step():
        ul.rank_attn_fwd(x["q"], x["k"], x["v"], P, rank, pos_d, chunks, o_seq=o_seq, lse=lse, workspace=ws_f)
        ul.rank_attn_bwd(x["q"], x["k"], x["v"], o_seq, x["do"], lse, P, rank, pos_d, chunks,
                         dq_seq=dq_seq, dk_seq=dk_seq, dv_seq=dv_seq, workspace=ws_b)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        g.replay()
        scratch = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), outs, ref):
            if name != "lse":
                H = a.shape[1]
                cols = slice(rank * H // P, (rank + 1) * H // P)
                a, b = a[:, cols], b[:, cols]
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        log(f"replay {rep} bit-identical")


@pytest.mark.gpu
def test_projection_and_loss_calls_graph_replays_match_eager():
    """The projections and the loss entry points captured together (shard projection into the send blocks,
    output projection, label shift, per-shard counts, their combination, cross entropy with its gradient on
    two shards, and the combination of the loss sums): every replay equals the eager calls."""
    require_gpu()
    dev = torch.device("cuda:0")
    M, hidden, Hq, Hkv, D, P, V = 1000, 512, 8, 2, 64, 2, 1000
    log(f"graph capture of projections and loss M={M} hidden={hidden} V={V}")
    g = torch.Generator(device=dev)
    g.manual_seed(79)

    def rnd(*shape, s=1.0):
        return (torch.randn(*shape, generator=g, device=dev) * s).to(torch.bfloat16)

    x, o_in = rnd(M, hidden), rnd(M, Hq * D)
    wqkv, wo = rnd((Hq + 2 * Hkv) * D, hidden, s=hidden ** -0.5), rnd(hidden, Hq * D, s=(Hq * D) ** -0.5)
    labels = torch.randint(0, V, (M,), generator=g, device=dev, dtype=torch.int32)
    labels[::7] = ul.IGNORE_INDEX
    pos = torch.from_numpy(synth.position_ids_from_lengths([400, 1, 599])).to(dev)
    T = M // P
    logits = [rnd(T, V, s=2.0) for _ in range(P)]
    q_send = torch.empty(P, M, Hq // P, D, dtype=torch.bfloat16, device=dev)
    k_send = torch.empty(P, M, Hkv // P, D, dtype=torch.bfloat16, device=dev)
    v_send = torch.empty_like(k_send)
    y = torch.empty(M, hidden, dtype=torch.bfloat16, device=dev)
    y_lab = torch.empty(M, dtype=torch.int32, device=dev)
    counts = torch.empty(P, dtype=torch.int64, device=dev)
    total = torch.empty(1, dtype=torch.int64, device=dev)
    sums = torch.empty(P, dtype=torch.float64, device=dev)
    loss = torch.empty(1, dtype=torch.float64, device=dev)
    loss_tok = torch.empty(M, dtype=torch.float32, device=dev)
    dlogits = [torch.empty(T, V, dtype=torch.bfloat16, device=dev) for _ in range(P)]
    outs = [q_send, k_send, v_send, y, y_lab, counts, total, sums, loss, loss_tok] + dlogits

    def step():
        ul.qkv_proj_pack(x, wqkv, Hq, Hkv, D, P, q_send, k_send, v_send)
        ul.out_proj(o_in, wo, y)
        ul.shift_labels(labels, pos, out=y_lab)
        for r in range(P):
            ul.ce_count(y_lab[r * T:(r + 1) * T], count=counts[r:r + 1])
        ul.loss_combine(counts, total_count=total)
        for r in range(P):
            ul.cross_entropy(logits[r], y_lab[r * T:(r + 1) * T], total_count=total, grad=True,
                             loss_tok=loss_tok[r * T:(r + 1) * T], loss_sum=sums[r:r + 1], dlogits=dlogits[r])
        ul.loss_combine(counts, loss_sums=sums, total_count=total, loss=loss)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert int(total.item()) == int((y_lab != ul.IGNORE_INDEX).sum().item())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for rep in range(3):
        for t in outs:
            if t.is_floating_point():
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        gr.replay()
        scratch = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager calls"
        log(f"replay {rep} bit-identical")
