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
