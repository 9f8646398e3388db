"""Oracle for the two Ulysses exchanges of one rank (test infrastructure only).

The method (pages "Hugging Face并行加速：10倍提升超长序列训练效率", nmedialink.com,
section "Ulysses的工作原理", steps 1, 3 and 5; and "DeepSpeed Ulysses 详解",
explore.n1n.ai, section "DeepSpeed-Ulysses 的核心机制：All-to-All 的艺术",
steps 1, 3 and 5):

* the sequence of N tokens is cut into P contiguous shards, shard i holding
  tokens [i*N/P, (i+1)*N/P);
* the first all-to-all turns "part of the sequence, all heads" into "the whole
  sequence, a subset of heads" on every device;
* the second all-to-all turns it back.

Conventions (readings where the pages are silent): the tensors are token-major
[tokens, heads, head_dim]; rank r owns the contiguous head group
[r*H/P, (r+1)*H/P) in ascending order; the heads must divide by P (page
"DeepSpeed Ulysses 详解", section "实践指南：如何配置 Ulysses 训练？") and the
sequence length must divide by P (page "Ulysses verteilt
Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch, section
"Integration in den Hugging-Face-Stack").

Two independent formulations are given: an index formula for one rank
(``seq_to_head`` / ``head_to_seq``) and a literal pack / exchange / unpack over
all P ranks (``all_to_all_*``).  Tests pin each against the other.
"""

import numpy as np


def _check(N, H, P, rank=None):
    if P < 1:
        raise ValueError("P must be >= 1")
    if N % P != 0:
        raise ValueError(f"sequence length {N} is not divisible by P={P}")
    if H % P != 0:
        raise ValueError(f"head count {H} is not divisible by P={P}")
    if rank is not None and not (0 <= rank < P):
        raise ValueError(f"rank {rank} outside [0, {P})")


def seq_to_head(x_seq, P, rank):
    """Rank ``rank``'s view after the first all-to-all.

    ``x_seq`` is [N, H, D]: the P sequence shards [N/P, H, D] stacked in shard
    order, so token s lives on device s // (N/P).  The result is [N, H/P, D]
    with out[s, k, :] = x_seq[s, rank*H/P + k, :] for every token s.
    """
    x_seq = np.asarray(x_seq)
    N, H, D = x_seq.shape
    _check(N, H, P, rank)
    hp = H // P
    heads = rank * hp + np.arange(hp)
    out = np.empty((N, hp, D), dtype=x_seq.dtype)
    for k in range(hp):
        out[:, k, :] = x_seq[:, heads[k], :]
    return out


def head_to_seq(x_head, x_seq, P, rank):
    """Rank ``rank``'s contribution to the second all-to-all.

    Returns a copy of ``x_seq`` ([N, H, D]) in which the head columns
    [rank*H/P, (rank+1)*H/P) are replaced by ``x_head`` ([N, H/P, D]); every
    other column is left untouched.
    """
    x_seq = np.array(x_seq, copy=True)
    x_head = np.asarray(x_head)
    N, H, D = x_seq.shape
    _check(N, H, P, rank)
    hp = H // P
    if x_head.shape != (N, hp, D):
        raise ValueError(f"head slice shape {x_head.shape} != {(N, hp, D)}")
    for k in range(hp):
        x_seq[:, rank * hp + k, :] = x_head[:, k, :]
    return x_seq


def all_to_all_seq_to_head(shards):
    """Literal first exchange over P devices.

    ``shards[i]`` is device i's sequence shard [N/P, H, D].  Device i packs
    one message per destination j holding its tokens for head group j; the
    all-to-all hands message (i -> j) to device j; device j unpacks by
    stacking the messages from i = 0..P-1 along the sequence.  Returns the P
    head slices [N, H/P, D].
    """
    P = len(shards)
    n_loc, H, D = np.asarray(shards[0]).shape
    _check(n_loc * P, H, P)
    hp = H // P
    # pack: send[i][j] = tokens of device i, heads of group j
    send = [[np.asarray(shards[i])[:, j * hp:(j + 1) * hp, :] for j in range(P)] for i in range(P)]
    # exchange: device j receives send[i][j] from every i
    recv = [[send[i][j] for i in range(P)] for j in range(P)]
    # unpack: stack along the sequence in source-device order
    return [np.concatenate(recv[j], axis=0) for j in range(P)]


def all_to_all_head_to_seq(slices):
    """Literal second exchange over P devices (inverse of the first).

    ``slices[j]`` is device j's head slice [N, H/P, D].  Device j sends the
    tokens of shard i to device i; device i stacks the messages from
    j = 0..P-1 along the head axis.  Returns the P sequence shards [N/P, H, D].
    """
    P = len(slices)
    N, hp, D = np.asarray(slices[0]).shape
    _check(N, hp * P, P)
    n_loc = N // P
    send = [[np.asarray(slices[j])[i * n_loc:(i + 1) * n_loc] for i in range(P)] for j in range(P)]
    recv = [[send[j][i] for j in range(P)] for i in range(P)]
    return [np.concatenate(recv[i], axis=1) for i in range(P)]


def relayout_bytes(N, H, D, P, elem_bytes):
    """Bytes one rank's exchange reads plus writes for one tensor.

    Each of the N*(H/P)*D elements of the rank's slice is read once and written
    once: 2*N*(H/P)*D*elem_bytes, the per-device O(n*d/P) volume of the page
    "Hugging Face并行加速" (nmedialink.com), section "通信复杂度分析".
    """
    _check(N, H, P)
    return 2 * N * (H // P) * D * elem_bytes
