"""Oracle for the projections on either side of the path (test infrastructure only).

The method (page "Hugging Face并行加速：10倍提升超长序列训练效率", nmedialink.com,
section "Ulysses的工作原理", step 2: every device projects its own sequence
shard into queries, keys and values; step 6: after the return exchange, the
output projection): a plain per-token linear map of the shard.

Conventions (readings where the pages are silent): weights are stored one row
per output feature, so y = x W^T; the fused QKV weight stacks the rows of W_q
(Hq*D rows), W_k and W_v (Hkv*D rows each), and head h of a tensor is its D
consecutive features.  The QKV results are delivered in the send layout of the
first exchange: block j holds heads [j*H/P, (j+1)*H/P) of every token of the
shard, the part rank j receives (pages as for ``relayout``).
"""

import numpy as np


def linear(x, w):
    """y = x W^T in float64: x [M, K], w [Nc, K] -> [M, Nc]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def split_heads(y, H, D):
    """[M, H*D] -> [M, H, D] (head h = features [h*D, (h+1)*D))."""
    y = np.asarray(y)
    return y.reshape(y.shape[0], H, D)


def send_blocks(t, P):
    """[M, H, D] -> [P, M, H/P, D]: block j is heads [j*H/P, (j+1)*H/P), the part rank j receives."""
    t = np.asarray(t)
    M, H, D = t.shape
    if H % P != 0:
        raise ValueError(f"head count {H} is not divisible by P={P}")
    hp = H // P
    return np.stack([t[:, j * hp:(j + 1) * hp, :] for j in range(P)])


def qkv_proj_pack(x, w_qkv, Hq, Hkv, D, P):
    """Projection of one shard into the send blocks.

    x [M, hidden], w_qkv [(Hq + 2*Hkv)*D, hidden].  Returns (q_send [P, M, Hq/P, D],
    k_send [P, M, Hkv/P, D], v_send [P, M, Hkv/P, D]) in float64.
    """
    y = linear(x, w_qkv)
    q = split_heads(y[:, :Hq * D], Hq, D)
    k = split_heads(y[:, Hq * D:(Hq + Hkv) * D], Hkv, D)
    v = split_heads(y[:, (Hq + Hkv) * D:], Hkv, D)
    return send_blocks(q, P), send_blocks(k, P), send_blocks(v, P)


def out_proj(o_seq, w_o):
    """Output projection of one shard: o_seq [M, Hq*D] (or [M, Hq, D]) times w_o [hidden, Hq*D]^T."""
    o = np.asarray(o_seq)
    return linear(o.reshape(o.shape[0], -1), w_o)
