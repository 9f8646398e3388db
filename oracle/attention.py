"""Oracle for the rank-local attention step (test infrastructure only).

After the first exchange each device holds the whole sequence for a subset of
heads and runs ordinary attention on it with no further communication (page
"Hugging Face并行加速：10倍提升超长序列训练效率", nmedialink.com, section
"Ulysses的工作原理", step 4 and the paragraph after the steps: heads are
independent; page "DeepSpeed Ulysses 详解", explore.n1n.ai, section
"DeepSpeed-Ulysses 的核心机制：All-to-All 的艺术", step 4).  Masking is causal
within each packed document, derived from position ids (page "Ulysses verteilt
Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch, section
"Integration in den Hugging-Face-Stack").

Readings taken where the pages are silent (the pages only say "standard
attention"):

* scaled dot-product softmax attention per head, scale = 1/sqrt(D) unless
  given;
* causal includes the diagonal: key j is visible to query i iff j <= i and
  both lie in the same document;
* grouped-query attention with consecutive groups: query head h reads KV head
  h // G, G = Hq / Hkv;
* LSE is the natural log of the sum of exp(scaled logits) over visible keys.

Everything is float64 with an explicit boolean mask.  The backward is the
chain rule of L = sum(dO * O): dP = dO V^T, dS = P * (dP - rowsum(P * dP)),
dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO, with dK and dV summed over
the G query heads of a group.

Blocking: queries are processed in blocks of ``block`` rows only to bound
memory.  For a block ending at row r the keys considered are 0..r: every key
after r is masked for every row of the block by causality, so dropping them
changes no term of any sum.
"""

import math

import numpy as np

from .docs import doc_ids, doc_bounds


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def _shapes(q, k, v=None):
    N, Hq, D = q.shape
    Nk, Hkv, Dk = k.shape
    if Nk != N or Dk != D:
        raise ValueError("q and k disagree on N or D")
    if v is not None and v.shape != k.shape:
        raise ValueError("k and v shapes differ")
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return N, Hq, Hkv, D, Hq // Hkv


def _scale(scale, D):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def _positions(position_ids, N):
    if position_ids is None:
        return np.arange(N)
    pos = np.asarray(position_ids).reshape(-1)
    if pos.shape[0] != N:
        raise ValueError("position_ids length != N")
    return pos


def _mask(rows, keys, doc):
    """Explicit mask M[a, b] = (keys[b] <= rows[a]) and doc[keys[b]] == doc[rows[a]]."""
    causal = keys[None, :] <= rows[:, None]
    same_doc = doc[keys][None, :] == doc[rows][:, None]
    return causal & same_doc


def _softmax_block(qb, kb, M, scale):
    """Masked softmax of scale*qb kb^T: returns P, row max m, row sum l of exp(S - m)."""
    S = scale * (qb @ kb.T)
    S = np.where(M, S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return E / l, m[:, 0], l[:, 0]


def attn_probs(q, k, position_ids=None, scale=None, head=0):
    """Full probability matrix P [N, N] of one query head (small N only)."""
    q = _as64(q)
    k = _as64(k)
    N, Hq, Hkv, D, G = _shapes(q, k)
    sc = _scale(scale, D)
    doc = doc_ids(_positions(position_ids, N))
    rows = np.arange(N)
    M = _mask(rows, rows, doc)
    P, _, _ = _softmax_block(q[:, head, :], k[:, head // G, :], M, sc)
    return P


def attn_fwd(q, k, v, position_ids=None, scale=None, block=512):
    """Forward: O [N, Hq, D] float64 and LSE [Hq, N] float64."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    sc = _scale(scale, D)
    doc = doc_ids(_positions(position_ids, N))
    o = np.zeros((N, Hq, D))
    lse = np.zeros((Hq, N))
    for b0 in range(0, N, block):
        rows = np.arange(b0, min(N, b0 + block))
        keys = np.arange(0, rows[-1] + 1)
        M = _mask(rows, keys, doc)
        for h in range(Hq):
            g = h // G
            P, m, l = _softmax_block(q[rows, h, :], k[keys, g, :], M, sc)
            o[rows, h, :] = P @ v[keys, g, :]
            lse[h, rows] = m + np.log(l)
    return o, lse


def attn_bwd(q, k, v, do, position_ids=None, scale=None, block=512):
    """Backward of L = sum(dO * O).

    Returns a dict with dq [N, Hq, D], dk and dv [N, Hkv, D], and the forward
    o, lse plus delta [Hq, N] = rowsum(P * dP), all float64.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    if do.shape != q.shape:
        raise ValueError("dO shape != q shape")
    sc = _scale(scale, D)
    doc = doc_ids(_positions(position_ids, N))
    o = np.zeros((N, Hq, D))
    lse = np.zeros((Hq, N))
    delta = np.zeros((Hq, N))
    dq = np.zeros((N, Hq, D))
    dk = np.zeros((N, Hkv, D))
    dv = np.zeros((N, Hkv, D))
    for b0 in range(0, N, block):
        rows = np.arange(b0, min(N, b0 + block))
        keys = np.arange(0, rows[-1] + 1)
        M = _mask(rows, keys, doc)
        for h in range(Hq):
            g = h // G
            kb, vb, qb, dob = k[keys, g, :], v[keys, g, :], q[rows, h, :], do[rows, h, :]
            P, m, l = _softmax_block(qb, kb, M, sc)
            o[rows, h, :] = P @ vb
            lse[h, rows] = m + np.log(l)
            dP = dob @ vb.T
            dlt = (P * dP).sum(axis=1)
            delta[h, rows] = dlt
            dS = P * (dP - dlt[:, None])
            dq[rows, h, :] = sc * (dS @ kb)
            dk[keys, g, :] += sc * (dS.T @ qb)
            dv[keys, g, :] += P.T @ dob
    return {"dq": dq, "dk": dk, "dv": dv, "o": o, "lse": lse, "delta": delta}


def _group_rows_by_doc(rows, start):
    """Split sorted unique rows into runs that share a document start."""
    rows = np.unique(np.asarray(rows, dtype=np.int64))
    groups = []
    for s in np.unique(start[rows]):
        groups.append(rows[start[rows] == s])
    return groups


def attn_fwd_rows(q, k, v, position_ids, rows, scale=None, batch=64):
    """Forward for selected query rows only: (rows, O[rows] [n, Hq, D], LSE[:, rows]).

    For a batch of rows of one document whose first token is s, the keys
    considered are s..max(rows): keys before s belong to other documents and
    keys after max(rows) are causally masked for every row of the batch.
    The explicit mask is then applied on that range.  Cost O(rows * n_i * D),
    usable at N = 1M.
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    sc = _scale(scale, D)
    pos = _positions(position_ids, N)
    doc = doc_ids(pos)
    start, _ = doc_bounds(pos)
    rows_sorted = np.unique(np.asarray(rows, dtype=np.int64))
    out_o = {}
    out_l = {}
    for grp in _group_rows_by_doc(rows_sorted, start):
        for c0 in range(0, len(grp), batch):
            rb = grp[c0:c0 + batch]
            keys = np.arange(start[rb[0]], rb[-1] + 1)
            M = _mask(rb, keys, doc)
            for h in range(Hq):
                g = h // G
                P, m, l = _softmax_block(_as64(q[rb, h, :]), _as64(k[keys, g, :]), M, sc)
                o = P @ _as64(v[keys, g, :])
                for a, r in enumerate(rb):
                    out_o.setdefault(int(r), np.zeros((Hq, D)))[h] = o[a]
                    out_l.setdefault(int(r), np.zeros(Hq))[h] = m[a] + math.log(l[a])
    O = np.stack([out_o[int(r)] for r in rows_sorted])
    L = np.stack([out_l[int(r)] for r in rows_sorted], axis=1)
    return rows_sorted, O, L


def attn_bwd_dq_rows(q, k, v, do, position_ids, rows, scale=None, batch=64):
    """dQ for selected query rows: (rows, dQ[rows] [n, Hq, D], delta[:, rows])."""
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    sc = _scale(scale, D)
    pos = _positions(position_ids, N)
    doc = doc_ids(pos)
    start, _ = doc_bounds(pos)
    rows_sorted = np.unique(np.asarray(rows, dtype=np.int64))
    out = {}
    out_d = {}
    for grp in _group_rows_by_doc(rows_sorted, start):
        for c0 in range(0, len(grp), batch):
            rb = grp[c0:c0 + batch]
            keys = np.arange(start[rb[0]], rb[-1] + 1)
            M = _mask(rb, keys, doc)
            for h in range(Hq):
                g = h // G
                kb, vb = _as64(k[keys, g, :]), _as64(v[keys, g, :])
                P, _, _ = _softmax_block(_as64(q[rb, h, :]), kb, M, sc)
                dP = _as64(do[rb, h, :]) @ vb.T
                dlt = (P * dP).sum(axis=1)
                dS = P * (dP - dlt[:, None])
                dqb = sc * (dS @ kb)
                for a, r in enumerate(rb):
                    out.setdefault(int(r), np.zeros((Hq, D)))[h] = dqb[a]
                    out_d.setdefault(int(r), np.zeros(Hq))[h] = dlt[a]
    return rows_sorted, np.stack([out[int(r)] for r in rows_sorted]), np.stack(
        [out_d[int(r)] for r in rows_sorted], axis=1)


def attn_bwd_dkdv_rows(q, k, v, do, position_ids, kv_rows, scale=None, batch=64):
    """dK and dV for selected key rows: (kv_rows, dK[kv_rows], dV[kv_rows]).

    Key j receives gradient from the query rows j..end(j) of its document.
    Those rows' full softmax rows are formed as in ``attn_fwd_rows``.  Cheap
    when the selected keys sit near the end of their documents.
    """
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    sc = _scale(scale, D)
    pos = _positions(position_ids, N)
    doc = doc_ids(pos)
    start, end = doc_bounds(pos)
    kv_sorted = np.unique(np.asarray(kv_rows, dtype=np.int64))
    dk_out = {int(j): np.zeros((Hkv, D)) for j in kv_sorted}
    dv_out = {int(j): np.zeros((Hkv, D)) for j in kv_sorted}
    for s in np.unique(start[kv_sorted]):
        js = kv_sorted[start[kv_sorted] == s]
        qrows = np.arange(js[0], end[js[0]] + 1)
        for c0 in range(0, len(qrows), batch):
            rb = qrows[c0:c0 + batch]
            keys = np.arange(s, rb[-1] + 1)
            M = _mask(rb, keys, doc)
            for h in range(Hq):
                g = h // G
                kb, vb = _as64(k[keys, g, :]), _as64(v[keys, g, :])
                qb, dob = _as64(q[rb, h, :]), _as64(do[rb, h, :])
                P, _, _ = _softmax_block(qb, kb, M, sc)
                dP = dob @ vb.T
                dlt = (P * dP).sum(axis=1)
                dS = P * (dP - dlt[:, None])
                for j in js:
                    col = int(j - s)
                    if col < len(keys):
                        dk_out[int(j)][g] += sc * (dS[:, col] @ qb)
                        dv_out[int(j)][g] += P[:, col] @ dob
    return (kv_sorted, np.stack([dk_out[int(j)] for j in kv_sorted]),
            np.stack([dv_out[int(j)] for j in kv_sorted]))


def attn_fwd_per_document(q, k, v, position_ids, scale=None, block=512):
    """Forward run on each document separately, results placed back in sequence order."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    start, end = doc_bounds(_positions(position_ids, N))
    o = np.zeros((N, Hq, D))
    lse = np.zeros((Hq, N))
    for s in np.unique(start):
        e = end[s] + 1
        od, ld = attn_fwd(q[s:e], k[s:e], v[s:e], None, scale, block)
        o[s:e] = od
        lse[:, s:e] = ld
    return o, lse


def attn_bwd_per_document(q, k, v, do, position_ids, scale=None, block=512):
    """Backward run on each document separately, results placed back in sequence order."""
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    N, Hq, Hkv, D, G = _shapes(q, k, v)
    start, end = doc_bounds(_positions(position_ids, N))
    res = {"dq": np.zeros((N, Hq, D)), "dk": np.zeros((N, Hkv, D)), "dv": np.zeros((N, Hkv, D)),
           "o": np.zeros((N, Hq, D)), "lse": np.zeros((Hq, N)), "delta": np.zeros((Hq, N))}
    for s in np.unique(start):
        e = end[s] + 1
        r = attn_bwd(q[s:e], k[s:e], v[s:e], do[s:e], None, scale, block)
        for name in ("dq", "dk", "dv", "o"):
            res[name][s:e] = r[name]
        for name in ("lse", "delta"):
            res[name][:, s:e] = r[name]
    return res
