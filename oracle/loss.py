"""Oracle for the token-weighted loss of a sequence-sharded step (test
infrastructure only).

What the pages fix:

* Sharding is done for the model by the data loader, and the loss is computed
  piecewise, each rank on its own shard (page "Ulysses 序列並行：百萬 Token
  上下文訓練", setupai.cc, section "增強重點摘要", the DataLoader point).
* A hand-written training loop has to weight the ranks' losses by their
  numbers of valid tokens; the trainers aggregate the loss that way themselves
  (page "Ulysses verteilt Millionen-Token-Kontexte auf mehrere GPUs",
  dailytechsnack.ch, section "Integration in den Hugging-Face-Stack").

Readings taken where the pages are silent (each is the plainest one):

* The loss is next-token cross entropy, l_t = ln sum_v exp(x_tv) - x_t,y_t,
  natural log, over the logits x_t of token t and its target y_t.
* Targets are shifted on the whole packed sequence before it is sharded, since
  the target of a shard's last token is the first token of the next shard:
  y_t = labels[t + 1] when token t + 1 exists and belongs to the same document
  (a position id of 0 starts a document, as for the attention mask), else the
  ignore index.  A label equal to the ignore index (-100 by default; a trainer
  puts it on tokens it does not train on) marks a token that is not counted.
* Token weighting: loss = (sum over ranks of the summed valid-token losses) /
  (sum over ranks of the valid-token counts).  This equals the mean over all
  valid tokens of the unsharded sequence for every rank count and every shard
  boundary, which is the point of the weighting; the plain mean of the ranks'
  own means is not equal to it when the counts differ.
* With no valid token anywhere the loss is 0 and so is its gradient (instead
  of 0 / 0).
* The gradient of that loss with respect to the logits of a valid token t is
  dloss / count_total * (softmax(x_t) - onehot(y_t)); an ignored token's row
  is zero.  Each rank needs the global count before its backward; the count
  depends on the labels only, so it is known before the logits are.
"""

import numpy as np

from .docs import doc_ids

IGNORE_INDEX = -100


def shift_labels(labels, position_ids=None, ignore_index=IGNORE_INDEX):
    """Next-token targets of the whole packed sequence (int64 [N])."""
    lab = np.asarray(labels).reshape(-1).astype(np.int64)
    N = lab.shape[0]
    out = np.full(N, ignore_index, dtype=np.int64)
    if N > 1:
        if position_ids is None:
            same_doc = np.ones(N - 1, dtype=bool)
        else:
            doc = doc_ids(position_ids)
            same_doc = doc[1:] == doc[:-1]
        out[:-1] = np.where(same_doc, lab[1:], ignore_index)
    return out


def _check_labels(labels, V, ignore_index):
    lab = np.asarray(labels).reshape(-1).astype(np.int64)
    bad = (lab != ignore_index) & ((lab < 0) | (lab >= V))
    if bad.any():
        raise ValueError(f"label {lab[bad][0]} is outside [0, {V}) and is not the ignore index")
    return lab


def token_ce(logits, labels, ignore_index=IGNORE_INDEX):
    """Per-token cross entropy (float64 [T], 0 for ignored tokens) and the row log-sum-exp (float64 [T])."""
    x = np.asarray(logits, dtype=np.float64)
    T, V = x.shape
    lab = _check_labels(labels, V, ignore_index)
    m = x.max(axis=1)
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    valid = lab != ignore_index
    y = np.where(valid, lab, 0)
    loss = np.where(valid, lse - x[np.arange(T), y], 0.0)
    return loss, lse


def valid_count(labels, ignore_index=IGNORE_INDEX):
    """Number of counted tokens of a shard."""
    return int((np.asarray(labels).reshape(-1) != ignore_index).sum())


def shard_partial(logits, labels, ignore_index=IGNORE_INDEX):
    """One rank's (summed valid-token loss, valid-token count)."""
    loss, _ = token_ce(logits, labels, ignore_index)
    return float(loss.sum()), valid_count(labels, ignore_index)


def combine(loss_sums, counts):
    """Token-weighted loss from the ranks' partials (what follows the all-reduce of both)."""
    total = int(np.sum(np.asarray(counts, dtype=np.int64)))
    if total == 0:
        return 0.0, 0
    return float(np.sum(np.asarray(loss_sums, dtype=np.float64))) / total, total


def ce_grad(logits, labels, total_count, dloss=1.0, ignore_index=IGNORE_INDEX):
    """d(loss)/d(logits) of one shard (float64 [T, V]) for the global valid count ``total_count``."""
    x = np.asarray(logits, dtype=np.float64)
    T, V = x.shape
    lab = _check_labels(labels, V, ignore_index)
    g = np.zeros_like(x)
    if total_count == 0:
        return g
    valid = lab != ignore_index
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    p = e / e.sum(axis=1, keepdims=True)
    g[valid] = p[valid]
    rows = np.nonzero(valid)[0]
    g[rows, lab[rows]] -= 1.0
    return g * (float(dloss) / total_count)


def sp_loss(logits, labels_shifted, P, ignore_index=IGNORE_INDEX):
    """Loss of a whole sequence computed as P ranks would: shard, per-rank partials, token-weighted combine."""
    x = np.asarray(logits)
    lab = np.asarray(labels_shifted).reshape(-1)
    N = lab.shape[0]
    if N % P:
        raise ValueError(f"N={N} is not divisible by P={P}")
    T = N // P
    sums, counts = [], []
    for r in range(P):
        s, c = shard_partial(x[r * T:(r + 1) * T], lab[r * T:(r + 1) * T], ignore_index)
        sums.append(s)
        counts.append(c)
    return combine(sums, counts)[0]
