"""CPU fp64 oracle for the per-rank hot path of Ulysses sequence parallelism.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The product path (the HIP library and its Python binding) never imports it,
and this package imports nothing from the product path: the two share no
code, no headers, no tables and no helpers.  Inputs reach both sides from
the seeded generators in ``synth/``, which hold none of the method's
arithmetic.

What is computed is the plain definition, in float64 numpy, with an explicit
boolean mask:

* ``relayout``  - the seq->head and head->seq exchanges of one rank, both as
  an index formula and as a literal pack / all-to-all / unpack over P shards.
* ``docs``      - document ids and per-row document bounds from position ids.
* ``attention`` - causal, packed-document, grouped-query softmax attention,
  forward and backward, plus sampled-row forms for very long sequences.
* ``projection`` - the QKV projection of one shard into the send blocks of
  the first exchange, and the output projection.
* ``loss``      - next-token targets of a packed sequence, per-token cross
  entropy of a shard, its token-weighted combination over ranks and the
  gradient of that loss.

Page citations name the page by its title and host and then the section.
The pages are:

* "Ulysses 序列並行：百萬 Token 上下文訓練" (setupai.cc)
* "Hugging Face并行加速：10倍提升超长序列训练效率" (nmedialink.com)
* "DeepSpeed Ulysses 详解：实现百万级长文本大模型训练的序列并行技术" (explore.n1n.ai)
* "Ulysses verteilt Millionen-Token-Kontexte auf mehrere GPUs" (dailytechsnack.ch)

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, brute force, finite differences, invariants that the
pages fix, and a library routine (torch CPU scaled-dot-product attention) on
single-document cases; the projections against per-element sums and the
exchange oracle; the loss against closed forms, direct per-element sums,
torch CPU cross entropy, finite differences and the invariance of the
token-weighted loss to the rank count.
"""

from .relayout import (
    seq_to_head,
    head_to_seq,
    all_to_all_seq_to_head,
    all_to_all_head_to_seq,
    relayout_bytes,
)
from .docs import doc_ids, doc_bounds
from .attention import (
    attn_fwd,
    attn_bwd,
    attn_probs,
    attn_fwd_rows,
    attn_bwd_dq_rows,
    attn_bwd_dkdv_rows,
    attn_fwd_per_document,
    attn_bwd_per_document,
)
from .projection import linear, split_heads, send_blocks, qkv_proj_pack, out_proj
from .loss import IGNORE_INDEX, shift_labels, token_ce, valid_count, shard_partial, combine, ce_grad, sp_loss

__all__ = [
    "seq_to_head",
    "head_to_seq",
    "all_to_all_seq_to_head",
    "all_to_all_head_to_seq",
    "relayout_bytes",
    "doc_ids",
    "doc_bounds",
    "attn_fwd",
    "attn_bwd",
    "attn_probs",
    "attn_fwd_rows",
    "attn_bwd_dq_rows",
    "attn_bwd_dkdv_rows",
    "attn_fwd_per_document",
    "attn_bwd_per_document",
    "linear",
    "split_heads",
    "send_blocks",
    "qkv_proj_pack",
    "out_proj",
    "IGNORE_INDEX",
    "shift_labels",
    "token_ce",
    "valid_count",
    "shard_partial",
    "combine",
    "ce_grad",
    "sp_loss",
]
