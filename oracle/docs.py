"""Oracle for documents packed into one sequence (test infrastructure only).

Packing replaces a 4-D attention mask by position ids, which keeps the extra
memory linear in the sequence length (page "Ulysses verteilt
Millionen-Token-Kontexte auf mehrere GPUs", dailytechsnack.ch, section
"Integration in den Hugging-Face-Stack"; page "Ulysses 序列並行：百萬 Token
上下文訓練", setupai.cc, section "增強重點摘要", last point).

Reading taken where the pages are silent: a position id equal to 0 starts a
new document; token 0 always starts one (even if its position id is not 0);
no other value or decrease starts a document.
"""

import numpy as np


def doc_ids(position_ids):
    """Document index of every token: doc[0] = 0, doc[t] = doc[t-1] + [pos[t] == 0]."""
    pos = np.asarray(position_ids).reshape(-1)
    N = pos.shape[0]
    doc = np.zeros(N, dtype=np.int64)
    if N > 1:
        doc[1:] = np.cumsum(pos[1:] == 0)
    return doc


def doc_bounds(position_ids):
    """Per-token (start, end), the first and last token of its document (inclusive)."""
    doc = doc_ids(position_ids)
    start = np.searchsorted(doc, doc, side="left").astype(np.int64)
    end = (np.searchsorted(doc, doc, side="right") - 1).astype(np.int64)
    return start, end
