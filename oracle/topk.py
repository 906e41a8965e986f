"""Softmax normaliser and per-row top-k, by definition (test infrastructure only).

EAGLE-2 ranks a node's children by the draft model's confidence, i.e. the
softmax probability of each token ("EAGLE 推测解码为什么比 Medusa 快" section
10.2-10.3).  Top-k here is the first k entries of a full stable sort of the row
by (logit descending, index ascending); -0.0 counts as +0.0.  The confidences
are returned as log-probabilities logq = logit - logsumexp(row).
"""
from __future__ import annotations

import numpy as np


def row_lse(row) -> float:
    v = np.asarray(row, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("NaN logit")
    m = np.max(v)
    return float(m + np.log(np.sum(np.exp(v - m))))


def row_topk(row, k: int):
    """Indices of the k largest entries, ties broken by lower index."""
    v = np.asarray(row, dtype=np.float64) + 0.0  # canonical zero
    if np.isnan(v).any():
        raise ValueError("NaN logit")
    order = np.lexsort((np.arange(v.size), -v))  # primary key -v, then index
    return order[:k].astype(np.int64)


def softmax_topk(logits: np.ndarray, k: int):
    """Per row: lse, top-k indices and their log-probabilities."""
    logits = np.atleast_2d(np.asarray(logits))
    M = logits.shape[0]
    lse = np.zeros(M)
    idx = np.zeros((M, k), dtype=np.int64)
    logq = np.zeros((M, k))
    for r in range(M):
        lse[r] = row_lse(logits[r])
        idx[r] = row_topk(logits[r], k)
        logq[r] = np.asarray(logits[r], np.float64)[idx[r]] - lse[r]
    return lse, idx, logq
