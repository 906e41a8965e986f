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


def gumbel_keys(row_logits, seed: int, rnd: int, row_id: int) -> np.ndarray:
    """Gumbel-perturbed ranking keys of one row, in fp32 as the kernel forms
    them: u_v from output word v % 4 of Philox4x64-10 counter (row_id, v // 4,
    0, 1) under key (seed, round), u = ((w >> 41) + 0.5) * 2^-23 (inside (0, 1),
    exact in fp32), g = -log(-log(u)), key = logit + g."""
    from .philox import philox4x64_10_np

    V = len(row_logits)
    groups = np.arange((V + 3) // 4, dtype=np.uint64)
    words = philox4x64_10_np(np.uint64(row_id), groups, np.uint64(0), np.uint64(1), (seed, rnd))
    w = np.stack(words, axis=1).reshape(-1)[:V]  # token v -> word v % 4 of group v // 4
    u = ((w >> np.uint64(41)).astype(np.float32) + np.float32(0.5)) * np.float32(2.0 ** -23)
    g = -np.log(-np.log(u))  # float32 arithmetic
    return (np.asarray(row_logits, np.float32) + g).astype(np.float32)


def gumbel_topk(logits: np.ndarray, k: int, seed: int, rnd: int, row_ids):
    """Sampled proposals (Gumbel-top-k): per row, the k largest Gumbel-perturbed
    logits (ties -> lower index) are k draws without replacement from the
    row's softmax, in draw order.  Returns lse, the drawn indices, their plain
    log-probabilities and the margin between the k-th and (k+1)-th keys (a
    decision closer than fp32 rounding of the key may differ between two
    correct implementations of log)."""
    logits = np.atleast_2d(np.asarray(logits))
    M = logits.shape[0]
    lse = np.zeros(M)
    idx = np.zeros((M, k), dtype=np.int64)
    logq = np.zeros((M, k))
    margin = np.zeros(M)
    for r in range(M):
        lse[r] = row_lse(logits[r])
        key = gumbel_keys(logits[r], seed, rnd, int(row_ids[r])).astype(np.float64) + 0.0
        order = np.lexsort((np.arange(key.size), -key))
        idx[r] = order[:k]
        srt = key[order[:k + 1]]
        margin[r] = float(np.min(np.abs(np.diff(srt)))) if srt.size > 1 else np.inf
        logq[r] = np.asarray(logits[r], np.float64)[idx[r]] - lse[r]
    return lse, idx, logq, margin
