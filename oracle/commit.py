"""Accepted-path commit of the draft layer's KV cache (test infrastructure only).

"eagle feature-level speculative decoding", section on committing the KV cache
as a transaction: after verification only the accepted path's entries join
the cache; rejected branches are dropped.  The j-th accepted drafted node
(depth j + 1) sits at rotary position L_b + j, so its k, v become prefix
position L_b + j and the prefix grows by the number of accepted drafts.

``commit_slots`` is the same transaction for the catch-up rows of the next
round (the drafter's own rows over the committed tokens, recomputed from the
target's true features): their k, v sit in tree slots 0..n-1 in position order
and become prefix positions L_b..L_b+n-1.
"""
from __future__ import annotations

import numpy as np

OVERFLOW, BAD_PATH = 1, 2


def commit(prefix_k, prefix_v, lens, caps, tree_k, tree_v, paths, accept_len, node_slot=None):
    """prefix_k/v: per sequence [Hkv, L_b, hd] arrays; caps: per sequence
    capacity (None = the length: no room); tree_k/v [B, 64, Hkv, hd]; paths:
    per sequence the accepted drafted nodes in order (the first accept_len-1
    entries count); node_slot: per sequence, tree slot of each node (None:
    slot = node).  Returns the new per-sequence prefixes, lengths and flags."""
    out_k, out_v, out_len, flags = [], [], [], []
    for b in range(len(prefix_k)):
        L = int(lens[b])
        C = L if caps is None else int(caps[b])
        A = max(int(accept_len[b]) - 1, 0)
        nodes = [int(x) for x in paths[b][:A]]
        n_nodes = len(paths[b])
        slots = [int(node_slot[b][n]) if node_slot is not None else n for n in nodes] if nodes else []
        bad = A > n_nodes - 1 or any(n < 1 or n >= n_nodes for n in nodes) or any(s < 0 or s >= 64 for s in slots)
        if bad or L + A > C:
            out_k.append(np.asarray(prefix_k[b]).copy())
            out_v.append(np.asarray(prefix_v[b]).copy())
            out_len.append(L)
            flags.append(BAD_PATH if bad else OVERFLOW)
            continue
        add_k = np.stack([tree_k[b, s] for s in slots], axis=1) if slots else np.zeros_like(prefix_k[b][:, :0])
        add_v = np.stack([tree_v[b, s] for s in slots], axis=1) if slots else np.zeros_like(prefix_v[b][:, :0])
        out_k.append(np.concatenate([np.asarray(prefix_k[b])[:, :L], add_k], axis=1))
        out_v.append(np.concatenate([np.asarray(prefix_v[b])[:, :L], add_v], axis=1))
        out_len.append(L + A)
        flags.append(0)
    return out_k, out_v, out_len, flags


def commit_slots(prefix_k, prefix_v, lens, caps, tree_k, tree_v, counts):
    """Append tree slots 0..counts[b]-1 of sequence b to its prefix at
    positions L_b.. (caps: per-sequence capacity, None = no room).  A count
    outside 0..64 is a malformed request.  Returns the new prefixes, lengths
    and flags (OVERFLOW / BAD_PATH leave the sequence unchanged)."""
    out_k, out_v, out_len, flags = [], [], [], []
    for b in range(len(prefix_k)):
        L = int(lens[b])
        C = L if caps is None else int(caps[b])
        n = int(counts[b])
        if n < 0 or n > 64 or L + n > C:
            out_k.append(np.asarray(prefix_k[b]).copy())
            out_v.append(np.asarray(prefix_v[b]).copy())
            out_len.append(L)
            flags.append(BAD_PATH if (n < 0 or n > 64) else OVERFLOW)
            continue
        add_k = np.stack([tree_k[b, s] for s in range(n)], axis=1) if n else np.zeros_like(prefix_k[b][:, :0])
        add_v = np.stack([tree_v[b, s] for s in range(n)], axis=1) if n else np.zeros_like(prefix_v[b][:, :0])
        out_k.append(np.concatenate([np.asarray(prefix_k[b])[:, :L], add_k], axis=1))
        out_v.append(np.concatenate([np.asarray(prefix_v[b])[:, :L], add_v], axis=1))
        out_len.append(L + n)
        flags.append(0)
    return out_k, out_v, out_len, flags
