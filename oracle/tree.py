"""Draft-tree construction, step by step (test infrastructure only).

EAGLE-2 ("EAGLE 推测解码为什么比 Medusa 快" section 10.3; "EAGLE 完全拆解",
EAGLE-2 section):
  * value(node) = product of the draft confidences along the root-to-node path;
    here kept as a log-value, logv(child) = fl32(logv(parent) + logq), an fp32
    left-to-right sum from logv(root) = 0;
  * expand: the k most valuable nodes of the newest layer are fed to the draft
    model; each contributes its top-k tokens as children;
  * rerank: the m most valuable nodes of the whole tree (root excluded) are kept;
    value never grows along a path and ties go to the shallower node, so the
    kept set is a connected tree.
Tie rule for equal values: frontier by creation order; rerank by (depth,
creation).  Creation order = (frontier position, child rank).

Static trees (EAGLE-1 "hand-designed" shapes) use a template: node i has a
fixed number of children, taken as the parent's top-ranked tokens in order.

The flattened tree puts the root first, then kept nodes by (depth, creation);
siblings therefore stay in rank order.  The ancestor mask of a node has one bit
per tree index for itself and each non-root ancestor ("eagle feature-level
speculative decoding", the visibility table of the tree-attention section).

Draft rows.  A node that is expanded gets one decoder row whose input is its
parent's feature and its own token; its rotary position is prefix_len + depth -
1 (siblings share a position).  In the per-depth loop of a dynamic tree, the
node at frontier position f of depth t writes its k, v to slot (t-1)*k + f; in a
static tree, to slot = its template index.  The row's mask is its parent's row
mask plus its own slot.
"""
from __future__ import annotations

import numpy as np


class Pool:
    """Candidate pool of one sequence (node 0 = root).  `invalid` is set when an
    expansion cannot be carried out (a NaN value, or a template asking a node
    for more children than its row ranks); the pool then stops growing and its
    flattened tree is the root alone."""

    def __init__(self, root_token: int, root_feat_row: int):
        self.invalid = False
        self.parent = [-1]
        self.token = [int(root_token)]
        self.depth = [0]
        self.logv = [np.float32(0.0)]
        self.feat_row = [int(root_feat_row)]  # row holding this node's feature once expanded
        self.slot = [-1]
        self.mask = [0]

    def __len__(self):
        return len(self.parent)

    def add(self, parent: int, token: int, logq) -> int:
        self.parent.append(int(parent))
        self.token.append(int(token))
        self.depth.append(self.depth[parent] + 1)
        self.logv.append(np.float32(np.float32(self.logv[parent]) + np.float32(logq)))
        self.feat_row.append(-1)
        self.slot.append(-1)
        self.mask.append(0)
        return len(self.parent) - 1


def expand(pool: Pool, frontier, topk_idx, topk_logq, k: int, nchild=None):
    """Create the children of every frontier node and choose the next frontier.

    topk_idx / topk_logq: per frontier position, the node's ranked tokens.
    nchild: static template child counts by node id (None = EAGLE-2).
    Returns the next frontier (pool ids).  A NaN log-value among the new
    children (a NaN logit row makes every log q of that row NaN), or a
    template count beyond the ranked tokens a row provides, marks the pool
    invalid instead: nothing is added and the frontier is empty.
    """
    if pool.invalid:
        return []
    want = [(f, r) for f, u in enumerate(frontier) for r in range(k if nchild is None else int(nchild[u]))]
    if any(r >= len(topk_idx[f]) for f, r in want) or any(
            np.isnan(np.float32(np.float32(pool.logv[frontier[f]]) + np.float32(topk_logq[f][r]))) for f, r in want):
        pool.invalid = True
        return []
    children = []
    for f, r in want:
        children.append(pool.add(frontier[f], topk_idx[f][r], topk_logq[f][r]))
    if nchild is None:
        ranked = sorted(children, key=lambda i: (-float(pool.logv[i]), i))
        return ranked[:k]
    return [c for c in children if int(nchild[c]) > 0]


def assign_rows(pool: Pool, frontier, step: int, k: int, static: bool, feat_row_base: int, prefix_len: int):
    """Decoder rows of the next draft step for this sequence's frontier.

    Returns a list of (token, parent_feat_row, pos, slot, mask) and records the
    feature row, slot and mask on each frontier node."""
    rows = []
    for f, u in enumerate(frontier):
        p = pool.parent[u]
        slot = u if static else step * k + f
        mask = pool.mask[p] | (1 << slot)
        pool.slot[u] = slot
        pool.mask[u] = mask
        pool.feat_row[u] = feat_row_base + f
        rows.append((pool.token[u], pool.feat_row[p], prefix_len + pool.depth[u] - 1, slot, mask))
    return rows


def finalize(pool: Pool, m: int = 0):
    """Rerank (top-m by value, ties to shallower then earlier) and flatten.

    m = 0 keeps every pool node (static templates).  An invalid pool gives the
    root alone.  Returns dict of arrays over tree indices: pool_id, parent,
    token, depth, mask (uint64)."""
    cand = [] if pool.invalid else list(range(1, len(pool)))
    if m:
        cand = sorted(cand, key=lambda i: (-float(pool.logv[i]), pool.depth[i], i))[:m]
    order = [0] + sorted(cand, key=lambda i: (pool.depth[i], i))
    where = {pid: t for t, pid in enumerate(order)}
    parent = [-1]
    for pid in order[1:]:
        if pool.parent[pid] not in where:
            raise ValueError("kept set is not connected")
        parent.append(where[pool.parent[pid]])
    mask = [0]
    for t in range(1, len(order)):
        mask.append(mask[parent[t]] | (1 << t))
    return {
        "pool_id": np.array(order, dtype=np.int64),
        "parent": np.array(parent, dtype=np.int64),
        "token": np.array([pool.token[i] for i in order], dtype=np.int64),
        "depth": np.array([pool.depth[i] for i in order], dtype=np.int64),
        "mask": np.array(mask, dtype=np.uint64),
        "logv": np.array([pool.logv[i] for i in order], dtype=np.float32),
    }


def visible_sets(parent):
    """For each node, the set of nodes it may attend to: its ancestors and
    itself, root included."""
    out = []
    for u in range(len(parent)):
        s, a = [], u
        while a >= 0:
            s.append(a)
            a = parent[a]
        out.append(sorted(s))
    return out
