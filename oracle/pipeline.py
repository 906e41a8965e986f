"""The whole draft-and-verify round composed from the oracle's steps (test
infrastructure only).

Order of a round ("EAGLE 推测解码为什么比 Medusa 快" section 6; "EAGLE 完全拆解",
the four-step inference pipeline):
  1. root: q_root = softmax(LM_Head(f_j)) from the true feature;
  2. per depth: expand the frontier (EAGLE-2 or a static template), then run one
     draft step over the new frontier rows and take each row's top-k;
  3. rerank and flatten the tree;
  4. one draft step over every drafted node of the flattened tree ("tree-wide
     step"): its logits are the draft distributions at every node and stand in
     for the target's verification forward once noise is added;
  5. recursive rejection sampling over the tree.
Feature rows and logit rows share one index space: rows [0, B) hold the true
root features / root logits, each later step appends its rows.

act_bf16 chooses the bf16 contract of each step's weight products (see
draft.draft_step): False (full-precision operands, the default), True, or
"auto" = bf16 operands for steps over more than ACT_BF16_MIN_ROWS rows of a
bf16 workload.
"""
from __future__ import annotations

import numpy as np

from . import draft as D
from . import tree as T
from .topk import gumbel_topk, softmax_topk
from .verify import verify_sequence


ACT_BF16_MIN_ROWS = 16


def act_for(act_bf16, n_rows: int) -> bool:
    return bool(act_bf16) if act_bf16 != "auto" else n_rows > ACT_BF16_MIN_ROWS


def draft_phase(shape, w, root_feat, root_token, prefix_k, prefix_v, prefix_len, kind: str, k: int, depth: int,
                m: int = 0, template=None, mirror: bool = True, tree_wide: bool = True, act_bf16=False,
                sample=None):
    """sample = (seed, round): children drawn without replacement from each
    expanded node's q (Gumbel-top-k over the row's fp32 logits, row id = the
    row's index in the round) instead of its top-k."""

    def select(lg, row0):
        if sample is None:
            _, i_, q_ = softmax_topk(lg.astype(np.float32), k)
        else:
            _, i_, q_, _ = gumbel_topk(lg.astype(np.float32), k, sample[0], sample[1], np.arange(lg.shape[0]) + row0)
        return i_, q_

    B = root_feat.shape[0]
    nchild = None
    if kind != "dynamic":
        nchild = np.zeros(len(template), dtype=np.int64)
        for p in template[1:]:
            nchild[p] += 1
    feats = [np.asarray(root_feat, np.float64)]
    root_logits = D.head_logits(shape, w, root_feat, mirror, act_for(act_bf16, B))
    logits = [root_logits]
    idx, logq = select(root_logits, 0)
    pools = [T.Pool(root_token[b], b) for b in range(B)]
    frontier = [[0] for _ in range(B)]
    sel_idx = [[idx[b]] for b in range(B)]
    sel_logq = [[logq[b]] for b in range(B)]
    tree_k, tree_v = D.new_tree_kv(shape, B)
    n_rows = B
    steps = []
    for s in range(depth):
        for b in range(B):
            frontier[b] = T.expand(pools[b], frontier[b], sel_idx[b], sel_logq[b], k, nchild)
        if s == depth - 1 or all(len(f) == 0 for f in frontier):
            break
        rows = {"seq": [], "token": [], "parent": [], "pos": [], "slot": [], "mask": []}
        base = n_rows
        for b in range(B):
            for (tok, par, pos, slot, mask) in T.assign_rows(pools[b], frontier[b], s, k, kind != "dynamic",
                                                             base + len(rows["seq"]), int(prefix_len[b])):
                rows["seq"].append(b)
                rows["token"].append(tok)
                rows["parent"].append(par)
                rows["pos"].append(pos)
                rows["slot"].append(slot)
                rows["mask"].append(mask)
        fb = np.concatenate(feats, axis=0)
        out = D.draft_step(shape, w, rows, fb, prefix_k, prefix_v, prefix_len, tree_k, tree_v, mirror,
                           act_bf16=act_for(act_bf16, len(rows["seq"])))
        feats.append(out["feat"])
        logits.append(out["logits"])
        n_rows += len(rows["seq"])
        steps.append(rows)
        idx, logq = select(out["logits"], base)
        o = 0
        for b in range(B):
            nf = len(frontier[b])
            sel_idx[b] = [idx[o + f] for f in range(nf)]
            sel_logq[b] = [logq[o + f] for f in range(nf)]
            o += nf
    trees = [T.finalize(pools[b], m) for b in range(B)]
    res = {"pools": pools, "trees": trees, "steps": steps, "feat_buf": np.concatenate(feats, axis=0),
           "logits": np.concatenate(logits, axis=0)}
    if tree_wide:
        rows = {"seq": [], "token": [], "parent": [], "pos": [], "slot": [], "mask": []}
        for b in range(B):
            tr, pool = trees[b], pools[b]
            for t in range(1, len(tr["parent"])):
                pid = int(tr["pool_id"][t])
                rows["seq"].append(b)
                rows["token"].append(int(tr["token"][t]))
                rows["parent"].append(pool.feat_row[pool.parent[pid]])
                rows["pos"].append(int(prefix_len[b]) + int(tr["depth"][t]) - 1)
                rows["slot"].append(t)
                rows["mask"].append(int(tr["mask"][t]))
        tk, tv = D.new_tree_kv(shape, B)
        out = D.draft_step(shape, w, rows, res["feat_buf"], prefix_k, prefix_v, prefix_len, tk, tv, mirror,
                           act_bf16=act_for(act_bf16, len(rows["seq"])))
        res["tree_wide_rows"] = rows
        res["tree_wide"] = out
    return res


def q_rows(res, b: int):
    """Row of the draft logits holding q at each tree node of sequence b (the
    row where that node was expanded; -1 for unexpanded leaves)."""
    tr, pool = res["trees"][b], res["pools"][b]
    return np.array([pool.feat_row[int(pid)] for pid in tr["pool_id"]], dtype=np.int64)


def verify_all(trees, target_logits, draft_logits, qrow, seed: int, rnd: int, greedy=False, iid=False):
    """Verify every sequence.  target_logits[b][i] per tree node; draft logits
    rows via qrow[b][i]."""
    outs = []
    for b, tr in enumerate(trees):
        dl = [draft_logits[r] if r >= 0 else None for r in qrow[b]]
        outs.append(verify_sequence(tr["parent"], tr["token"], target_logits[b], dl, seed, rnd, b, greedy, iid))
    return outs
