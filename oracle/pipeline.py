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
  5. recursive rejection sampling over the tree;
  6. catch-up and commit ("eagle feature-level speculative decoding", KV
     commit section: the drafter continues from the committed path A-B-X, not
     from its own predicted state; study note section 6.2 and implementation
     note 3: the accepted path's true features start the next round): the
     drafter's rows over the committed tokens are recomputed from the target's
     true features, their k, v join the prefix, and the row of the verifier's
     next token gives the next round's root feature.
Feature rows and logit rows share one index space: rows [0, B) hold the root
features / root logits, each later step appends its rows.

act_bf16 chooses the bf16 contract of each step's weight products (see
draft.draft_step): False (full-precision operands, the default), True, or a
function of a step's row count returning one of those (a caller that runs
some steps under one contract and some under the other says which here).
"""
from __future__ import annotations

import numpy as np

from . import draft as D
from . import tree as T
from .commit import commit_slots
from .topk import gumbel_topk, softmax_topk
from .verify import verify_sequence


def act_for(act_bf16, n_rows: int) -> bool:
    return bool(act_bf16(n_rows)) if callable(act_bf16) else bool(act_bf16)


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
        rows = tree_wide_rows(trees, pools, prefix_len)
        tk, tv = D.new_tree_kv(shape, B)
        out = D.draft_step(shape, w, rows, res["feat_buf"], prefix_k, prefix_v, prefix_len, tk, tv, mirror,
                           act_bf16=act_for(act_bf16, len(rows["seq"])))
        res["tree_wide_rows"] = rows
        res["tree_wide"] = out
    return res


def tree_wide_rows(trees, pools, prefix_len):
    """Rows of one draft step over every drafted node of the flattened trees:
    node t of sequence b takes its parent's feature row (the true feature for
    depth 1, else the parent's predicted feature), its own token, rotary
    position L_b + depth - 1, tree slot t and the node's ancestor mask."""
    rows = {"seq": [], "token": [], "parent": [], "pos": [], "slot": [], "mask": []}
    for b, (tr, pool) in enumerate(zip(trees, pools)):
        for t in range(1, len(tr["parent"])):
            pid = int(tr["pool_id"][t])
            rows["seq"].append(b)
            rows["token"].append(int(tr["token"][t]))
            rows["parent"].append(pool.feat_row[pool.parent[pid]])
            rows["pos"].append(int(prefix_len[b]) + int(tr["depth"][t]) - 1)
            rows["slot"].append(t)
            rows["mask"].append(int(tr["mask"][t]))
    return rows


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


def catchup_rows(tree_token, path, accept_len, next_token, prefix_len, true_row0):
    """Catch-up rows of one sequence after its verification.

    The round's root sits at sequence position L_b (the draft layer's prefix
    holds positions 0..L_b-1); the A = accept_len - 1 accepted drafted nodes
    x_1..x_A sit at L_b+1..L_b+A and the verifier's next token X (correction or
    bonus) at L_b+A+1.  The drafter's row at position p joins the true feature
    at p with the embedding of the token at p+1 (feature first, advanced token
    second), so row i = 0..A is
        [f_true(node at path position i) ; e(x_{i+1})]   (x_{A+1} = X)
    at rotary position L_b + i, written to tree slot i and seeing slots 0..i
    (the committed tokens form a chain).  The true feature of tree node n is
    feature row true_row0 + n (the root is node 0).  Returns A + 1 tuples
    (token, parent_row, pos, slot, mask)."""
    A = int(accept_len) - 1
    nodes = [0] + [int(n) for n in path[:A]]
    toks = [int(tree_token[n]) for n in path[:A]] + [int(next_token)]
    return [(toks[i], true_row0 + nodes[i], int(prefix_len) + i, i, (1 << (i + 1)) - 1) for i in range(A + 1)]


def catchup_step(shape, w, trees, outs, true_feat, prefix_k, prefix_v, prefix_len, prefix_cap, mirror: bool = True):
    """Catch-up draft step over every sequence's committed tokens, then the
    commit of its k, v (slots 0..A_b) to the prefix.  trees/outs: the round's
    flattened trees and verify results; true_feat [B*N, d]: the target's true
    feature at every tree node (row b*N + node).  Returns the rows, the step's
    outputs, the new prefix (k, v, lengths), commit flags, and the next
    round's root features (f^ of each sequence's last row) and root tokens."""
    B = len(trees)
    N = len(trees[0]["token"])
    rows = {"seq": [], "token": [], "parent": [], "pos": [], "slot": [], "mask": []}
    last = []
    for b in range(B):
        o = outs[b]
        for (tok, par, pos, slot, mask) in catchup_rows(trees[b]["token"], o["path"], o["accept_len"],
                                                        o["next_token"], prefix_len[b], b * N):
            rows["seq"].append(b)
            rows["token"].append(tok)
            rows["parent"].append(par)
            rows["pos"].append(pos)
            rows["slot"].append(slot)
            rows["mask"].append(mask)
        last.append(len(rows["seq"]) - 1)
    tk, tv = D.new_tree_kv(shape, B)
    out = D.draft_step(shape, w, rows, true_feat, prefix_k, prefix_v, prefix_len, tk, tv, mirror, want_logits=False)
    counts = [outs[b]["accept_len"] for b in range(B)]  # A_b + 1 committed positions
    pk, pv, lens, flags = commit_slots(prefix_k, prefix_v, prefix_len, prefix_cap, tk, tv, counts)
    return {"rows": rows, "out": out, "tree_k": tk, "tree_v": tv, "prefix_k": pk, "prefix_v": pv,
            "prefix_len": np.array(lens), "flags": flags, "root_feat": out["feat"][last],
            "root_token": np.array([outs[b]["next_token"] for b in range(B)])}


def decode_rounds(shape, w, root_feat, root_token, prefix_k, prefix_v, prefix_len, prefix_cap, kind: str, k: int,
                  depth: int, m: int, template, n_rounds: int, target_for, true_feat_for, seed: int = 0,
                  greedy: bool = False, mirror: bool = True):
    """n_rounds rounds of draft phase, verification, catch-up and commit.
    target_for(r, res) -> per-sequence target logits [N, V] of round r's tree
    nodes (res = the round's draft_phase result); true_feat_for(r, res) ->
    [B*N, d] true features of those nodes.  Round r verifies with Philox round
    r.  Returns one dict per round."""
    rounds = []
    feat, tok = np.asarray(root_feat, np.float64), np.asarray(root_token)
    pk, pv, lens = list(prefix_k), list(prefix_v), np.asarray(prefix_len)
    for r in range(n_rounds):
        res = draft_phase(shape, w, feat, tok, pk, pv, lens, kind, k, depth, m, template, mirror)
        B = len(res["trees"])
        targets = target_for(r, res)
        qrow = [q_rows(res, b) for b in range(B)]
        outs = verify_all(res["trees"], targets, res["logits"], qrow, seed, r, greedy)
        cu = catchup_step(shape, w, res["trees"], outs, true_feat_for(r, res), pk, pv, lens, prefix_cap, mirror)
        rounds.append({"res": res, "targets": targets, "verify": outs, "catchup": cu, "prefix_len_in": lens.copy()})
        pk, pv, lens = cu["prefix_k"], cu["prefix_v"], cu["prefix_len"]
        feat, tok = cu["root_feat"], cu["root_token"]
    return rounds
