"""Pins for the oracle's round composition (CPU only): the per-depth draft rows
(tree.assign_rows), the draft phase and tree-wide step (pipeline.draft_phase,
pipeline.tree_wide_rows), and the catch-up / commit between rounds
(pipeline.catchup_rows, pipeline.catchup_step, commit.commit_slots).

* Every per-depth row sits at rotary position L_b + depth - 1 and sees exactly
  its node's ancestors and itself (the visibility rule of the tree-attention
  section of "eagle feature-level speculative decoding"); the same node's row
  in the tree-wide step, built independently from the flattened tree, gives
  the same f^ and logits (within 1e-10).  Planted mistakes in the row builder
  (a dropped ancestor bit, a position off by one, a wrong parent feature) fail
  these checks.
* A chain template through the draft phase equals a hand-built chain loop.
* Catch-up + commit: after a round the drafter's cache equals that of the
  draft layer run as a plain causal decoder over the committed sequence with
  the target's true features, and the next root feature equals that decoder's
  output at the verifier's next token ("eagle feature-level speculative
  decoding", KV commit section: the drafter continues from A-B-X, not from its
  own predicted state).  Planted mistakes in the catch-up rows fail.
* Invalid expansions (NaN values, template counts beyond the ranked tokens)
  give an invalid pool and a root-only tree.
"""
import dataclasses

import numpy as np
import pytest

from oracle import draft as OD
from oracle import pipeline as OP
from oracle import tree as OT
from oracle.numerics import rmsnorm, rope_rotate_half, silu
from workloads import CONFIGS, TEMPLATES, Shape, make_prefix_kv, make_weights, normal_array

TINY = CONFIGS[1]


def _setup(shape, batch, lens, std=0.2):
    cfg = dataclasses.replace(TINY, shape=shape, batch=batch)
    w = make_weights(cfg, std=std)  # larger weights so every term matters
    lens = np.asarray(lens, dtype=np.int32)
    pk, pv = make_prefix_kv(cfg, lens)
    return w, lens, [k.astype(np.float64) for k in pk], [v.astype(np.float64) for v in pv]


def _bits(m):
    return [s for s in range(64) if (int(m) >> s) & 1]


def round_violations(res, lens):
    """Everything the per-depth rows and the tree-wide step of one round must
    satisfy; returns a list of violations (empty = consistent)."""
    bad = []
    pools, trees = res["pools"], res["trees"]
    B = len(pools)
    owner = {}
    for b, pool in enumerate(pools):
        for pid in range(1, len(pool)):
            if pool.feat_row[pid] >= 0:
                owner[pool.feat_row[pid]] = (b, pid)
    base = B
    for st in res["steps"]:
        for i in range(len(st["seq"])):
            b, pid = owner[base + i]
            pool = pools[b]
            if st["seq"][i] != b or st["token"][i] != pool.token[pid]:
                bad.append(("row", base + i))
            if st["parent"][i] != pool.feat_row[pool.parent[pid]]:
                bad.append(("parent", base + i))
            if st["pos"][i] != int(lens[b]) + pool.depth[pid] - 1:
                bad.append(("pos", base + i))
            slot_node = {pool.slot[q]: q for q in range(1, len(pool)) if pool.slot[q] >= 0}
            seen = {slot_node.get(s, -1) for s in _bits(st["mask"][i])}
            anc, a = set(), pid
            while a > 0:
                anc.add(a)
                a = pool.parent[a]
            if seen != anc:
                bad.append(("mask", base + i))
        base += len(st["seq"])
    if "tree_wide" not in res:
        return bad
    tw, twr = res["tree_wide"], res["tree_wide_rows"]
    row = 0
    for b, tr in enumerate(trees):
        vis = OT.visible_sets([int(p) for p in tr["parent"]])
        for t in range(1, len(tr["parent"])):
            if set(_bits(twr["mask"][row])) != {s for s in vis[t] if s > 0}:
                bad.append(("tree-wide mask", b, t))
            pid = int(tr["pool_id"][t])
            fr = pools[b].feat_row[pid]
            if fr >= 0:  # expanded in the per-depth loop: the same row, computed twice
                if np.max(np.abs(res["feat_buf"][fr] - tw["feat"][row])) > 1e-10:
                    bad.append(("feat", b, t))
                if np.max(np.abs(res["logits"][fr] - tw["logits"][row])) > 1e-10:
                    bad.append(("logits", b, t))
            row += 1
    return bad


CASES = {
    "chain5-f32": (TINY.shape, 1, [32], "static", 1, 4, 0, TEMPLATES["chain5"]),
    "static26-f32": (TINY.shape, 1, [11], "static", 4, 5, 0, TEMPLATES["static26"]),
    "eagle2-f32-ragged": (Shape(64, 4, 2, 16, 96, 300, dtype="f32"), 2, [5, 9], "dynamic", 3, 4, 8, None),
    "eagle2-bf16": (Shape(128, 2, 2, 64, 96, 300), 2, [7, 4], "dynamic", 3, 3, 6, None),
}


def _round(name):
    shape, B, lens, kind, k, depth, m, tmpl = CASES[name]
    w, lens, pk, pv = _setup(shape, B, lens)
    feat = normal_array(7, 0, (B, shape.d))
    tok = np.arange(B) + 3
    return OP.draft_phase(shape, w, feat, tok, pk, pv, lens, kind, k, depth, m, tmpl), lens


@pytest.mark.parametrize("name", list(CASES))
def test_per_depth_rows_and_tree_wide_step_agree(name):
    res, lens = _round(name)
    assert res["steps"], "the round drafts at least one decoder step"
    expanded = sum(1 for b, tr in enumerate(res["trees"]) for pid in tr["pool_id"][1:]
                   if res["pools"][b].feat_row[int(pid)] >= 0)
    assert expanded > 0
    assert round_violations(res, lens) == []


def test_planted_row_mistakes_are_caught(monkeypatch):
    real = OT.assign_rows

    def drop_parent_bits(pool, frontier, step, k, static, base, L):
        out = real(pool, frontier, step, k, static, base, L)
        for f, u in enumerate(frontier):
            pool.mask[u] = 1 << pool.slot[u]
        return [(t, p, pos, s, 1 << s) for (t, p, pos, s, m) in out]

    def pos_off_by_one(pool, frontier, step, k, static, base, L):
        return [(t, p, pos + 1, s, m) for (t, p, pos, s, m) in real(pool, frontier, step, k, static, base, L)]

    def root_feature(pool, frontier, step, k, static, base, L):
        return [(t, pool.feat_row[0], pos, s, m) for (t, p, pos, s, m) in real(pool, frontier, step, k, static, base, L)]

    for wrong, kinds in ((drop_parent_bits, {"mask", "feat"}), (pos_off_by_one, {"pos", "feat"}),
                         (root_feature, {"parent", "feat"})):
        monkeypatch.setattr(OT, "assign_rows", wrong)
        res, lens = _round("eagle2-f32-ragged")
        found = {v[0] for v in round_violations(res, lens)}
        assert kinds <= found, (wrong.__name__, found)
    monkeypatch.setattr(OT, "assign_rows", real)

    real_tw = OP.tree_wide_rows

    def tw_pos_shift(trees, pools, prefix_len):
        r = real_tw(trees, pools, prefix_len)
        r["pos"] = [p + 1 for p in r["pos"]]
        return r

    monkeypatch.setattr(OP, "tree_wide_rows", tw_pos_shift)
    res, lens = _round("eagle2-f32-ragged")
    assert "feat" in {v[0] for v in round_violations(res, lens)}


def test_chain_draft_phase_equals_hand_built_chain_loop():
    shape, B, lens, kind, k, depth, m, tmpl = CASES["chain5-f32"]
    w, lens, pk, pv = _setup(shape, B, lens)
    feat = normal_array(7, 0, (1, shape.d))
    res = OP.draft_phase(shape, w, feat, np.array([3]), pk, pv, lens, kind, k, depth, m, tmpl)
    # by hand: node i (depth i) of the chain has token argmax of the previous row, input [f_{i-1} ; e(t_i)],
    # position L + i - 1, slot i, and sees slots 1..i
    L = int(lens[0])
    fb = feat.astype(np.float64)
    logits = OD.head_logits(shape, w, feat, mirror=False)
    tk, tv = OD.new_tree_kv(shape, 1)
    toks = []
    for i in range(1, depth):
        t = int(np.argmax(logits[-1]))
        toks.append(t)
        rows = dict(seq=[0], token=[t], parent=[fb.shape[0] - 1], pos=[L + i - 1], slot=[i],
                    mask=[sum(1 << s for s in range(1, i + 1))])
        o = OD.draft_step(shape, w, rows, fb, pk, pv, lens, tk, tv, mirror=False)
        fb = np.concatenate([fb, o["feat"]])
        logits = np.concatenate([logits, o["logits"]])
    toks.append(int(np.argmax(logits[-1])))
    assert [int(t) for t in res["trees"][0]["token"][1:]] == toks
    assert np.max(np.abs(res["feat_buf"] - fb)) < 1e-10
    assert np.max(np.abs(res["logits"] - logits)) < 1e-10


# ----------------------------------------------------------------- catch-up


def _causal_reference(shape, w, feats, toks):
    """The draft layer as a plain causal decoder over a committed sequence:
    row p = [f_p ; e(t_{p+1})] at rotary position p attends to rows 0..p
    through the textbook causal mask.  Returns rotated k, v [T, Hkv, hd] and
    f^ [T, d] (T = len(toks) - 1)."""
    T = len(toks) - 1
    d, H, Hkv, hd = shape.d, shape.n_heads, shape.n_kv_heads, shape.head_dim
    f = np.asarray(feats, np.float64)
    a = np.concatenate([f[:T], np.asarray(w.embed, np.float64)[np.asarray(toks[1:])]], axis=1)
    x = a @ np.asarray(w.fc_w, np.float64).T + np.asarray(w.fc_b, np.float64)
    n1 = rmsnorm(x, w.norm1, shape.rms_eps)
    q = (n1 @ np.asarray(w.wq, np.float64).T).reshape(T, H, hd)
    k = (n1 @ np.asarray(w.wk, np.float64).T).reshape(T, Hkv, hd)
    v = (n1 @ np.asarray(w.wv, np.float64).T).reshape(T, Hkv, hd)
    for p in range(T):
        q[p] = [rope_rotate_half(q[p, h], p, shape.rope_theta) for h in range(H)]
        k[p] = [rope_rotate_half(k[p, h], p, shape.rope_theta) for h in range(Hkv)]
    causal = np.tril(np.ones((T, T), dtype=bool))
    att = np.zeros((T, H, hd))
    for h in range(H):
        g = h // (H // Hkv)
        s = q[:, h] @ k[:, g].T / np.sqrt(hd)
        s = np.where(causal, s, -np.inf)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        att[:, h] = (e / e.sum(axis=1, keepdims=True)) @ v[:, g]
    hres = x + att.reshape(T, H * hd) @ np.asarray(w.wo, np.float64).T
    n2 = rmsnorm(hres, w.norm2, shape.rms_eps)
    act = silu(n2 @ np.asarray(w.w_gate, np.float64).T) * (n2 @ np.asarray(w.w_up, np.float64).T)
    return k, v, hres + act @ np.asarray(w.w_down, np.float64).T


def _catchup_case(shape, L0, D, A):
    """A committed sequence, its causal reference, and one round's chain tree
    rooted at position L0 whose first A drafted nodes were accepted."""
    w, _, _, _ = _setup(shape, 1, [1])
    T = L0 + D + 2
    toks = [int(t) for t in np.random.default_rng(L0 * 100 + A).integers(0, shape.vocab, T + 1)]
    feats = normal_array(9, L0, (T + 1, shape.d)).astype(np.float64)
    rk, rv, rf = _causal_reference(shape, w, feats, toks)
    prefix_k = [np.transpose(rk[:L0], (1, 0, 2)).copy()]
    prefix_v = [np.transpose(rv[:L0], (1, 0, 2)).copy()]
    N = D + 1  # chain: node n at sequence position L0 + n
    tree = {"token": np.array(toks[L0:L0 + N]), "parent": np.arange(-1, N - 1)}
    path = list(range(1, A + 1)) + [-1] * (N - A)
    out = {"path": path, "accept_len": A + 1, "next_token": toks[L0 + A + 1]}
    true_feat = feats[L0:L0 + N]
    return w, rk, rv, rf, prefix_k, prefix_v, tree, out, true_feat


@pytest.mark.parametrize("shape", [TINY.shape, Shape(64, 4, 2, 16, 96, 300, dtype="f32")])
@pytest.mark.parametrize("A", [0, 2, 4])
def test_catchup_commit_equals_causal_drafter(shape, A):
    L0, D = 6, 4
    w, rk, rv, rf, pk, pv, tree, out, tf = _catchup_case(shape, L0, D, A)
    cu = OP.catchup_step(shape, w, [tree], [out], tf, pk, pv, np.array([L0]), np.array([L0 + D + 1]), mirror=False)
    n = L0 + A + 1
    assert cu["flags"] == [0] and int(cu["prefix_len"][0]) == n
    assert np.max(np.abs(cu["prefix_k"][0] - np.transpose(rk[:n], (1, 0, 2)))) < 1e-10
    assert np.max(np.abs(cu["prefix_v"][0] - np.transpose(rv[:n], (1, 0, 2)))) < 1e-10
    # the next round's root: the decoder's output at the verifier's next token (position L0 + A + 1)
    assert np.max(np.abs(cu["root_feat"][0] - rf[n - 1])) < 1e-10
    assert int(cu["root_token"][0]) == out["next_token"]


def test_planted_catchup_mistakes_are_caught(monkeypatch):
    shape, L0, D, A = TINY.shape, 6, 4, 3
    real = OP.catchup_rows
    wrongs = [
        lambda *a: [(t, p + 1, pos, s, m) for (t, p, pos, s, m) in real(*a)],  # the node's own feature
        lambda *a: [(t, p, pos + 1, s, m) for (t, p, pos, s, m) in real(*a)],  # position off by one
        lambda *a: [(t, p, pos, s, 1 << s) for (t, p, pos, s, m) in real(*a)],  # earlier rows not seen
    ]
    for wrong in wrongs:
        monkeypatch.setattr(OP, "catchup_rows", wrong)
        w, rk, rv, rf, pk, pv, tree, out, tf = _catchup_case(shape, L0, D, A)
        tf = np.concatenate([tf, tf[-1:]])  # room for a shifted parent row
        cu = OP.catchup_step(shape, w, [tree], [out], tf, pk, pv, np.array([L0]), np.array([L0 + D + 1]),
                             mirror=False)
        n = L0 + A + 1
        err = max(np.max(np.abs(cu["prefix_k"][0] - np.transpose(rk[:n], (1, 0, 2)))),
                  np.max(np.abs(cu["root_feat"][0] - rf[n - 1])))
        assert err > 1e-6


def test_commit_slots_special_cases():
    from oracle.commit import BAD_PATH, OVERFLOW, commit_slots
    pk = [np.zeros((2, 3, 4)), np.ones((2, 5, 4))]
    tk = np.arange(2 * 64 * 2 * 4, dtype=np.float64).reshape(2, 64, 2, 4)
    k, v, lens, flags = commit_slots(pk, pk, [3, 5], [5, 6], tk, tk, [2, 2])
    assert flags == [0, OVERFLOW] and lens == [5, 5]
    assert np.array_equal(k[0][:, 3], tk[0, 0]) and np.array_equal(k[0][:, 4], tk[0, 1])
    assert np.array_equal(k[1], pk[1])
    _, _, lens, flags = commit_slots(pk, pk, [3, 5], None, tk, tk, [0, 65])
    assert flags == [0, BAD_PATH] and lens == [3, 5]


def test_decode_rounds_chain_the_rounds():
    """Three rounds at the tiny workload: each round's prefix grows by its
    accepted length (accepted drafts + the next token), its root is the
    previous round's next token, and its depth-1 rows sit right after the
    grown prefix."""
    shape, B, lens0, kind, k, depth, m, tmpl = CASES["static26-f32"]
    w, lens, pk, pv = _setup(shape, B, lens0)
    N = len(tmpl)

    def target_for(r, res):
        tw = res["tree_wide"]["logits"]
        noise = normal_array(11, r, (N, shape.vocab), 0.5)
        root = res["logits"][0] if r == 0 else res["logits"][0] + noise[0]
        return [np.concatenate([root[None], tw[:N - 1] + noise[1:]]).astype(np.float32)]

    def true_feat_for(r, res):
        f = normal_array(12, r, (N, shape.d)).astype(np.float64)
        if r == 0:
            f[0] = res["feat_buf"][0]  # the first round's root feature is the true one
        return f

    feat = normal_array(7, 0, (1, shape.d))
    rounds = OP.decode_rounds(shape, w, feat, np.array([3]), pk, pv, lens, np.array([lens[0] + 20]), kind, k, depth,
                              m, tmpl, 3, target_for, true_feat_for)
    L = int(lens[0])
    for r, rd in enumerate(rounds):
        assert int(rd["prefix_len_in"][0]) == L
        steps = rd["res"]["steps"]
        assert all(p == L for p in steps[0]["pos"])  # depth-1 rows at the round's first new position
        if r:
            assert int(rd["res"]["trees"][0]["token"][0]) == rounds[r - 1]["verify"][0]["next_token"]
        assert rd["catchup"]["flags"] == [0]
        L += rd["verify"][0]["accept_len"]
        assert int(rd["catchup"]["prefix_len"][0]) == L


def test_nan_values_and_oversized_templates_invalidate_the_pool():
    pool = OT.Pool(3, 0)
    nxt = OT.expand(pool, [0], [[5, 6, 7]], [[np.float32(-0.1), np.float32(np.nan), np.float32(-2)]], 3)
    assert nxt == [] and pool.invalid and len(pool) == 1
    assert [int(p) for p in OT.finalize(pool, 2)["parent"]] == [-1]
    # a template node asking for more children than its row ranks
    pool = OT.Pool(3, 0)
    nchild = np.array([3, 0, 0, 0])
    assert OT.expand(pool, [0], [[5, 6]], [[np.float32(-0.1), np.float32(-0.2)]], 2, nchild) == []
    assert pool.invalid and [int(p) for p in OT.finalize(pool, 0)["parent"]] == [-1]
    # a valid pool keeps growing
    pool = OT.Pool(3, 0)
    assert OT.expand(pool, [0], [[5, 6]], [[np.float32(-0.1), np.float32(-0.2)]], 2) == [1, 2]
    assert not pool.invalid
