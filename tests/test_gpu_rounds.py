"""Several rounds with the drafter's catch-up between them, through the C ABI.

After verification the drafter continues from the committed path ("eagle
feature-level speculative decoding", KV commit section: with A-B-D drafted
and A-B-X committed, the drafter goes on from A-B-X, not from D's predicted
state; "EAGLE 推测解码为什么比 Medusa 快" section 6.2: the accepted path's true
features start the next round).  eagle_catchup_rows + a features-only draft
step + eagle_commit_catchup rebuild the drafter's rows over the committed
tokens from the target's true features, commit their k, v to the prefix, and
hand the next round its root feature.

* tiny fp32 chain workload: three free-running rounds on the GPU equal the
  oracle's multi-round decode from the same seeded inputs (floats 1e-4; trees,
  decisions, commits exactly);
* 7B static-26 workload: three rounds, every stage checked against the oracle
  from the GPU's own inputs to that stage: catch-up rows bit-exact (with the
  documented padding), the catch-up's f^ within 2e-2, the committed cache
  bit-exact against the oracle's commit of the GPU's slots and within one bf16
  step of the oracle's own k, v from the true features (k, v computed from the
  draft's predicted features would be far off), the next round's first draft
  step attending to the grown cache within 2e-2, verification bit-exact.
The target's tree forward is not part of this path: its features at the tree
nodes are seeded N(0, 1) draws (workloads.make_true_features) and its logits
are the tree-wide draft logits plus N(0, 0.5) noise (the root row copies the
draft root row in the first round, whose root feature is the true one).
"""
import numpy as np
import pytest
import torch

import eagle_feature_level_amd as E
from eagle_feature_level_amd.engine import EagleRound
from oracle import draft as OD
from oracle import pipeline as OP
from oracle.commit import commit_slots
from workloads import (CONFIGS, TEMPLATES, make_prefix_kv, make_prefix_lens, make_root_features, make_root_tokens,
                       make_target_noise, make_true_features, make_weights)
from workloads import device as dev

pytestmark = pytest.mark.gpu


def _np(t):
    return t.detach().cpu().numpy()


def _setup(cid, extra):
    cfg = CONFIGS[cid]
    s = cfg.shape
    w = make_weights(cfg)
    lens = make_prefix_lens(cfg)
    ks, vs = make_prefix_kv(cfg, lens)
    pf = dev.prefix(ks, vs, lens, s.dtype, extra=extra)
    kind = "dynamic" if cfg.tree == "dynamic" else "static"
    eng = EagleRound(dev.shape_dict(s), dev.weights(w, s.dtype), cfg.batch, kind, cfg.topk, cfg.depth, cfg.rerank_m,
                     TEMPLATES.get(cfg.tree), pf)
    return cfg, eng, w, lens, ks, vs, pf


def _target_np(cfg, r, root_logits, tw_logits, N):
    """Round r's target logits [B*N, V] from the round's draft logits."""
    B, V = cfg.batch, cfg.shape.vocab
    noise = make_target_noise(cfg, B * N, sub=r).reshape(B, N, V)
    tgt = np.empty((B, N, V), np.float32)
    tgt[:, 1:] = tw_logits[:B * (N - 1)].reshape(B, N - 1, V) + noise[:, 1:]
    tgt[:, 0] = root_logits[:B] if r == 0 else root_logits[:B] + noise[:, 0]
    return tgt.reshape(B * N, V)


def _true_feat_np(cfg, r, N, root_feat):
    f = make_true_features(cfg, r, cfg.batch * N).astype(np.float64)
    if r == 0:
        f.reshape(cfg.batch, N, -1)[:, 0] = root_feat  # the first round's root feature is the true one
    return f


def _prefix_blocks(pf, lens_cap, H, hd):
    off = _np(pf["off"])
    k, v = _np(pf["k"].float()), _np(pf["v"].float())
    return ([k[off[b]:off[b] + H * C * hd].reshape(H, C, hd) for b, C in enumerate(lens_cap)],
            [v[off[b]:off[b] + H * C * hd].reshape(H, C, hd) for b, C in enumerate(lens_cap)])


def _padded_rows(want, A, b, R):
    """The documented fixed-shape layout: rows past A repeat row A in their own slot."""
    out = []
    for i in range(R):
        tok, par, pos, _, _ = want[min(i, A)]
        r_ = min(i, A)
        out.append((tok, par, pos, i, ((1 << r_) - 1) | (1 << i)))
    return out


def test_tiny_rounds_free_running_match_oracle_decode():
    cfg = CONFIGS[1]
    extra = 3 * (cfg.depth + 1)
    cfg, eng, w, lens, ks, vs, pf = _setup(1, extra)
    s, B, N = cfg.shape, cfg.batch, eng.n_nodes
    feat = make_root_features(cfg)
    tok = make_root_tokens(cfg)
    n_rounds = 3

    def target_for(r, res):
        return list(_target_np(cfg, r, res["logits"][:B], res["tree_wide"]["logits"], N).reshape(B, N, -1))

    def true_feat_for(r, res):
        return _true_feat_np(cfg, r, N, res["feat_buf"][:B])

    ref = OP.decode_rounds(s, w, feat, tok, ks, vs, lens, lens + extra, "static", cfg.topk, cfg.depth, 0,
                           TEMPLATES[cfg.tree], n_rounds, target_for, true_feat_for)
    root_f, root_t = torch.from_numpy(feat).cuda(), dev.ints(tok)
    for r in range(n_rounds):
        rd = ref[r]
        eng.draft_phase(root_f, root_t)
        eng.tree_wide()
        torch.cuda.synchronize()
        lg = rd["res"]["logits"]
        gaps = [np.sort(lg[i])[-1] - np.sort(lg[i])[-2] for i in range(lg.shape[0])]
        if min(gaps) < 2.5e-4:
            pytest.skip(f"oracle top-1 near-tie in round {r}")
        assert np.max(np.abs(_np(eng.logits) - lg)) < 1e-4, r
        assert list(_np(eng.tree["token"])) == list(rd["res"]["trees"][0]["token"]), r
        tgt = _target_np(cfg, r, _np(eng.logits), _np(eng.tw_logits), N)
        eng.verify(torch.from_numpy(tgt).cuda(), 0, r)
        torch.cuda.synchronize()
        want = rd["verify"][0]
        if (want["margins"] and min(want["margins"]) < 1e-4) or want["draw_margin"] < 1e-4:
            pytest.skip(f"verification near-tie in round {r}")
        assert int(eng.v_len[0]) == want["accept_len"] and int(eng.v_next[0]) == want["next_token"], r
        tf = _true_feat_np(cfg, r, N, _np(eng.feat[:B]).astype(np.float64))
        eng.catch_up(torch.from_numpy(tf.astype(np.float32)).cuda())
        torch.cuda.synchronize()
        cu = rd["catchup"]
        assert list(_np(eng.c_flags)) == cu["flags"] == [0] * B
        assert list(_np(pf["len"])) == list(cu["prefix_len"]), r
        assert np.max(np.abs(_np(eng.feat[:B]) - cu["root_feat"])) < 1e-4, r
        gk, gv = _prefix_blocks(pf, lens + extra, s.n_kv_heads, s.head_dim)
        n = int(cu["prefix_len"][0])
        assert np.max(np.abs(gk[0][:, :n] - cu["prefix_k"][0])) < 1e-4
        assert np.max(np.abs(gv[0][:, :n] - cu["prefix_v"][0])) < 1e-4
        root_f, root_t = eng.next_round_inputs()
        assert int(root_t[0]) == want["next_token"]


def _bf16_step(x):
    """One bf16 unit in the last place of |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 1e-30)
    return np.exp2(np.floor(np.log2(a)) - 7)


def test_rounds_with_catchup_7b_staged():
    cfg = CONFIGS[2]
    extra = 3 * (cfg.depth + 1)
    cfg, eng, w, lens, ks, vs, pf = _setup(2, extra)
    s, B, N, R = cfg.shape, cfg.batch, eng.n_nodes, eng.cu_R
    caps = lens + extra
    pk = [k.astype(np.float64) for k in ks]
    pv = [v.astype(np.float64) for v in vs]
    plen = np.array(lens, dtype=np.int64)
    feat = make_root_features(cfg)
    root_f, root_t = torch.from_numpy(feat).cuda(), dev.ints(make_root_tokens(cfg))
    prev_next = None
    accepted = []
    for r in range(3):
        eng.draft_phase(root_f, root_t)
        eng.tree_wide()
        torch.cuda.synchronize()
        # the round starts where the last one left off
        st = eng.steps[0]
        assert all(int(p) == int(plen[0]) for p in _np(st.pos)), r
        if prev_next is not None:
            assert int(_np(eng.tree["token"])[0]) == prev_next
        fb = _np(eng.feat).astype(np.float64)
        ref = OD.head_logits(s, w, fb[:B])
        assert np.max(np.abs(_np(eng.logits[:B]) - ref)) < 2e-2, r
        # first per-depth step, attending to the (grown) cache: every row against the oracle
        n = B * st.n_next
        rows = dict(seq=[0] * n, token=_np(st.token).astype(np.int64), parent=_np(st.parent).astype(np.int64),
                    pos=_np(st.pos).astype(np.int64), slot=_np(st.slot).astype(np.int64),
                    mask=_np(st.mask).view(np.uint64))
        tk, tv = OD.new_tree_kv(s, B)
        ref = OD.draft_step(s, w, rows, fb, pk, pv, plen, tk, tv, mirror=True)
        assert np.max(np.abs(fb[st.feat_row0:st.feat_row0 + n] - ref["feat"])) < 2e-2, r
        assert np.max(np.abs(_np(eng.logits[st.feat_row0:st.feat_row0 + n]) - ref["logits"])) < 2e-2, r
        # verification, bit-exact on the GPU's fp32 logits
        tgt = _target_np(cfg, r, _np(eng.logits), _np(eng.tw_logits), N)
        eng.verify(torch.from_numpy(tgt).cuda(), 0, r)
        torch.cuda.synchronize()
        tree = {"parent": _np(eng.tree["parent"]), "token": _np(eng.tree["token"])}
        qrow = _np(eng.tree["qrow"]).astype(np.int64)
        want = OP.verify_all([tree], [tgt], _np(eng.logits), [qrow], 0, r)[0]
        path, alen, vnext = _np(eng.v_path), _np(eng.v_len), _np(eng.v_next)
        if not ((want["margins"] and min(want["margins"]) < 1e-5) or want["draw_margin"] < 3e-6):
            assert int(alen[0]) == want["accept_len"] and list(path[:alen[0] - 1]) == want["path"], r
            assert int(vnext[0]) == want["next_token"], r
        accepted.append(int(alen[0]) - 1)
        # catch-up
        tf = _true_feat_np(cfg, r, N, fb[:B])
        eng.catch_up(torch.from_numpy(tf.astype(np.float32)).cuda())
        torch.cuda.synchronize()
        c = {k_: _np(v_) for k_, v_ in eng.cu.items()}
        outs = [dict(path=list(path[b * N:(b + 1) * N]), accept_len=int(alen[b]), next_token=int(vnext[b]))
                for b in range(B)]
        for b in range(B):
            A = outs[b]["accept_len"] - 1
            want_rows = OP.catchup_rows(tree["token"][b * N:(b + 1) * N], outs[b]["path"], A + 1,
                                        outs[b]["next_token"], plen[b], b * N)
            got = [(int(c["token"][i]), int(c["parent"][i]), int(c["pos"][i]), int(c["slot"][i]),
                    int(c["mask"][i:i + 1].view(np.uint64)[0])) for i in range(b * R, (b + 1) * R)]
            assert got == _padded_rows(want_rows, A, b, R), (r, b)
            assert int(c["last_row"][b]) == b * R + A and int(c["count"][b]) == A + 1
        assert list(c["row_start"]) == [b * R for b in range(B + 1)]
        # the oracle's catch-up from the true features, on the oracle's view of the cache
        cu = OP.catchup_step(s, w, [{"token": tree["token"][b * N:(b + 1) * N]} for b in range(B)], outs, tf, pk, pv,
                             plen, caps, mirror=True)
        real = [b * R + i for b in range(B) for i in range(outs[b]["accept_len"])]
        assert np.max(np.abs(_np(eng.cu_feat)[real] - cu["out"]["feat"])) < 2e-2, r
        # the committed cache: the GPU's own slots appended bit for bit ...
        gslot_k = _np(eng.tree_k.float()).astype(np.float64)
        gslot_v = _np(eng.tree_v.float()).astype(np.float64)
        counts = [o["accept_len"] for o in outs]
        ok_, ov_, olen, oflags = commit_slots(pk, pv, plen, caps, gslot_k, gslot_v, counts)
        assert list(_np(eng.c_flags)) == oflags == [0] * B
        assert list(_np(pf["len"])) == list(olen), r
        gk, gv = _prefix_blocks(pf, caps, s.n_kv_heads, s.head_dim)
        for b in range(B):
            Ln = olen[b]
            assert np.array_equal(gk[b][:, :Ln], ok_[b]) and np.array_equal(gv[b][:, :Ln], ov_[b]), (r, b)
            assert not gk[b][:, Ln:].any() and not gv[b][:, Ln:].any()  # the room past the length is untouched
            # ... and within one bf16 step (plus the fp32 accumulation error of the products, ~1e-4 at
            # d = 4096) of the oracle's k, v computed from the true features
            for got_, ref_ in ((gk[b][:, plen[b]:Ln], cu["prefix_k"][b][:, plen[b]:Ln]),
                               (gv[b][:, plen[b]:Ln], cu["prefix_v"][b][:, plen[b]:Ln])):
                excess = np.abs(got_ - ref_) - _bf16_step(np.maximum(np.abs(got_), np.abs(ref_)))
                print(f"round {r}: committed k/v beyond one bf16 step by at most {excess.max():.2e}")
                assert excess.max() <= 1e-3, r
        # the next round's root: the catch-up's f^ of the next token's row
        assert np.array_equal(_np(eng.feat[:B]), _np(eng.cu_feat)[c["last_row"]])
        assert np.max(np.abs(_np(eng.feat[:B]) - cu["root_feat"])) < 2e-2
        pk, pv, plen = ok_, ov_, np.array(olen, dtype=np.int64)
        prev_next = int(vnext[0])
        root_f, root_t = eng.next_round_inputs()
    assert accepted[0] >= 1  # the first round's root child is always accepted (q == p)
    print("accepted drafts per round:", accepted)


def test_catchup_malformed_and_overflow_flags():
    """A verification result with an out-of-range path node is flagged
    malformed (count -1: nothing committed, rows of A = 0); a commit beyond the
    capacity is flagged and leaves the cache as it was."""
    cfg = CONFIGS[1]
    cfg, eng, w, lens, ks, vs, pf = _setup(1, 2)
    B, N, R = cfg.batch, eng.n_nodes, eng.cu_R
    i32 = dict(dtype=torch.int32, device="cuda")
    tok = torch.arange(N, **i32) + 5
    c = {k_: torch.full_like(v_, -9) for k_, v_ in eng.cu.items()}
    path = torch.tensor([1, 9, -1, -1, -1], **i32)  # node 9 does not exist
    E.eagle_catchup_rows(B, N, R - 1, tok, path, torch.tensor([3], **i32), torch.tensor([77], **i32), pf["len"], 0,
                         c["token"], c["parent"], c["pos"], c["slot"], c["mask"], c["row_start"], c["last_row"],
                         c["count"])
    torch.cuda.synchronize()
    assert int(c["count"][0]) == -1 and int(c["last_row"][0]) == 0
    assert list(_np(c["token"])) == [77] * R and list(_np(c["pos"])) == [int(lens[0])] * R
    assert list(_np(c["mask"]).view(np.uint64)) == [1 << i for i in range(R)]
    flags = torch.full((B,), -1, **i32)
    k0 = pf["k"].clone()
    E.eagle_commit_catchup(eng.shape, B, c["count"], eng.tree_k, eng.tree_v, pf["k"], pf["v"], pf["off"], pf["len"],
                           pf["cap"], None, None, None, flags)
    torch.cuda.synchronize()
    assert int(flags[0]) == E.EAGLE_COMMIT_BAD_PATH and int(pf["len"][0]) == int(lens[0])
    # room for 2 positions, 4 asked
    E.eagle_commit_catchup(eng.shape, B, torch.tensor([4], **i32), eng.tree_k, eng.tree_v, pf["k"], pf["v"],
                           pf["off"], pf["len"], pf["cap"], None, None, None, flags)
    torch.cuda.synchronize()
    assert int(flags[0]) == E.EAGLE_COMMIT_OVERFLOW and int(pf["len"][0]) == int(lens[0])
    assert torch.equal(pf["k"], k0)


def test_commit_with_node_slots_matches_oracle():
    """eagle_commit with an explicit node -> slot map (the accepted nodes' k, v
    held in other slots than their tree index) appends the right slots."""
    from oracle.commit import commit as o_commit
    cfg = CONFIGS[2]
    cfg, eng, w, lens, ks, vs, pf = _setup(2, 8)
    s, B = cfg.shape, cfg.batch
    N = 6
    g = np.random.default_rng(3)
    tk = torch.from_numpy(g.standard_normal((B, 64, s.n_kv_heads, s.head_dim)).astype(np.float32)).to(torch.bfloat16)
    tv = torch.from_numpy(g.standard_normal((B, 64, s.n_kv_heads, s.head_dim)).astype(np.float32)).to(torch.bfloat16)
    tk, tv = tk.cuda(), tv.cuda()
    path = np.array([[2, 4, 5, -1, -1, -1]], dtype=np.int32)
    slots = np.array([[-1, 40, 17, 63, 3, 9]], dtype=np.int32)
    i32 = dict(dtype=torch.int32, device="cuda")
    flags = torch.full((B,), -1, **i32)
    E.eagle_commit(eng.shape, B, N, torch.from_numpy(path).cuda(), torch.tensor([4], **i32),
                   torch.from_numpy(slots).cuda(), tk, tv, pf["k"], pf["v"], pf["off"], pf["len"], pf["cap"], flags)
    torch.cuda.synchronize()
    want_k, want_v, want_len, want_flags = o_commit([k.astype(np.float64) for k in ks],
                                                    [v.astype(np.float64) for v in vs], lens, lens + 8,
                                                    _np(tk.float()).astype(np.float64),
                                                    _np(tv.float()).astype(np.float64), [list(path[0])], [4],
                                                    [list(slots[0])])
    assert list(_np(flags)) == want_flags == [0] and list(_np(pf["len"])) == want_len == [int(lens[0]) + 3]
    gk, gv = _prefix_blocks(pf, lens + 8, s.n_kv_heads, s.head_dim)
    assert np.array_equal(gk[0][:, :want_len[0]], want_k[0]) and np.array_equal(gv[0][:, :want_len[0]], want_v[0])
