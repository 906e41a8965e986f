"""Pins for the oracle's draft step (CPU only).

* a tree of chain shape makes tree attention plain causal attention;
* the example tree of the tree-attention section reproduces its visibility table;
* one row of a draft step at the tiny shape is recomputed with scalar loops;
* GQA equals MHA over replicated K/V heads;
* a per-depth chain loop equals one step over the whole chain.
"""
import json
import math
import os

import numpy as np

from oracle import draft as D
from oracle import tree as T
from oracle.numerics import round_bf16
from workloads import CONFIGS, Shape, make_prefix_kv, make_weights, normal_array

from conftest import GOLDEN


def _causal_attention(qs, ks, vs):
    """Textbook causal attention over one head: softmax(QK^T/sqrt(d) + M) V with
    M[i, j] = -inf for j > i."""
    n, hd = qs.shape
    s = qs @ ks.T / np.sqrt(hd)
    s = np.where(np.tril(np.ones((n, n), dtype=bool)), s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ vs


def test_chain_tree_attention_is_causal_attention():
    g = np.random.default_rng(0)
    L, n, H, hd = 7, 5, 2, 8
    pk, pv = g.standard_normal((H, L, hd)), g.standard_normal((H, L, hd))
    ck, cv = g.standard_normal((n, H, hd)), g.standard_normal((n, H, hd))
    q = g.standard_normal((n, H, hd))
    tk = np.full((D.N_SLOTS, H, hd), np.nan)
    tv = np.full((D.N_SLOTS, H, hd), np.nan)
    tk[1:n + 1], tv[1:n + 1] = ck, cv
    for i in range(n):
        mask = sum(1 << s for s in range(1, i + 2))  # chain: all earlier nodes and self
        got = D.tree_attention_row(q[i], pk, pv, L, tk, tv, mask, H, H)
        for h in range(H):
            allk = np.concatenate([pk[h], ck[:, h]])
            allv = np.concatenate([pv[h], cv[:, h]])
            allq = np.concatenate([np.zeros((L, hd)), q[:, h]])
            allq[L + i] = q[i, h]
            ref = _causal_attention(allq, allk, allv)[L + i]
            assert np.allclose(got[h], ref, rtol=0, atol=1e-12)


def test_visibility_table_from_masks():
    with open(os.path.join(GOLDEN, "visibility_table.json")) as f:
        fx = json.load(f)
    parent = fx["parent"]
    names = fx["nodes"]
    # the table's A is the first drafted node; give the tree a root above it
    pool = T.Pool(0, 0)
    ids = {}
    for i, p in enumerate(parent):
        ids[i] = pool.add(0 if p < 0 else ids[p], i, -0.1 * (i + 1))
    tr = T.finalize(pool, 0)
    for t in range(1, len(tr["parent"])):
        vis = [names[int(tr["token"][s])] for s in range(1, len(tr["parent"])) if (int(tr["mask"][t]) >> s) & 1]
        assert sorted(vis) == sorted(fx["visible"][names[int(tr["token"][t])]])
    # and the plain ancestor-set definition agrees
    vs = T.visible_sets(parent)
    for i, nm in enumerate(names):
        assert sorted(names[j] for j in vs[i]) == sorted(fx["visible"][nm])


def _scalar_row(shape, w, fparent, tok, pos, prefix_k, prefix_v, L, anc_k, anc_v, rb=None):
    """One decoder row written with scalar loops only (no vector algebra).
    rb, if given, rounds the activation operand of each weight product."""
    d, H, Hkv, hd, F, V = shape.d, shape.n_heads, shape.n_kv_heads, shape.head_dim, shape.ffn, shape.vocab
    rb = rb or (lambda v: v)
    a = rb([float(fparent[i]) for i in range(d)] + [float(w.embed[tok][i]) for i in range(d)])
    x = []
    for o in range(d):
        s = float(w.fc_b[o])
        for i in range(2 * d):
            s += float(w.fc_w[o][i]) * a[i]
        x.append(s)

    def rms(v, gain):
        ms = sum(t * t for t in v) / len(v)
        r = 1.0 / math.sqrt(ms + shape.rms_eps)
        return [v[i] * r * float(gain[i]) for i in range(len(v))]

    def lin(W, v, nout):
        return [sum(float(W[o][i]) * v[i] for i in range(len(v))) for o in range(nout)]

    def rope(vec):
        half = hd // 2
        out = list(vec)
        for i in range(half):
            ang = pos * shape.rope_theta ** (-2.0 * i / hd)
            c, s = math.cos(ang), math.sin(ang)
            out[i] = vec[i] * c - vec[i + half] * s
            out[i + half] = vec[i + half] * c + vec[i] * s
        return out

    n1 = rb(rms(x, w.norm1))
    q = lin(w.wq, n1, H * hd)
    k = lin(w.wk, n1, Hkv * hd)
    v = lin(w.wv, n1, Hkv * hd)
    qh = [rope(q[h * hd:(h + 1) * hd]) for h in range(H)]
    kh = [rope(k[h * hd:(h + 1) * hd]) for h in range(Hkv)]
    vh = [v[h * hd:(h + 1) * hd] for h in range(Hkv)]
    attn = []
    for h in range(H):
        g = h // (H // Hkv)
        keys = [[float(t) for t in prefix_k[g][j]] for j in range(L)] + [[float(t) for t in ak[g]] for ak in anc_k] + [kh[g]]
        vals = [[float(t) for t in prefix_v[g][j]] for j in range(L)] + [[float(t) for t in av[g]] for av in anc_v] + [vh[g]]
        sc = [sum(qh[h][i] * kk[i] for i in range(hd)) / math.sqrt(hd) for kk in keys]
        mx = max(sc)
        e = [math.exp(s - mx) for s in sc]
        z = sum(e)
        attn += [sum(e[j] / z * vals[j][i] for j in range(len(keys))) for i in range(hd)]
    o = lin(w.wo, rb(attn), d)
    h_res = [x[i] + o[i] for i in range(d)]
    n2 = rb(rms(h_res, w.norm2))
    gt = lin(w.w_gate, n2, F)
    up = lin(w.w_up, n2, F)
    act = [gt[i] / (1.0 + math.exp(-gt[i])) * up[i] for i in range(F)]
    dn = lin(w.w_down, rb(act), d)
    feat = [h_res[i] + dn[i] for i in range(d)]
    fr = rb(feat)
    logits = [sum(float(w.lm_head[t][i]) * fr[i] for i in range(d)) for t in range(V)]
    return np.array(feat), np.array(logits), np.array(kh), np.array(vh)


def _tiny_setup(shape_override=None):
    cfg = CONFIGS[1]
    shape = shape_override or cfg.shape
    import dataclasses
    cfg2 = dataclasses.replace(cfg, shape=shape)
    w = make_weights(cfg2, std=0.2)  # larger weights so every term matters
    lens = np.array([6], dtype=np.int32)
    pk, pv = make_prefix_kv(cfg2, lens)
    return shape, w, lens, pk, pv


def test_draft_row_matches_scalar_loops():
    shape, w, lens, pk, pv = _tiny_setup()
    fparent = normal_array(1, 0, (3, shape.d))
    tk, tv = D.new_tree_kv(shape, 1)
    # a depth-2 row whose depth-1 ancestor sits in slot 3
    anc_k = normal_array(1, 1, (shape.n_kv_heads, shape.head_dim))
    anc_v = normal_array(1, 2, (shape.n_kv_heads, shape.head_dim))
    tk[0, 3], tv[0, 3] = anc_k, anc_v
    rows = dict(seq=[0], token=[77], parent=[2], pos=[7], slot=[5], mask=[(1 << 3) | (1 << 5)])
    out = D.draft_step(shape, w, rows, fparent, pk, pv, lens, tk, tv, mirror=False)
    feat, logits, kh, vh = _scalar_row(shape, w, fparent[2], 77, 7, pk[0], pv[0], 6, [anc_k], [anc_v])
    assert np.allclose(out["feat"][0], feat, rtol=0, atol=1e-10)
    assert np.allclose(out["logits"][0], logits, rtol=0, atol=1e-10)
    assert np.allclose(tk[0, 5], kh, rtol=0, atol=1e-12) and np.allclose(tv[0, 5], vh, rtol=0, atol=1e-12)


def test_draft_row_bf16_operands_match_scalar_loops():
    """act_bf16: the six weight-product operands rounded to bf16, checked
    against the scalar-loop row with torch's own bf16 conversion doing the
    rounding."""
    import torch

    small = Shape(64, 4, 2, 16, 172, 512, dtype="bf16")
    shape, w, lens, pk, pv = _tiny_setup(small)
    fparent = normal_array(1, 0, (3, shape.d))
    tk, tv = D.new_tree_kv(shape, 1)
    anc_k = normal_array(1, 1, (shape.n_kv_heads, shape.head_dim))
    anc_v = normal_array(1, 2, (shape.n_kv_heads, shape.head_dim))
    tk[0, 3], tv[0, 3] = anc_k, anc_v
    rows = dict(seq=[0], token=[77], parent=[2], pos=[7], slot=[5], mask=[(1 << 3) | (1 << 5)])
    out = D.draft_step(shape, w, rows, fparent, pk, pv, lens, tk, tv, mirror=False, act_bf16=True)

    def rb(v):
        return [float(t) for t in torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double()]

    feat, logits, kh, vh = _scalar_row(shape, w, fparent[2], 77, 7, pk[0], pv[0], 6, [anc_k], [anc_v], rb=rb)
    assert np.allclose(out["feat"][0], feat, rtol=0, atol=1e-10)
    assert np.allclose(out["logits"][0], logits, rtol=0, atol=1e-10)
    # and the rounding is felt: the split-operand contract gives other values
    tk2, tv2 = D.new_tree_kv(shape, 1)
    tk2[0, 3], tv2[0, 3] = anc_k, anc_v
    ref = D.draft_step(shape, w, rows, fparent, pk, pv, lens, tk2, tv2, mirror=False)
    assert np.max(np.abs(ref["logits"][0] - logits)) > 1e-4


def test_gqa_equals_mha_with_replicated_kv():
    g = np.random.default_rng(5)
    H, Hkv, hd, L = 4, 2, 8, 5
    q = g.standard_normal((H, hd))
    pk, pv = g.standard_normal((Hkv, L, hd)), g.standard_normal((Hkv, L, hd))
    tk, tv = np.full((64, Hkv, hd), np.nan), np.full((64, Hkv, hd), np.nan)
    tk[0], tv[0] = g.standard_normal((Hkv, hd)), g.standard_normal((Hkv, hd))
    got = D.tree_attention_row(q, pk, pv, L, tk, tv, 1, H, Hkv)
    rep = lambda a, ax: np.repeat(a, H // Hkv, axis=ax)
    ref = D.tree_attention_row(q, rep(pk, 0), rep(pv, 0), L, rep(tk, 1), rep(tv, 1), 1, H, H)
    assert np.allclose(got, ref, rtol=0, atol=1e-14)


def test_chain_loop_equals_one_step_over_chain():
    shape, w, lens, pk, pv = _tiny_setup()
    feat0 = normal_array(1, 3, (1, shape.d))
    toks = [5, 9, 300]
    # per-depth loop: row i uses the previous row's predicted feature
    tk, tv = D.new_tree_kv(shape, 1)
    fb = feat0.astype(np.float64)
    feats = []
    for i, t in enumerate(toks):
        rows = dict(seq=[0], token=[t], parent=[fb.shape[0] - 1], pos=[6 + i], slot=[i + 1],
                    mask=[sum(1 << s for s in range(1, i + 2))])
        o = D.draft_step(shape, w, rows, fb, pk, pv, lens, tk, tv, mirror=False)
        fb = np.concatenate([fb, o["feat"]])
        feats.append(o["feat"][0])
    # one step over the chain, parents taken from the loop's features
    tk2, tv2 = D.new_tree_kv(shape, 1)
    rows = dict(seq=[0] * 3, token=toks, parent=[0, 1, 2], pos=[6, 7, 8], slot=[1, 2, 3],
                mask=[sum(1 << s for s in range(1, i + 2)) for i in range(3)])
    o = D.draft_step(shape, w, rows, fb, pk, pv, lens, tk2, tv2, mirror=False)
    assert np.allclose(o["feat"], np.array(feats), rtol=0, atol=1e-10)


def test_bf16_mirror_rounds_only_the_kv_cache():
    cfg = CONFIGS[2]
    small = Shape(128, 2, 2, 64, 96, 300)
    shape, w, lens, pk, pv = _tiny_setup(small)
    f = round_bf16(normal_array(2, 0, (2, shape.d)))
    tk, tv = D.new_tree_kv(shape, 1)
    rows = dict(seq=[0, 0], token=[1, 2], parent=[0, 1], pos=[6, 6], slot=[1, 2], mask=[2, 4])
    a = D.draft_step(shape, w, rows, f, pk, pv, lens, tk, tv, mirror=True)
    tk2, tv2 = D.new_tree_kv(shape, 1)
    b = D.draft_step(shape, w, rows, f, pk, pv, lens, tk2, tv2, mirror=False)
    # k, v in the slots are bf16 values under the mirror; q and the residual stream are not rounded
    assert np.array_equal(round_bf16(tk[0, 1]), tk[0, 1])
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["q"], b["q"])
    # the readings differ only through the cache rounding, by a little
    assert 0 < np.max(np.abs(a["feat"] - b["feat"])) < 0.05


def test_fuse_features_selecting_the_top_layer_is_eagle_one():
    """With W = [0 | 0 | I] and no bias, the fused feature is the high-layer
    feature itself: EAGLE-3's fusion reduces to EAGLE-1's single feature."""
    d = 8
    g = np.random.default_rng(4)
    low, mid, high = (g.standard_normal((3, d)) for _ in range(3))
    w = np.concatenate([np.zeros((d, d)), np.zeros((d, d)), np.eye(d)], axis=1)
    assert np.array_equal(D.fuse_features(None, w, None, low, mid, high), high)


def test_fuse_features_matches_scalar_loops():
    d = 6
    g = np.random.default_rng(5)
    low, mid, high = (g.standard_normal((2, d)) for _ in range(3))
    w = g.standard_normal((d, 3 * d))
    b = g.standard_normal(d)
    got = D.fuse_features(None, w, b, low, mid, high)
    for r in range(2):
        cat = list(low[r]) + list(mid[r]) + list(high[r])
        for o in range(d):
            want = float(b[o]) + sum(float(w[o][i]) * cat[i] for i in range(3 * d))
            assert abs(got[r, o] - want) < 1e-12
