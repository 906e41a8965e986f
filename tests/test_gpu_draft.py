"""GPU parity of eagle_softmax_topk and eagle_draft_step against the fp64 oracle.

Float outputs within max-abs 2e-2 (bf16) / 1e-4 (fp32); top-k indices
bit-exact on identical fp32 logits (ties -> lower index, -0.0 == +0.0).
Inputs are seeded and synthetic; shapes span several GEMM tiles, the skinny
(M <= 32) and tiled kernels, GQA, ragged prefixes (including empty) and a
ragged K/V tail."""
import dataclasses

import numpy as np
import pytest
import torch

import eagle_feature_level_amd as E
from oracle import draft as OD
from oracle.topk import softmax_topk as o_topk
from workloads import CONFIGS, Shape, bf16_values, make_prefix_kv, make_weights, normal_array, uniform_ints
from workloads import device as dev

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


def _ws(nbytes):
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("rows,vocab,k", [(1, 32000, 10), (7, 32000, 4), (33, 4096, 16), (200, 32000, 10),
                                          (3, 512, 1), (961, 32000, 10), (3, 50000, 16), (4, 32768, 10)])
def test_softmax_topk_bit_exact(rows, vocab, k):
    g = np.random.default_rng(rows * 7 + k)
    x = (g.standard_normal((rows, vocab)) * 2).astype(np.float32)
    # adversarial: quantised values (many ties), -0.0 / +0.0 pairs, a plateau at the top
    x[::3] = np.round(x[::3] * 2) / 2
    x[0, :40] = 3.5
    x[0, 100] = -0.0
    x[0, 5] = 0.0
    if rows > 1:
        x[1, :] = -0.0
        x[1, 7] = 0.0
    if rows > 2 and vocab >= 4096 * 8:
        # the 32 largest values all in the stride-4096 share of one float4 column
        cols = (8 + 4096 * np.arange(8)[:, None] + np.arange(4)).ravel()
        x[2, cols] = 10.0 + np.arange(32, dtype=np.float32) % 5
    t = torch.from_numpy(x).cuda()
    lse = torch.empty(rows, device="cuda")
    idx = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    lq = torch.empty(rows, k, device="cuda")
    shape = E.make_shape(256, 2, 2, 128, 256, vocab)
    ws = _ws(E.eagle_workspace_bytes(shape, rows, 1, 0))
    E.eagle_softmax_topk(rows, vocab, t, k, lse, idx, lq, ws)
    torch.cuda.synchronize()
    o_lse, o_idx, o_lq = o_topk(x, k)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert np.allclose(lse.cpu().numpy(), o_lse, rtol=1e-6, atol=1e-5)
    assert np.allclose(lq.cpu().numpy(), o_lq, rtol=0, atol=2e-5)


def _setup(shape: Shape, batch, lens, seed, std=0.05):
    cfg = dataclasses.replace(CONFIGS[2] if shape.dtype == "bf16" else CONFIGS[1], cid=100 + seed, shape=shape,
                              batch=batch)
    w = make_weights(cfg, std=std)
    ks, vs = make_prefix_kv(cfg, np.asarray(lens))
    return cfg, w, ks, vs


def _rows(cfg, counts, lens, seed, n_feat):
    """Random tree rows: per sequence `counts[b]` rows with distinct slots; each
    row sees a random subset of earlier slots (pre-filled or from this call) and
    itself."""
    g = np.random.default_rng(1000 + seed)
    V = cfg.shape.vocab
    rows = {k: [] for k in ("seq", "token", "parent", "pos", "slot", "mask")}
    start = [0]
    for b, c in enumerate(counts):
        slots = g.choice(np.arange(8, 64), size=c, replace=False)
        for i in range(c):
            pre = g.choice(8, size=int(g.integers(0, 4)), replace=False)  # pre-filled slots 0..7
            mine = [int(s) for s in slots[:i] if g.random() < 0.5]
            mask = int(sum(1 << int(s) for s in pre)) | int(sum(1 << s for s in mine)) | (1 << int(slots[i]))
            rows["seq"].append(b)
            rows["token"].append(int(g.integers(0, V)))
            rows["parent"].append(int(g.integers(0, n_feat)))
            rows["pos"].append(int(lens[b]) + int(g.integers(0, 6)))
            rows["slot"].append(int(slots[i]))
            rows["mask"].append(mask)
        start.append(start[-1] + c)
    return rows, start


def _run_draft(shape, counts, lens, seed, head_only=False, topk=4, act=False, std=0.05, blocked=False, oracle=True):
    cfg, w, ks, vs = _setup(shape, len(counts), lens, seed, std=std)
    B = len(counts)
    n_feat = 9
    feat = normal_array(200 + seed, 0, (n_feat, shape.d))
    if shape.dtype == "bf16":
        feat = bf16_values(feat)
    rows, start = _rows(cfg, counts, lens, seed, n_feat)
    M = len(rows["seq"])
    hkv, hd = shape.n_kv_heads, shape.head_dim
    # pre-filled tree slots 0..7 of every sequence
    tk0 = normal_array(300 + seed, 0, (B, 64, hkv, hd))
    tv0 = normal_array(300 + seed, 1, (B, 64, hkv, hd))
    if shape.dtype == "bf16":
        tk0, tv0 = bf16_values(tk0), bf16_values(tv0)
    wt = dev.weights(w, shape.dtype)
    pf = dev.prefix(ks, vs, lens, shape.dtype)
    tree_k = dev.tensor(tk0.reshape(-1), shape.dtype).view(B, 64, hkv, hd)
    tree_v = dev.tensor(tv0.reshape(-1), shape.dtype).view(B, 64, hkv, hd)
    es = E.make_shape(**dev.shape_dict(shape))
    if blocked:
        for n in ("fc_w", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down", "lm_head"):
            t = wt[n]
            r_, c_ = t.shape[0], t.numel() // t.shape[0]
            wt[n + "_b"] = torch.empty(E.eagle_blocked_weight_bytes(r_, c_), dtype=torch.uint8, device="cuda")
            E.eagle_block_weight(t, r_, c_, wt[n + "_b"])
    ew = E.make_weights(wt)
    t_rows = {k: dev.ints(rows[k]) for k in ("token", "parent", "pos", "slot")}
    t_mask = dev.masks(rows["mask"])
    t_start = dev.ints(start)
    er = E.make_rows(M, B, max(counts), t_start, t_rows["token"], t_rows["parent"], t_rows["pos"], t_rows["slot"],
                     t_mask)
    kv = E.make_kv(pf["k"], pf["v"], pf["off"], pf["len"], pf["max_len"], tree_k, tree_v)
    f_in = torch.from_numpy(feat).cuda()
    o_feat = torch.full((M, shape.d), float("nan"), device="cuda")
    o_log = torch.full((M, shape.vocab), float("nan"), device="cuda")
    o_lse = torch.empty(M, device="cuda")
    o_idx = torch.empty(M, topk, dtype=torch.int32, device="cuda")
    o_lq = torch.empty(M, topk, device="cuda")
    out = E.make_out(o_feat, o_log, o_lse, topk, o_idx, o_lq)
    ws = _ws(E.eagle_workspace_bytes(es, M, B, pf["max_len"]))
    ws.fill_(0xFF)  # poisoned workspace: every value read must have been written in this call
    flags = (E.EAGLE_HEAD_ONLY if head_only else 0) | (E.EAGLE_ACT_BF16 if act else 0)
    E.eagle_draft_step(es, ew, flags, er, f_in, kv, out, ws)
    torch.cuda.synchronize()
    gpu = dict(logits=o_log.cpu().numpy(), feat=o_feat.cpu().numpy(), idx=o_idx.cpu().numpy(),
               lse=o_lse.cpu().numpy(), tree_k=tree_k.float().cpu().numpy(), tree_v=tree_v.float().cpu().numpy())
    if not oracle:
        return None, gpu, rows, None, None
    # oracle
    tk, tv = tk0.astype(np.float64).copy(), tv0.astype(np.float64).copy()
    if head_only:
        from oracle.draft import head_logits
        ref = {"logits": head_logits(shape, w, feat[rows["parent"]], act_bf16=act)}
    else:
        ref = OD.draft_step(shape, w, rows, feat, ks, vs, lens, tk, tv, mirror=True, act_bf16=act)
    return ref, gpu, rows, tk, tv


def _check_topk_valid(ref_logits, gpu_idx, tol):
    """GPU top-k must be a valid top-k of the oracle logits up to tolerance;
    where the oracle's ranking has clear gaps it must match exactly."""
    k = gpu_idx.shape[1]
    for r in range(ref_logits.shape[0]):
        order = np.lexsort((np.arange(ref_logits.shape[1]), -ref_logits[r]))
        kth = ref_logits[r, order[k - 1]]
        assert np.all(ref_logits[r, gpu_idx[r]] >= kth - 2 * tol)
        gaps = -np.diff(ref_logits[r, order[:k + 1]])
        if np.all(gaps > 2 * tol):
            assert list(gpu_idx[r]) == list(order[:k])


@pytest.mark.parametrize("counts,lens", [([1], [37]), ([3, 2], [0, 70]), ([9, 0, 8], [130, 5, 64]),
                                         ([20, 20, 1], [130, 0, 77]), ([56, 50, 40], [200, 64, 1])])
def test_draft_step_bf16_gqa(counts, lens):
    shape = Shape(256, 4, 2, 128, 384, 1000)
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=sum(counts))
    tol = TOL["bf16"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    for r in range(len(rows["seq"])):
        b, s = rows["seq"][r], rows["slot"][r]
        for got, want in ((gpu["tree_k"][b, s], tk[b, s]), (gpu["tree_v"][b, s], tv[b, s])):
            assert np.all(np.abs(got - want) <= 2.0**-7 * np.abs(want) + 1e-3)
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# Few (sequence, kv head) groups: the attention plan gives the tree slots a
# split of their own beside prefix splits of whole tiles.  Cases: one tile
# (no split), several splits with a ragged last tile, an empty prefix in one
# sequence, splits past a short sequence's end, 16 queries per kv head, and
# 1, 2 and 8 query heads per kv head.
@pytest.mark.parametrize("heads,kv_heads,counts,lens", [(2, 2, [10], [700]), (4, 2, [8, 3], [1000, 129]),
                                                       (4, 2, [1, 5, 8], [300, 0, 513]), (8, 1, [2, 1], [128, 1]),
                                                       (8, 1, [1], [2049]), (2, 2, [16, 16], [0, 255])])
def test_draft_step_bf16_few_queries(heads, kv_heads, counts, lens):
    shape = Shape(256, heads, kv_heads, 128, 384, 1000)
    assert max(counts) * heads // kv_heads <= 16
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=11 + sum(counts) + sum(lens))
    tol = TOL["bf16"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# bf16 GEMM operands (EAGLE_ACT_BF16) against the oracle under the same contract,
# through the three kernels: up to 16 rows (register-streamed weights), 17..256
# (wide kernel), 257+ (LDS-tiled kernel); the d = 1024 cases split K over the
# grid (partial sums + reduce, including the sum-of-squares epilogues).
@pytest.mark.parametrize("d,counts,lens", [(256, [1], [37]), (256, [9, 0, 8], [130, 5, 64]),
                                           (256, [20, 20, 1], [130, 0, 77]),
                                           (256, [56, 56, 56, 56, 40], [200, 64, 1, 0, 33]),
                                           (1024, [6, 7], [3, 100]), (1024, [30, 10], [64, 9]),
                                           (1024, [56, 56, 56, 56, 56], [40, 0, 3, 77, 128])])
def test_draft_step_bf16_act(d, counts, lens):
    shape = Shape(d, d // 128 * 2, d // 128, 128, 3 * d // 2 if d == 256 else 2816, 1000 if d == 256 else 4096)
    # weights ~N(0, 0.02) as in the draft-head workloads
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=5 + sum(counts) + d, act=True, std=0.02)
    tol = TOL["bf16"]
    print(f"feature max-abs {np.max(np.abs(gpu['feat'] - ref['feat'])):.2e}, "
          f"logit max-abs {np.max(np.abs(gpu['logits'] - ref['logits'])):.2e}")
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    for r in range(len(rows["seq"])):
        b, s = rows["seq"][r], rows["slot"][r]
        for got, want in ((gpu["tree_k"][b, s], tk[b, s]), (gpu["tree_v"][b, s], tv[b, s])):
            assert np.all(np.abs(got - want) <= 2.0**-7 * np.abs(want) + 1e-3)
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# Split operands through the large-M kernel with K split over the grid in
# uneven parts: at d = 1024 the K of 1024, 2048 and 2816 are 32, 64 and 88
# blocks of 32, spread over up to five splits.
@pytest.mark.parametrize("counts,lens", [([56, 56, 56, 56, 56], [40, 0, 3, 77, 128]),
                                         ([56, 56, 56, 56, 48, 30], [5, 64, 0, 9, 300, 1])])
def test_draft_step_bf16_tile_ksplit(counts, lens):
    d = 1024
    shape = Shape(d, d // 128 * 2, d // 128, 128, 2816, 4096)
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=9 + sum(counts), std=0.02)
    tol = TOL["bf16"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# 65 to 80 rows (the wide kernel, one 80-row tile) and 129 to 160 rows (the
# large-M kernel with one 160-row activation tile per workgroup), K split over
# the grid (d = 1024), split operands and EAGLE_ACT_BF16.
@pytest.mark.parametrize("counts,lens,act", [([40, 25], [7, 200], False), ([56, 24], [64, 0], False),
                                             ([30, 40, 10], [1, 90, 33], True),
                                             ([56, 56, 17], [40, 0, 300], False), ([56, 56, 38], [12, 77, 5], False),
                                             ([56, 56, 48], [3, 64, 128], True)])
def test_draft_step_bf16_mid_tile(counts, lens, act):
    d = 1024
    shape = Shape(d, d // 128 * 2, d // 128, 128, 2816, 4096)
    assert 65 <= sum(counts) <= 80 or 129 <= sum(counts) <= 160
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=13 + sum(counts), act=act, std=0.02)
    tol = TOL["bf16"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# Grids of more than one round of 256 workgroups with a partial last round:
# the large-M kernel runs whole rounds of unsplit tiles and the remaining
# tiles split over K (the SwiGLU product: 130 x 2 tiles, the LM head: 157 x 2).
def test_draft_step_bf16_tile_split_tail():
    shape = Shape(1024, 16, 8, 128, 16640, 40000)
    counts, lens = [56, 56, 56, 56, 56, 20], [12, 0, 300, 64, 5, 77]
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=77, std=0.02)
    tol = TOL["bf16"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# More than 64 queries per kv head (eight query heads per kv head): several
# 64-query blocks over the same keys (80, 128 and 136 queries).
@pytest.mark.parametrize("counts,lens", [([10, 9], [700, 129]), ([16], [300]), ([17, 3], [64, 1000])])
def test_draft_step_bf16_many_queries(counts, lens):
    shape = Shape(256, 8, 1, 128, 384, 1000)
    assert max(counts) * 8 > 64
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=31 + sum(counts) + sum(lens))
    tol = TOL["bf16"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


# EAGLE_ACT_BF16 at the full 7B draft-head shape: outside the 2e-2 bar (stated
# beside the flag in eagle.h), so the test records the deviation from the fp64
# oracle that rounds the same operands and bounds it loosely; without the flag
# the same rows must meet the bar.
@pytest.mark.parametrize("act", [True, False])
def test_act_bf16_deviation_at_the_7b_shape(act):
    shape = CONFIGS[2].shape
    ref, gpu, rows, tk, tv = _run_draft(shape, [4, 2], [300, 77], seed=21, act=act, std=0.02)
    dev_logits = float(np.max(np.abs(gpu["logits"] - ref["logits"])))
    dev_feat = float(np.max(np.abs(gpu["feat"] - ref["feat"])))
    print(f"7B shape, EAGLE_ACT_BF16={act}: logit max-abs {dev_logits:.3e}, feature max-abs {dev_feat:.3e}")
    if act:
        assert dev_logits < 0.1 and dev_feat < 0.1
    else:
        assert dev_logits < TOL["bf16"] and dev_feat < TOL["bf16"]


@pytest.mark.parametrize("counts,lens", [([1], [32]), ([4, 1], [32, 3]), ([3, 3, 3], [0, 17, 40])])
def test_draft_step_f32_tiny(counts, lens):
    shape = CONFIGS[1].shape
    ref, gpu, rows, tk, tv = _run_draft(shape, counts, lens, seed=7 + sum(counts), topk=1)
    tol = TOL["f32"]
    assert np.max(np.abs(gpu["feat"] - ref["feat"])) < tol
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


@pytest.mark.parametrize("dtype,act", [("bf16", False), ("bf16", True), ("f32", False)])
def test_head_only_is_root_distribution(dtype, act):
    shape = Shape(256, 4, 2, 128, 384, 1000) if dtype == "bf16" else CONFIGS[1].shape
    ref, gpu, rows, _, _ = _run_draft(shape, [2, 1], [10, 20], seed=3, head_only=True, act=act)
    tol = TOL[dtype]
    assert np.max(np.abs(gpu["logits"] - ref["logits"])) < tol
    _check_topk_valid(ref["logits"], gpu["idx"], tol)


def test_draft_step_is_deterministic():
    shape = Shape(256, 4, 2, 128, 384, 1000)
    _, g1, _, _, _ = _run_draft(shape, [20, 13], [90, 3], seed=11)
    _, g2, _, _, _ = _run_draft(shape, [20, 13], [90, 3], seed=11)
    for key in ("feat", "logits", "idx", "lse"):
        assert np.array_equal(g1[key], g2[key]), key


@pytest.mark.parametrize("rows,vocab,k,row_base", [(3, 32000, 10, 0), (40, 32000, 4, 1000), (7, 512, 1, 5),
                                                   (961, 32000, 10, 77), (2, 4096, 16, 3)])
def test_sample_topk_matches_oracle(rows, vocab, k, row_base):
    """Sampled proposals (Gumbel-top-k) against the oracle on the same fp32
    logits: identical draws and log-probabilities; a row whose k-th and
    (k+1)-th perturbed keys lie within 1e-5 of each other counts as a near-tie
    (the two sides' fp32 log may differ in the last bit) and is skipped."""
    from oracle.topk import gumbel_topk
    g = np.random.default_rng(rows + vocab + k)
    x = (g.standard_normal((rows, vocab)) * 2).astype(np.float32)
    x[0, :50] = 3.25  # a plateau of equal logits
    t = torch.from_numpy(x).cuda()
    lse = torch.empty(rows, device="cuda")
    idx = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    lq = torch.empty(rows, k, device="cuda")
    shape = E.make_shape(256, 2, 2, 128, 256, vocab)
    ws = _ws(E.eagle_workspace_bytes(shape, rows, 1, 0))
    seed, rnd = 12345, 6
    E.eagle_sample_topk(rows, vocab, t, k, seed, rnd, row_base, lse, idx, lq, ws)
    torch.cuda.synchronize()
    o_lse, o_idx, o_lq, margin = gumbel_topk(x, k, seed, rnd, np.arange(rows) + row_base)
    gi = idx.cpu().numpy()
    near = margin < 1e-5
    assert near.sum() <= max(1, rows // 100)
    assert np.array_equal(gi[~near], o_idx[~near])
    assert np.allclose(lse.cpu().numpy(), o_lse, rtol=1e-6, atol=1e-5)
    assert np.allclose(lq.cpu().numpy()[~near], o_lq[~near], rtol=0, atol=2e-5)
    # draws without replacement; not the deterministic top-k
    assert all(len(set(r)) == k for r in gi)
    if k > 1:
        _, det, _ = o_topk(x, k)
        assert not np.array_equal(gi, det)


@pytest.mark.parametrize("dtype,rows,bias", [("bf16", 1, True), ("bf16", 5, False), ("bf16", 40, True),
                                             ("bf16", 300, True), ("f32", 3, True)])
def test_fuse_features_matches_oracle(dtype, rows, bias):
    """EAGLE-3 three-feature fusion on the GPU against the oracle: d = 4096
    (the 7B draft head; 12288-wide fused input) through the skinny, wide and
    large-M GEMMs, and the tiny fp32 head."""
    shape = Shape(4096, 32, 32, 128, 11008, 32000) if dtype == "bf16" else CONFIGS[1].shape
    d = shape.d
    g = np.random.default_rng(rows + d)
    w = (g.standard_normal((d, 3 * d)) * 0.02).astype(np.float32)
    b = (g.standard_normal(d) * 0.02).astype(np.float32) if bias else None
    if dtype == "bf16":
        w = bf16_values(w)
        b = bf16_values(b) if bias else None
    low, mid, high = ((g.standard_normal((rows, d)) + 0.1 * s).astype(np.float32) for s in range(3))
    es = E.make_shape(**dev.shape_dict(shape))
    t = lambda a: dev.tensor(a.reshape(-1), shape.dtype)
    out = torch.full((rows, d), float("nan"), device="cuda")
    ws = _ws(E.eagle_fuse_workspace_bytes(es, rows))
    E.eagle_fuse_features(es, t(w), t(b) if bias else None, rows, torch.from_numpy(low).cuda(),
                          torch.from_numpy(mid).cuda(), torch.from_numpy(high).cuda(), out, ws)
    torch.cuda.synchronize()
    ref = OD.fuse_features(shape, w, b, low, mid, high)
    assert np.max(np.abs(out.cpu().numpy() - ref)) < TOL[dtype]


def test_block_weight_layout():
    """eagle_block_weight: 16-row x 128-column blocks of 4 KB, each band's
    blocks in column order, in a block the 32-column quarters in turn (16 rows
    of 32 values each), rows past the end 0 (a rearrangement, bit-exact)."""
    rows, cols = 40, 384
    w = bf16_values(normal_array(77, 0, (rows, cols)))
    t = dev.tensor(w.reshape(-1), "bf16").view(rows, cols)
    out = torch.full((E.eagle_blocked_weight_bytes(rows, cols),), 0x7F, dtype=torch.uint8, device="cuda")
    E.eagle_block_weight(t, rows, cols, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    pad = np.zeros((48, cols), dtype=np.uint16)
    pad[:rows] = bits
    want = pad.reshape(3, 16, 3, 4, 32).transpose(0, 2, 3, 1, 4).ravel()
    assert got.shape == want.shape and np.array_equal(got, want)


# The blocked copies change only where the GEMMs read their weights: the
# skinny (<= 16 rows) and wide (17..256 rows) kernels read them and sum the
# same products in the same order; above 256 rows the row-major matrices are
# read.  Every output must be bit-identical with and without them.
@pytest.mark.parametrize("counts,lens", [([3, 2], [0, 70]), ([9, 0, 8], [130, 5, 64]), ([20, 20, 1], [130, 0, 77]),
                                         ([56, 50, 40, 56, 54], [200, 64, 1, 90, 33]),
                                         ([56, 56, 56, 56, 56, 20], [30, 64, 1, 90, 33, 7])])
def test_blocked_weights_give_identical_results(counts, lens):
    shape = Shape(256, 4, 2, 128, 384, 1000)
    seed = 41 + sum(counts)
    _, g0, _, _, _ = _run_draft(shape, counts, lens, seed=seed, oracle=False)
    _, g1, _, _, _ = _run_draft(shape, counts, lens, seed=seed, oracle=False, blocked=True)
    for k in g0:
        assert np.array_equal(g0[k], g1[k], equal_nan=True), k
