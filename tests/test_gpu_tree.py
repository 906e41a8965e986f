"""GPU parity of eagle_tree_init / eagle_tree_expand / eagle_tree_finalize:
bit-exact pools (including fp32 log-values), frontiers, next draft rows and
flattened trees, on seeded top-k inputs with many exact ties."""
import numpy as np
import pytest
import torch

import eagle_feature_level_amd as E
from oracle import tree as OT
from workloads import TEMPLATES, template_child_counts
from workloads import device as dev

pytestmark = pytest.mark.gpu


def _topk_inputs(g, rows, topk, V):
    idx = np.stack([g.choice(V, size=topk, replace=False) for _ in range(rows)]).astype(np.int32)
    # log-probs, sorted descending, quantised to 1/4 so that sums tie exactly
    lq = -np.sort(np.round(g.exponential(1.5, size=(rows, topk)) * 4) / 4, axis=1).astype(np.float32)
    return idx, lq


@pytest.mark.parametrize("kind,B,k,depth,m", [("dynamic", 4, 10, 6, 60), ("dynamic", 3, 4, 5, 20),
                                              ("static26", 2, 4, 5, 0), ("chain5", 3, 1, 4, 0)])
def test_expand_finalize_bit_exact(kind, B, k, depth, m):
    g = np.random.default_rng(hash((kind, B, k)) % 2**32)
    V = 32000
    lens = g.integers(1, 3000, size=B).astype(np.int32)
    static = kind != "dynamic"
    if static:
        tmpl = TEMPLATES[kind]
        nchild_np = template_child_counts(tmpl)
        cap = len(tmpl)
        topk = max(1, int(nchild_np.max()))
        dep = np.zeros(cap, int)
        for i in range(1, cap):
            dep[i] = dep[tmpl[i]] + 1
        ns = [int(np.sum((dep == s + 1) & (nchild_np > 0))) for s in range(depth - 1)]
        n_nodes = cap
        nchild = dev.ints(nchild_np)
    else:
        cap = 1 + k + (depth - 1) * k * k
        topk = k
        ns = [k] * (depth - 1)
        n_nodes = m + 1
        nchild, nchild_np = None, None
    i32 = dict(dtype=torch.int32, device="cuda")
    pt = dict(parent=torch.zeros(B * cap, **i32), token=torch.zeros(B * cap, **i32), depth=torch.zeros(B * cap, **i32),
              logv=torch.zeros(B * cap, device="cuda"), feat_row=torch.zeros(B * cap, **i32),
              slot=torch.zeros(B * cap, **i32), mask=torch.zeros(B * cap, dtype=torch.int64, device="cuda"),
              count=torch.zeros(B, **i32), frontier=torch.zeros(B * 64, **i32))
    pool = E.make_pool(cap, **pt)
    root_tok = g.integers(0, V, size=B).astype(np.int32)
    E.eagle_tree_init(B, pool, dev.ints(root_tok), 0)
    t_len = dev.ints(lens)
    pools = [OT.Pool(int(root_tok[b]), b) for b in range(B)]
    fronts = [[0] for _ in range(B)]
    n_prev, row0 = 1, B
    for s in range(depth):
        last = s == depth - 1
        n_next = 0 if last else ns[s]
        idx, lq = _topk_inputs(g, B * n_prev, topk, V)
        nx = {key: torch.full((max(B * n_next, 1),), -7, **i32) for key in ("token", "parent", "pos", "slot")}
        nx["mask"] = torch.zeros(max(B * n_next, 1), dtype=torch.int64, device="cuda")
        nx["start"] = torch.zeros(B + 1, **i32)
        E.eagle_tree_expand(B, k, s, nchild, pool, n_prev, topk, dev.ints(idx), torch.from_numpy(lq).cuda(), n_next,
                            row0, t_len, nx["token"], nx["parent"], nx["pos"], nx["slot"], nx["mask"], nx["start"])
        torch.cuda.synchronize()
        want_rows = []
        for b in range(B):
            fronts[b] = OT.expand(pools[b], fronts[b], idx[b * n_prev:(b + 1) * n_prev],
                                  lq[b * n_prev:(b + 1) * n_prev], k, nchild_np)
            if not last:
                assert len(fronts[b]) == n_next
                want_rows += OT.assign_rows(pools[b], fronts[b], s, k, static, row0 + b * n_next, int(lens[b]))
        # pools bit-exact
        cnt = pt["count"].cpu().numpy()
        par, tok, dpt = pt["parent"].cpu().numpy(), pt["token"].cpu().numpy(), pt["depth"].cpu().numpy()
        lv = pt["logv"].cpu().numpy()
        for b in range(B):
            n = len(pools[b])
            assert cnt[b] == n
            assert list(par[b * cap:b * cap + n]) == pools[b].parent
            assert list(tok[b * cap:b * cap + n]) == pools[b].token
            assert list(dpt[b * cap:b * cap + n]) == pools[b].depth
            assert np.array_equal(lv[b * cap:b * cap + n], np.array(pools[b].logv, dtype=np.float32))
        if not last:
            got = list(zip(nx["token"].cpu().numpy(), nx["parent"].cpu().numpy(), nx["pos"].cpu().numpy(),
                           nx["slot"].cpu().numpy(), nx["mask"].cpu().numpy().view(np.uint64)))
            assert [tuple(int(v) for v in r) for r in got] == [tuple(int(v) for v in r) for r in want_rows]
            assert list(nx["start"].cpu().numpy()) == [b * n_next for b in range(B + 1)]
            row0 += B * n_next
            n_prev = n_next
    # rerank + flatten
    tr = {key: torch.full((B * n_nodes,), -9, **i32) for key in ("parent", "token", "depth", "pool", "qrow")}
    tr["mask"] = torch.zeros(B * n_nodes, dtype=torch.int64, device="cuda")
    nw = B * (n_nodes - 1)
    rw = {key: torch.full((nw,), -9, **i32) for key in ("token", "parent", "pos", "slot")}
    rw["mask"] = torch.zeros(nw, dtype=torch.int64, device="cuda")
    rw["start"] = torch.zeros(B + 1, **i32)
    E.eagle_tree_finalize(B, m, n_nodes, pool, t_len, tr["parent"], tr["token"], tr["depth"], tr["pool"], tr["mask"],
                          tr["qrow"], rw["token"], rw["parent"], rw["pos"], rw["slot"], rw["mask"], rw["start"])
    torch.cuda.synchronize()
    g_tr = {key: v.cpu().numpy() for key, v in tr.items()}
    g_rw = {key: v.cpu().numpy() for key, v in rw.items()}
    for b in range(B):
        want = OT.finalize(pools[b], m)
        sl = slice(b * n_nodes, (b + 1) * n_nodes)
        assert list(g_tr["pool"][sl]) == list(want["pool_id"])
        assert list(g_tr["parent"][sl]) == list(want["parent"])
        assert list(g_tr["token"][sl]) == list(want["token"])
        assert list(g_tr["depth"][sl]) == list(want["depth"])
        assert list(g_tr["mask"][sl].view(np.uint64)) == list(want["mask"])
        assert list(g_tr["qrow"][sl]) == [pools[b].feat_row[int(p)] for p in want["pool_id"]]
        for t in range(1, n_nodes):
            r = b * (n_nodes - 1) + t - 1
            pid = int(want["pool_id"][t])
            assert g_rw["token"][r] == want["token"][t]
            assert g_rw["parent"][r] == pools[b].feat_row[pools[b].parent[pid]]
            assert g_rw["pos"][r] == lens[b] + want["depth"][t] - 1
            assert g_rw["slot"][r] == t
            assert int(g_rw["mask"][r:r + 1].view(np.uint64)[0]) == int(want["mask"][t])
    assert list(g_rw["start"]) == [b * (n_nodes - 1) for b in range(B + 1)]


def _empty_pool(B, cap):
    i32 = dict(dtype=torch.int32, device="cuda")
    pt = dict(parent=torch.zeros(B * cap, **i32), token=torch.zeros(B * cap, **i32), depth=torch.zeros(B * cap, **i32),
              logv=torch.zeros(B * cap, device="cuda"), feat_row=torch.zeros(B * cap, **i32),
              slot=torch.zeros(B * cap, **i32), mask=torch.zeros(B * cap, dtype=torch.int64, device="cuda"),
              count=torch.zeros(B, **i32), frontier=torch.zeros(B * 64, **i32))
    return pt, E.make_pool(cap, **pt)


def _expand(B, k, step, nchild, pool, n_prev, topk, idx, lq, n_next, row0, lens):
    i32 = dict(dtype=torch.int32, device="cuda")
    nx = {key: torch.full((max(B * n_next, 1),), -7, **i32) for key in ("token", "parent", "pos", "slot")}
    nx["mask"] = torch.zeros(max(B * n_next, 1), dtype=torch.int64, device="cuda")
    nx["start"] = torch.zeros(B + 1, **i32)
    E.eagle_tree_expand(B, k, step, nchild, pool, n_prev, topk, dev.ints(idx), torch.from_numpy(lq).cuda(), n_next,
                        row0, dev.ints(lens), nx["token"], nx["parent"], nx["pos"], nx["slot"], nx["mask"],
                        nx["start"])
    torch.cuda.synchronize()
    return nx


def _finalize(B, m, n_nodes, pool, lens):
    i32 = dict(dtype=torch.int32, device="cuda")
    tr = {key: torch.full((B * n_nodes,), -9, **i32) for key in ("parent", "token", "depth", "pool", "qrow")}
    tr["mask"] = torch.zeros(B * n_nodes, dtype=torch.int64, device="cuda")
    nw = B * (n_nodes - 1)
    rw = {key: torch.full((max(nw, 1),), -9, **i32) for key in ("token", "parent", "pos", "slot")}
    rw["mask"] = torch.zeros(max(nw, 1), dtype=torch.int64, device="cuda")
    rw["start"] = torch.zeros(B + 1, **i32)
    E.eagle_tree_finalize(B, m, n_nodes, pool, dev.ints(lens), tr["parent"], tr["token"], tr["depth"], tr["pool"],
                          tr["mask"], tr["qrow"], rw["token"], rw["parent"], rw["pos"], rw["slot"], rw["mask"],
                          rw["start"])
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in tr.items()}, {key: v.cpu().numpy() for key, v in rw.items()}


def _check_tree(g_tr, g_rw, b, n_nodes, want, pool_o, L):
    """The oracle's flattened tree, then the documented padding up to n_nodes."""
    sl = slice(b * n_nodes, (b + 1) * n_nodes)
    n = len(want["parent"])
    par, tok, dep, pid = g_tr["parent"][sl], g_tr["token"][sl], g_tr["depth"][sl], g_tr["pool"][sl]
    assert list(par[:n]) == list(want["parent"]) and list(tok[:n]) == list(want["token"])
    assert list(dep[:n]) == list(want["depth"]) and list(pid[:n]) == list(want["pool_id"])
    assert list(g_tr["mask"][sl].view(np.uint64)[:n]) == list(want["mask"])
    assert list(g_tr["qrow"][sl][:n]) == [pool_o.feat_row[int(p)] for p in want["pool_id"]]
    for t in range(n, n_nodes):  # padding
        assert (par[t], tok[t], dep[t], pid[t], g_tr["qrow"][sl][t]) == (-2, 0, 0, -1, -1)
        assert int(g_tr["mask"][sl].view(np.uint64)[t]) == 1 << t
        r = b * (n_nodes - 1) + t - 1
        assert (g_rw["token"][r], g_rw["parent"][r], g_rw["pos"][r], g_rw["slot"][r]) == (0, pool_o.feat_row[0], L, t)


def test_expand_nan_row_and_overflow_invalidate_the_pool():
    """Sequence 0 expands normally; sequence 1's root row is NaN (every child's
    value NaN): its pool is invalid (count -1) and its tree is the root alone,
    padded.  Then a second expansion overflows sequence 0's small pool."""
    B, k, V = 2, 3, 32000
    cap = 1 + k + 2  # room for one expansion only
    g = np.random.default_rng(5)
    lens = np.array([100, 7], np.int32)
    pt, pool = _empty_pool(B, cap)
    root_tok = np.array([11, 12], np.int32)
    E.eagle_tree_init(B, pool, dev.ints(root_tok), 0)
    idx, lq = _topk_inputs(g, B, k, V)
    lq[1, :] = np.nan
    _expand(B, k, 0, None, pool, 1, k, idx, lq, k, B, lens)
    cnt = pt["count"].cpu().numpy()
    assert cnt[0] == 1 + k and cnt[1] == -1
    pools = [OT.Pool(int(root_tok[b]), b) for b in range(B)]
    fr = [OT.expand(pools[b], [0], idx[b:b + 1], lq[b:b + 1], k) for b in range(B)]
    assert pools[1].invalid and not pools[0].invalid
    OT.assign_rows(pools[0], fr[0], 0, k, False, B, int(lens[0]))  # the frontier's next-step rows
    for m, n_nodes in ((2, 3), (5, 6)):  # (5, 6): sequence 0 keeps its 3 children and pads 2 entries
        g_tr, g_rw = _finalize(B, m, n_nodes, pool, lens)
        for b in range(B):
            _check_tree(g_tr, g_rw, b, n_nodes, OT.finalize(pools[b], m), pools[b], int(lens[b]))
    # second expansion: 3 frontier nodes x 3 children do not fit in cap 6
    idx2, lq2 = _topk_inputs(g, B * k, k, V)
    _expand(B, k, 1, None, pool, k, k, idx2, lq2, k, B + B * k, lens)
    assert list(pt["count"].cpu().numpy()) == [-1, -1]
    g_tr, g_rw = _finalize(B, 3, 4, pool, lens)
    for b in range(B):
        _check_tree(g_tr, g_rw, b, 4, {"parent": [-1], "token": [int(root_tok[b])], "depth": [0], "pool_id": [0],
                                       "mask": [0]}, pools[b], int(lens[b]))


def test_static_template_inconsistent_requests_invalidate_the_pool():
    """A template node asking for more children than topk, or an n_next that is
    not the number of new children with children, leaves the pool invalid
    (count -1) and writes no next rows."""
    V = 32000
    g = np.random.default_rng(6)
    lens = np.array([50], np.int32)
    for tmpl, topk, n_next in ((TEMPLATES["static26"], 2, 3), (TEMPLATES["chain5"], 1, 2),
                               (TEMPLATES["static26"], 4, 2)):
        nchild_np = template_child_counts(tmpl)
        pt, pool = _empty_pool(1, len(tmpl))
        E.eagle_tree_init(1, pool, dev.ints([9]), 0)
        idx, lq = _topk_inputs(g, 1, topk, V)
        nx = _expand(1, 1, 0, dev.ints(nchild_np), pool, 1, topk, idx, lq, n_next, 1, lens)
        assert int(pt["count"][0]) == -1, (topk, n_next)
        assert (nx["token"].cpu().numpy() == -7).all()
        po = OT.Pool(9, 0)
        if topk < int(nchild_np[0]):  # the oracle's own reading of the first case
            assert OT.expand(po, [0], idx, lq, 1, nchild_np) == [] and po.invalid
        g_tr, g_rw = _finalize(1, 0, len(tmpl), pool, lens)
        _check_tree(g_tr, g_rw, 0, len(tmpl), {"parent": [-1], "token": [9], "depth": [0], "pool_id": [0],
                                               "mask": [0]}, OT.Pool(9, 0), 50)
