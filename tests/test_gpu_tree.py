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
