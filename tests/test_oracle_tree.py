"""Pins for top-k and tree construction (CPU only).

* top-k = first k of a full sort by (value desc, index asc), on adversarial ties;
* EAGLE-2 value never grows along a path, and the reranked set is a connected
  tree (study note section 10.3, the two properties and exercise 5);
* expand and rerank equal brute-force definitions on a fully enumerated tiny
  draft tree, with value = product of confidences in fp64;
* the static templates have the stated shapes.
"""
import itertools

import numpy as np
import scipy.special

from oracle import tree as T
from oracle.numerics import softmax
from oracle.topk import row_lse, row_topk, softmax_topk
from workloads import TEMPLATES, template_child_counts


def test_topk_brute_force_with_ties():
    g = np.random.default_rng(0)
    for trial in range(200):
        V = int(g.integers(1, 60))
        row = g.integers(-3, 4, size=V).astype(np.float32)  # many ties
        if trial % 3 == 0:
            row[g.integers(0, V, size=3)] = -0.0
        k = int(g.integers(1, V + 1))
        ref = sorted(range(V), key=lambda i: (-float(row[i]), i))[:k]
        assert list(row_topk(row, k)) == ref


def test_topk_negative_zero_ties_with_positive_zero():
    row = np.array([-0.0, 0.0, -0.0, -1.0], dtype=np.float32)
    assert list(row_topk(row, 3)) == [0, 1, 2]


def test_lse_and_logq():
    g = np.random.default_rng(1)
    x = (g.standard_normal((3, 1000)) * 2).astype(np.float32)
    lse, idx, logq = softmax_topk(x, 5)
    for r in range(3):
        assert np.isclose(lse[r], scipy.special.logsumexp(x[r].astype(np.float64)), rtol=0, atol=1e-12)
        assert np.allclose(np.exp(logq[r]), scipy.special.softmax(x[r].astype(np.float64))[idx[r]])


def _toy_draft(V, seed):
    """A deterministic toy draft model: q(. | prefix) from a hash of the prefix."""
    def q_of(prefix):
        g = np.random.default_rng([seed] + list(prefix) + [99])
        return softmax(g.standard_normal(V) * 2.0)
    return q_of


def test_eagle2_against_brute_force_definitions():
    V, k, depth, m = 6, 3, 4, 12
    for seed in range(20):
        q_of = _toy_draft(V, seed)
        pool = T.Pool(0, 0)
        frontier = [0]
        prefix_of = {0: ()}
        for s in range(depth):
            idx, lq = [], []
            for u in frontier:
                row = np.log(q_of(prefix_of[u])).astype(np.float32)
                order = row_topk(row, k)
                idx.append(order)
                lq.append(row[order] - np.float32(row_lse(row)))
            before = len(pool)
            frontier = T.expand(pool, frontier, idx, lq, k)
            for c in range(before, len(pool)):
                prefix_of[c] = prefix_of[pool.parent[c]] + (pool.token[c],)
            # brute force: the new frontier = the k new nodes of largest value
            new = list(range(before, len(pool)))
            val = {c: np.prod([q_of(prefix_of[c][:j])[prefix_of[c][j]] for j in range(len(prefix_of[c]))])
                   for c in new}
            best = sorted(new, key=lambda c: (-val[c], c))[:k]
            assert set(best) == set(frontier), seed
        # value never grows along a path (fp32 log-values)
        for c in range(1, len(pool)):
            assert pool.logv[c] <= pool.logv[pool.parent[c]]
        tr = T.finalize(pool, m)
        kept = set(int(i) for i in tr["pool_id"][1:])
        # brute force rerank: the m most valuable nodes of the pool
        allv = {c: np.prod([q_of(prefix_of[c][:j])[prefix_of[c][j]] for j in range(len(prefix_of[c]))])
                for c in range(1, len(pool))}
        ref = sorted(allv, key=lambda c: (-allv[c], pool.depth[c], c))[:m]
        assert kept == set(ref), seed
        # connected, parents precede children, siblings in creation order
        for t in range(1, len(tr["parent"])):
            p = int(tr["parent"][t])
            assert 0 <= p < t
            assert int(tr["pool_id"][p]) == pool.parent[int(tr["pool_id"][t])]
            assert int(tr["depth"][t]) == int(tr["depth"][p]) + 1


def test_rerank_tie_prefers_shallower():
    # child logq = 0 so child value == parent value exactly
    pool = T.Pool(0, 0)
    a = pool.add(0, 1, np.float32(-0.5))
    b = pool.add(a, 2, np.float32(0.0))
    c = pool.add(0, 3, np.float32(-0.5))
    tr = T.finalize(pool, 2)
    assert [int(x) for x in tr["pool_id"]] == [0, a, c]  # b ties with a and c but is deeper
    tr = T.finalize(pool, 3)
    assert [int(x) for x in tr["pool_id"]] == [0, a, c, b]


def test_static_templates():
    s26 = TEMPLATES["static26"]
    depth = [0] * len(s26)
    for i in range(1, len(s26)):
        depth[i] = depth[s26[i]] + 1
    counts = np.bincount(depth)
    assert list(counts) == [1, 4, 6, 8, 5, 2] and len(s26) == 26 and max(depth) == 5
    assert all(s26[i] <= s26[i + 1] for i in range(1, len(s26) - 1))  # BFS, siblings contiguous
    # rank rule up to depth 4: a node at depth t with sibling rank r has max(0, b_t - r) children
    b = [4, 3, 2, 1]
    nch = template_child_counts(s26)
    rank = [0] * len(s26)
    for i in range(1, len(s26)):
        rank[i] = sum(1 for j in range(1, i) if s26[j] == s26[i])
    for i in range(len(s26)):
        if depth[i] < 4:
            assert nch[i] == max(0, b[depth[i]] - rank[i]), i
    # the two extra depth-5 nodes sit under the depth-4 nodes with least path rank-sum
    def rsum(i):
        s = 0
        while i > 0:
            s += rank[i]
            i = s26[i]
        return s
    d4 = [i for i in range(len(s26)) if depth[i] == 4]
    best = sorted(d4, key=lambda i: (rsum(i), i))[:2]
    assert sorted(i for i in d4 if nch[i] > 0) == sorted(best)
    assert TEMPLATES["chain5"] == [-1, 0, 1, 2, 3]


def test_static_expand_reproduces_template():
    s26 = TEMPLATES["static26"]
    nch = template_child_counts(s26)
    pool = T.Pool(0, 0)
    frontier = [0]
    for s in range(5):
        idx = [[100 * u + r for r in range(4)] for u in frontier]
        lq = [[-0.1 * (r + 1) for r in range(4)] for u in frontier]
        frontier = T.expand(pool, frontier, idx, lq, 4, nch)
    assert pool.parent == s26
    tr = T.finalize(pool, 0)
    assert [int(x) for x in tr["pool_id"]] == list(range(26))
    # rank r child of node u carries the parent's r-th token
    for i in range(1, 26):
        r = sum(1 for j in range(1, i) if s26[j] == s26[i])
        assert pool.token[i] == 100 * s26[i] + r


def test_gumbel_topk_draws_without_replacement_from_softmax():
    """Gumbel-top-k against the law it must follow: the first proposal ~ p, and
    the ordered pair (first, second) ~ p_i p_j / (1 - p_i), the probability of
    drawing i then j without replacement.  Pearson chi-square over 20000
    seeded rows, alpha = 1e-3."""
    from scipy.stats import chi2

    from oracle.topk import gumbel_topk

    logits = np.array([1.2, -0.3, 0.5, 2.0, -1.0], dtype=np.float32)
    p = np.exp(logits.astype(np.float64) - logits.max())
    p /= p.sum()
    n = 20000
    rows = np.tile(logits, (n, 1))
    _, idx, _, _ = gumbel_topk(rows, 2, 7, 3, np.arange(n))
    first = np.bincount(idx[:, 0], minlength=5)
    stat = np.sum((first - n * p) ** 2 / (n * p))
    assert stat < chi2.ppf(1 - 1e-3, 4), stat
    V = 5
    pair = np.zeros((V, V))
    for a, b in idx:
        pair[a, b] += 1
    exp = np.array([[p[i] * p[j] / (1 - p[i]) if i != j else 0.0 for j in range(V)] for i in range(V)]) * n
    m = exp > 0
    stat2 = np.sum((pair[m] - exp[m]) ** 2 / exp[m])
    assert stat2 < chi2.ppf(1 - 1e-3, m.sum() - 1), stat2
    # no repeats within a row, and the proposals differ from the deterministic top-2
    assert np.all(idx[:, 0] != idx[:, 1])
    assert np.mean(idx[:, 0] == 3) < 0.6


def test_gumbel_uniforms_are_inside_the_open_interval():
    from oracle.philox import philox4x64_10
    from oracle.topk import gumbel_keys

    # word v % 4 of counter (row, v // 4, 0, 1): recompute token 6 with the scalar generator
    w = philox4x64_10((11, 6 // 4, 0, 1), (5, 9))[6 % 4]
    u = ((w >> 41) + 0.5) * 2.0 ** -23
    assert 0.0 < u < 1.0
    key = gumbel_keys(np.zeros(8, np.float32), 5, 9, 11)
    assert abs(float(key[6]) - (-np.log(-np.log(u)))) < 1e-5


def test_commit_special_cases():
    """Accepted-path commit: a fully accepted chain appends its slots in order,
    nothing accepted changes nothing, capacity and malformed paths are flagged
    and leave the prefix as it was."""
    from oracle.commit import BAD_PATH, OVERFLOW, commit

    g = np.random.default_rng(2)
    H, hd, L = 2, 4, 3
    pk = [g.standard_normal((H, L, hd)), g.standard_normal((H, L, hd))]
    pv = [g.standard_normal((H, L, hd)), g.standard_normal((H, L, hd))]
    tk, tv = g.standard_normal((2, 64, H, hd)), g.standard_normal((2, 64, H, hd))
    paths = [[1, 2, 3, -1, -1], [-1, -1, -1, -1, -1]]
    k2, v2, lens, flags = commit(pk, pv, [L, L], [L + 4, L + 4], tk, tv, paths, [4, 1])
    assert lens == [L + 3, L] and flags == [0, 0]
    assert np.array_equal(k2[0][:, :L], pk[0]) and np.array_equal(k2[1], pk[1])
    for j in range(3):
        assert np.array_equal(k2[0][:, L + j], tk[0, 1 + j]) and np.array_equal(v2[0][:, L + j], tv[0, 1 + j])
    # explicit slots: node n lives in slot 10 + n
    slots = [[10 + n for n in range(5)]] * 2
    k3, _, _, _ = commit(pk, pv, [L, L], [L + 4, L + 4], tk, tv, [[2, 4, -1, -1, -1]] * 2, [3, 3], slots)
    assert np.array_equal(k3[1][:, L], tk[1, 12]) and np.array_equal(k3[1][:, L + 1], tk[1, 14])
    # no room; then a node index out of range
    _, _, lens, flags = commit(pk, pv, [L, L], None, tk, tv, [[1, 2, 3, -1, -1], [1, -1, -1, -1, -1]], [4, 2])
    assert flags == [OVERFLOW, OVERFLOW] and lens == [L, L]
    _, _, lens, flags = commit(pk, pv, [L, L], [9, 9], tk, tv, [[1, 7, -1, -1, -1]] * 2, [3, 3])
    assert flags == [BAD_PATH, BAD_PATH] and lens == [L, L]
