"""Pins for the oracle's verifier (CPU only).

* a node with one child is textbook speculative sampling under the same uniforms;
* the greedy worked example (accept A, B; correction X);
* the first draft token is free: q == p at the root gives acceptance 1 always;
* exact enumeration: with candidates drawn without replacement from q the
  emitted tokens follow p exactly (first token and second token), and
  single-candidate acceptance equals sum min(p, q) = 1 - TV; negative controls
  (deterministic top-k proposals; the i.i.d. rule under without-replacement
  proposals) deviate;
* the sampled walk's empirical law passes a chi-square test against p;
* the expected tokens per round reproduce the pages' worked examples.
"""
import json
import os

import numpy as np
import pytest
import scipy.stats

from oracle.numerics import softmax
from oracle.philox import uniform, EVENT_DRAW
from oracle.verify import (exact_round_law, first_token_law, second_token_law, speculative_sample_one,
                           verify_sequence)

from conftest import GOLDEN


def _rand_dist(g, V, sparsity=0.0):
    p = g.random(V) ** 3
    if sparsity:
        p[g.random(V) < sparsity] = 0.0
        if p.sum() == 0:
            p[0] = 1.0
    return p / p.sum()


def test_one_child_is_textbook_speculative_sampling():
    g = np.random.default_rng(0)
    V = 7
    agree = 0
    for trial in range(400):
        p = _rand_dist(g, V)
        q = _rand_dist(g, V)
        x = int(g.choice(V, p=q))
        target = np.log(np.stack([p, _rand_dist(g, V)]))
        draft = np.log(np.stack([q, _rand_dist(g, V)]))
        out = verify_sequence([-1, 0], [0, x], target, draft, seed=11, rnd=trial, seq=0)
        ua = uniform(11, trial, 0, 0, 0)
        if ua < min(1.0, p[x] / q[x]):
            # accepted: the bonus comes from the child's own target row
            assert out["path"] == [1]
            pc = softmax(target[1])
            cdf = np.cumsum(pc)
            ub = uniform(11, trial, 0, 1, EVENT_DRAW)
            assert out["next_token"] == int(np.searchsorted(cdf, ub * cdf[-1], side="right"))
        else:
            ref = speculative_sample_one(p, q, x, ua, uniform(11, trial, 0, 0, EVENT_DRAW))
            assert out["path"] == [] and out["next_token"] == ref
        agree += 1
    assert agree == 400


def test_greedy_worked_example():
    with open(os.path.join(GOLDEN, "greedy_example.json")) as f:
        fx = json.load(f)
    names = fx["nodes"]
    vocab = ["A", "B", "C", "D", "E", "X"]
    V = len(vocab)
    tok = [0] + [vocab.index(n) for n in names[1:]]
    N = len(names)
    target = np.zeros((N, V))
    for node, nxt in fx["target_argmax_after"].items():
        target[names.index(node), vocab.index(nxt)] = 5.0
    draft = np.random.default_rng(3).standard_normal((N, V))
    for seed in range(20):
        out = verify_sequence(fx["parent"], tok, target, draft, seed, 0, 0, greedy=True)
        assert [names[i] for i in out["path"]] == fx["accepted"]
        assert vocab[out["next_token"]] == fx["correction"]
        assert out["accept_len"] == len(fx["accepted"]) + 1


def test_first_draft_token_is_free():
    g = np.random.default_rng(4)
    V, N = 50, 4
    for seed in range(300):
        logits = g.standard_normal(V) * 3
        target = np.stack([logits] + [g.standard_normal(V) for _ in range(N - 1)])
        draft = np.stack([logits] + [g.standard_normal(V) for _ in range(N - 1)])
        x = int(g.choice(V, p=softmax(logits)))
        out = verify_sequence([-1, 0, 1, 1], [0, x, 3, 4], target, draft, seed, 0, 0)
        assert out["path"][:1] == [1]


def _tables(g, V, depth, sparsity=0.0):
    cache_p, cache_q = {}, {}

    def p_of(prefix):
        if prefix not in cache_p:
            cache_p[prefix] = _rand_dist(g, V, sparsity)
        return cache_p[prefix]

    def q_of(prefix):
        if prefix not in cache_q:
            cache_q[prefix] = _rand_dist(g, V, sparsity)
        return cache_q[prefix]
    return p_of, q_of


@pytest.mark.parametrize("V,shape", [(3, (2, 1)), (4, (3, 2)), (5, (2, 2, 1)), (6, (1, 1, 1)), (4, (4, 1))])
def test_exact_law_is_target_law_without_replacement(V, shape):
    g = np.random.default_rng(V * 10 + len(shape))
    for trial in range(6):
        p_of, q_of = _tables(g, V, len(shape), sparsity=0.3 if trial % 2 else 0.0)
        nchild = lambda prefix: shape[len(prefix)] if len(prefix) < len(shape) else 0
        law = exact_round_law(p_of, q_of, nchild, "wor", iid_rule=False, max_len=len(shape))
        assert abs(sum(law.values()) - 1) < 1e-12
        assert np.allclose(first_token_law(law, V), p_of(()), rtol=0, atol=1e-12)
        for a in range(V):
            s2 = second_token_law(law, V, a)
            if s2.sum() > 0:
                assert np.allclose(s2, p_of((a,)), rtol=0, atol=1e-12)


def test_iid_rule_is_exact_for_iid_proposals():
    g = np.random.default_rng(7)
    V = 4
    for trial in range(6):
        p_of, q_of = _tables(g, V, 1)
        law = exact_round_law(p_of, q_of, lambda pr: 3 if len(pr) == 0 else 0, "iid", iid_rule=True, max_len=1)
        assert np.allclose(first_token_law(law, V), p_of(()), rtol=0, atol=1e-12)


def test_negative_controls_deviate():
    g = np.random.default_rng(8)
    V = 5
    worst_topk, worst_mix = 0.0, 0.0
    for trial in range(10):
        p_of, q_of = _tables(g, V, 1)
        nchild = lambda pr: 2 if len(pr) == 0 else 0
        law = exact_round_law(p_of, q_of, nchild, "topk", iid_rule=False, max_len=1)
        worst_topk = max(worst_topk, np.abs(first_token_law(law, V) - p_of(())).max())
        law = exact_round_law(p_of, q_of, nchild, "wor", iid_rule=True, max_len=1)
        worst_mix = max(worst_mix, np.abs(first_token_law(law, V) - p_of(())).max())
    assert worst_topk > 0.05
    assert worst_mix > 0.01


def test_single_candidate_acceptance_is_one_minus_tv():
    g = np.random.default_rng(9)
    V = 6
    for trial in range(20):
        p, q = _rand_dist(g, V), _rand_dist(g, V)
        acc = sum(q[x] * min(1.0, p[x] / q[x]) for x in range(V))
        assert np.isclose(acc, np.minimum(p, q).sum(), rtol=0, atol=1e-14)
        assert np.isclose(acc, 1 - 0.5 * np.abs(p - q).sum(), rtol=0, atol=1e-14)
        # the enumerator: probability that the first emitted token came from acceptance
        law = exact_round_law(lambda pr: p if not pr else np.full(V, 1 / V), lambda pr: q,
                              lambda pr: 1 if not pr else 0, "wor", max_len=1)
        p_len2 = sum(v for k, v in law.items() if len(k) == 2)
        assert np.isclose(p_len2, acc, rtol=0, atol=1e-12)


def test_sampled_walk_chi_square_against_target():
    """Empirical law of the sampled walk (Philox uniforms) vs p, on a small
    static tree with candidates drawn without replacement from q (harness-drawn)."""
    g = np.random.default_rng(10)
    V = 8
    p0 = _rand_dist(g, V)
    q0 = _rand_dist(g, V)
    parent = [-1, 0, 0, 0, 1, 1]
    target_child = np.log(_rand_dist(g, V))
    draft_child = np.log(_rand_dist(g, V))
    n = 20000
    counts = np.zeros(V)
    draw = np.random.default_rng(11)
    for r in range(n):
        c = list(draw.choice(V, size=3, replace=False, p=q0))
        c1 = list(draw.choice(V, size=2, replace=False, p=np.exp(draft_child)))
        token = [0] + c + c1
        target = np.stack([np.log(p0)] + [target_child] * 5)
        draft = np.stack([np.log(q0)] + [draft_child] * 5)
        out = verify_sequence(parent, token, target, draft, 5, r, 0)
        first = token[out["path"][0]] if out["path"] else out["next_token"]
        counts[first] += 1
    stat, pval = scipy.stats.chisquare(counts, p0 * n)
    assert pval > 1e-3, (pval, counts, p0 * n)


def _alpha_pair(alpha, V=4):
    """Path-independent (p, q) with sum min(p, q) = alpha."""
    p = np.array([alpha, 1 - alpha, 0.0, 0.0])
    q = np.array([alpha, 0.0, 1 - alpha, 0.0])
    return p, q


def test_expected_tokens_worked_examples():
    with open(os.path.join(GOLDEN, "expected_tokens.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        alpha = case["alpha"]
        K = len(alpha)
        pairs = [_alpha_pair(a) for a in alpha]
        # exact: enumerate the chain's law
        law = exact_round_law(lambda pr: pairs[len(pr)][0] if len(pr) < K else np.full(4, 0.25),
                              lambda pr: pairs[len(pr)][1], lambda pr: 1 if len(pr) < K else 0, "wor",
                              max_len=K)
        e_len = sum(len(k) * v for k, v in law.items())
        assert round(e_len, 3) == pytest.approx(case["expected_tokens"], abs=6e-4), case
        # sampled walk through the oracle, 4000 rounds within 4 sigma
        g = np.random.default_rng(12)
        lens = []
        parent = list(range(-1, K))
        for r in range(4000):
            toks = [0]
            for i in range(K):
                toks.append(int(g.choice(4, p=pairs[i][1])))
            with np.errstate(divide="ignore"):
                target = np.stack([np.log(pairs[i][0]) for i in range(K)] + [np.zeros(4)])
                draft = np.stack([np.log(pairs[i][1]) for i in range(K)] + [np.zeros(4)])
            out = verify_sequence(parent, toks, target, draft, 1, r, 0)
            lens.append(out["accept_len"])
        lens = np.array(lens)
        assert abs(lens.mean() - e_len) < 4 * lens.std() / np.sqrt(len(lens)) + 1e-9, case


def test_missing_draft_distribution_is_flagged_and_corrected_from_p():
    """A node with children but no draft distribution: flag BADTREE, stop, and
    draw the correction from that node's target (a one-hot target makes the
    draw certain)."""
    from oracle.verify import F_BADTREE
    V = 6
    parent, token = [-1, 0, 0], [0, 2, 4]
    root = np.full(V, -np.inf)
    root[3] = 0.0
    tg = [root, np.zeros(V), np.zeros(V)]
    for rnd in range(5):
        out = verify_sequence(parent, token, tg, [None, None, None], 0, rnd, 0)
        assert out["flags"] == F_BADTREE and out["path"] == [] and out["accept_len"] == 1
        assert out["next_token"] == 3
