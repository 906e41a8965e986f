"""Tree-structured recursive rejection sampling, fp64 (test infrastructure only).

The rule for one candidate x drawn from the draft distribution q against the
target distribution p: accept with probability min(1, p(x)/q(x)); on rejection
sample from norm(max(0, p - q)) ("EAGLE 推测解码为什么比 Medusa 快" section 6.2;
"eagle feature-level speculative decoding", section "随机采样验证", where
q(x) a(x) = min(q, p) and the residual adds back max(0, p - q); "EAGLE 完全拆解",
section on why plain draft models fall short, a_i and p_res).

On a tree the rule is applied recursively from the root: a node's children are
tried in rank order as successive rounds of speculative sampling; after a
rejected child the target distribution becomes the residual and (default
without-replacement variant) the rejected token is removed from q, which is
renormalised.  The ``iid`` variant keeps q unchanged.  If every child is
rejected a correction token is drawn from the current residual; if an accepted
node has no children a bonus token is drawn from that node's target
distribution.  accept_len = accepted draft tokens + 1.

Readings where the pages are silent:
* u is on the 2^-24 grid in [0,1) and x is accepted iff u < p(x)/q(x), which
  equals the pages' u <= min(1, p/q) with probability 1;
* q(x) = 0: accept iff p(x) > 0;
* residual mass Z = 0 (reachable only through rounding): keep the current p;
* q's remaining mass 0 after removals: skip the remaining siblings;
* a node with children but no draft distribution is a malformed tree: it is
  flagged and the correction is drawn from the node's target distribution;
* draws use the inverse CDF in ascending token order: the smallest y with
  sum_{z<=y} w(z) > u * sum(w);
* greedy verification ("eagle feature-level speculative decoding", section
  "Greedy 验证"): p = onehot(argmax target logits, ties -> lower index), run
  through the same walk.
"""
from __future__ import annotations

import itertools

import numpy as np

from .numerics import softmax
from .philox import EVENT_DRAW, uniform

F_ZRES = 1  # residual mass was zero; current p kept
F_QZERO = 2  # a candidate had q(x) = 0
F_QEMPTY = 4  # q ran out of mass; remaining siblings skipped
F_BADTREE = 16  # a node with children had no draft distribution


def argmax_low(v) -> int:
    v = np.asarray(v, dtype=np.float64) + 0.0
    return int(np.flatnonzero(v == np.max(v))[0])


def inverse_cdf(w, u: float):
    """Smallest y with cumsum(w)[y] > u * sum(w); also returns the distance of
    u*Z to the nearest CDF boundary (for near-tie reporting)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    t = u * c[-1]
    y = int(np.searchsorted(c, t, side="right"))
    y = min(y, len(w) - 1)
    lo = c[y - 1] if y > 0 else 0.0
    margin = min(abs(t - lo), abs(c[y] - t)) / max(c[-1], 1e-300)
    return y, margin


def children_of(parent, u: int):
    return [i for i in range(len(parent)) if int(parent[i]) == u]


def verify_sequence(parent, token, target_logits, draft_logits, seed: int, rnd: int, seq: int,
                    greedy: bool = False, iid: bool = False):
    """Walk one sequence's tree.

    parent, token: per tree node (node 0 = root, siblings in rank order).
    target_logits[i]: target logits at node i (distribution of the token after
    node i).  draft_logits[i]: draft logits at node i (q for node i's children);
    only needed for nodes with children.
    Returns dict(path, accept_len, next_token, flags, margins).
    """
    u_node = 0
    path = []
    flags = 0
    margins = []  # relative distances |u - p/q| of each decision
    draw_margin = None
    while True:
        kids = children_of(parent, u_node)
        t = np.asarray(target_logits[u_node], dtype=np.float64)
        if greedy:
            p = np.zeros_like(t)
            p[argmax_low(t)] = 1.0
        else:
            p = softmax(t)
        if not kids:
            y, draw_margin = inverse_cdf(p, uniform(seed, rnd, seq, u_node, EVENT_DRAW))
            return dict(path=path, accept_len=len(path) + 1, next_token=y, flags=flags, margins=margins,
                        draw_margin=draw_margin, stop_node=u_node)
        if draft_logits[u_node] is None:
            flags |= F_BADTREE
            y, draw_margin = inverse_cdf(p, uniform(seed, rnd, seq, u_node, EVENT_DRAW))
            return dict(path=path, accept_len=len(path) + 1, next_token=y, flags=flags, margins=margins,
                        draw_margin=draw_margin, stop_node=u_node)
        q = softmax(np.asarray(draft_logits[u_node], dtype=np.float64))
        accepted = None
        for i, c in enumerate(kids):
            if np.sum(q) <= 0.0:
                flags |= F_QEMPTY
                break
            x = int(token[c])
            r = uniform(seed, rnd, seq, u_node, i)
            if q[x] > 0.0:
                ratio = p[x] / q[x]
                ok = r < ratio
                margins.append(abs(r - ratio))
            else:
                flags |= F_QZERO
                ok = p[x] > 0.0
            if ok:
                accepted = c
                break
            res = np.maximum(0.0, p - q)
            z = np.sum(res)
            if z > 0.0:
                p = res / z
            else:
                flags |= F_ZRES
            if not iid:
                q = q.copy()
                q[x] = 0.0
                s = np.sum(q)
                if s > 0.0:
                    q = q / s
        if accepted is None:
            y, draw_margin = inverse_cdf(p, uniform(seed, rnd, seq, u_node, EVENT_DRAW))
            return dict(path=path, accept_len=len(path) + 1, next_token=y, flags=flags, margins=margins,
                        draw_margin=draw_margin, stop_node=u_node)
        path.append(accepted)
        u_node = accepted


def speculative_sample_one(p, q, x: int, u_accept: float, u_draw: float) -> int:
    """Textbook one-token speculative sampling: accept the draft token x with
    probability min(1, p(x)/q(x)), else draw from norm(max(0, p - q))."""
    p = np.asarray(p, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    if u_accept < min(1.0, p[x] / q[x]):
        return x
    w = np.maximum(0.0, p - q)
    c = np.cumsum(w)
    return int(min(np.searchsorted(c, u_draw * c[-1], side="right"), len(w) - 1))


# --------------------------------------------------------------------------
# Exact law of the verifier's output on tiny vocabularies (brute force).
# --------------------------------------------------------------------------

def _wor_sequences(q, c):
    """All ordered samples of c distinct tokens drawn without replacement from
    q, with their probabilities (fewer when q has fewer than c tokens of
    positive mass)."""
    V = len(q)
    c = min(c, int(np.count_nonzero(np.asarray(q) > 0)))
    for seq in itertools.permutations(range(V), c):
        prob, rem = 1.0, 1.0
        for x in seq:
            if rem <= 0.0 or q[x] <= 0.0:
                prob = 0.0
                break
            prob *= q[x] / rem
            rem -= q[x]
        if prob > 0.0:
            yield seq, prob


def _iid_sequences(q, c):
    V = len(q)
    for seq in itertools.product(range(V), repeat=c):
        prob = float(np.prod([q[x] for x in seq]))
        if prob > 0.0:
            yield seq, prob


def _topk_sequences(q, c):
    order = sorted(range(len(q)), key=lambda i: (-q[i], i))
    yield tuple(order[:c]), 1.0


def exact_round_law(p_of, q_of, nchild_of, proposal: str = "wor", iid_rule: bool = False, max_len: int = 4):
    """Exact distribution of the emitted token tuple of one verification round.

    p_of(prefix) / q_of(prefix): target / draft distributions after a prefix
    (tuple of tokens).  nchild_of(prefix): number of children of the node
    reached by that prefix (0 = leaf).  proposal: how a node's children are
    drawn from its q ("wor" = without replacement, "iid", "topk").
    Returns {tuple(emitted tokens): probability}.
    """
    gen = {"wor": _wor_sequences, "iid": _iid_sequences, "topk": _topk_sequences}[proposal]
    out = {}

    def add(key, pr):
        out[key] = out.get(key, 0.0) + pr

    def node(prefix, weight):
        p0 = np.asarray(p_of(prefix), dtype=np.float64)
        c = nchild_of(prefix) if len(prefix) < max_len else 0
        if c == 0:
            for y in range(len(p0)):
                if p0[y] > 0:
                    add(prefix + (y,), weight * p0[y])
            return
        q0 = np.asarray(q_of(prefix), dtype=np.float64)
        for cands, pr in gen(q0, c):
            walk(prefix, cands, 0, p0, q0, weight * pr)

    def walk(prefix, cands, i, p, q, weight):
        if i == len(cands) or np.sum(q) <= 0.0:
            for y in range(len(p)):
                if p[y] > 0:
                    add(prefix + (y,), weight * p[y])
            return
        x = cands[i]
        a = min(1.0, p[x] / q[x]) if q[x] > 0 else (1.0 if p[x] > 0 else 0.0)
        if a > 0:
            node(prefix + (x,), weight * a)
        if a < 1:
            res = np.maximum(0.0, p - q)
            z = np.sum(res)
            p2 = res / z if z > 0 else p
            q2 = q
            if not iid_rule:
                q2 = q.copy()
                q2[x] = 0.0
                s = np.sum(q2)
                if s > 0:
                    q2 = q2 / s
            walk(prefix, cands, i + 1, p2, q2, weight * (1 - a))

    node((), 1.0)
    return out


def first_token_law(law: dict, V: int) -> np.ndarray:
    m = np.zeros(V)
    for k, pr in law.items():
        m[k[0]] += pr
    return m


def second_token_law(law: dict, V: int, first: int) -> np.ndarray:
    """Law of the second emitted token given that the first emitted token is
    `first` and was an accepted draft (i.e. the round emitted >= 2 tokens)."""
    m = np.zeros(V)
    for k, pr in law.items():
        if len(k) >= 2 and k[0] == first:
            m[k[1]] += pr
    s = m.sum()
    return m / s if s > 0 else m
