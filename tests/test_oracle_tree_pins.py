"""Pins of the tree-verification oracle to facts fixed outside it.

  * A path topology is the chain step: the chain oracle gives the same
    tokens, counts, margins and draws on random inputs.
  * Exact enumeration: with each fork's candidates drawn independently from
    the drafter's q, the first emitted token is distributed as p of the root
    row, and the token after a kept node as p of that node's row -- the
    distribution-preserving property the pages attribute to EAGLE's rule at
    every fork.  Candidate tokens are enumerated with their q weights; the
    accept and draw uniforms are integrated by bisecting the oracle's own
    decisions.
  * The residual after j sibling rejections equals max(0, p - c_j q) / S_j
    with c_0 = 0, S_0 = 1, c_{j+1} = c_j + S_j (a closed form checked against
    the oracle's step-by-step residuals).
  * The worst-case count of residual sums against a brute-force walk over
    every keep/reject sequence.
  * Planted mistakes in the sibling step fail the enumeration.
"""

import itertools

import numpy as np
import pytest

from oracle import tree_ref as TR
from oracle import verify_ref as R
from synth import inputs as I


def _dist(rng, V, zeros=()):
    x = rng.random(V) + 0.05
    x[list(zeros)] = 0.0
    return x / x.sum()


def _run(p_rows, q_rows, parent, tokens, uniforms, force_path=None):
    """The oracle with target probabilities given directly (logits = log p)."""
    T1, V = p_rows.shape
    hidden = np.zeros((1, T1, 8), dtype=np.uint16)
    W = np.zeros((V, 8), dtype=np.uint16)
    with np.errstate(divide="ignore"):
        L = np.log(p_rows)
    return TR.verify_tree(hidden, W, parent, np.asarray(tokens, dtype=np.int64)[None],
                          q_rows[None], np.asarray(uniforms, dtype=np.float64)[None], logits=L,
                          force_path=None if force_path is None else [force_path])


# ---------------------------------------------------------------------------
def test_topology_helpers():
    parent = [-1, -1, 0, 0, 2, -1]
    assert TR.children(parent, -1) == [0, 1, 5]
    assert TR.children(parent, 0) == [2, 3]
    assert TR.children(parent, 3) == []
    assert list(TR.depth_of(parent)) == [1, 1, 2, 2, 3, 1]
    assert TR.max_depth(parent) == 3
    # rows with children: root (row 0), node 0 (row 1), node 2 (row 3)
    assert list(TR.q_slots(parent)) == [0, 1, -1, 2, -1, -1, -1]
    with pytest.raises(ValueError):
        TR.check_topology([-1, 2, 0])


def test_path_topology_is_the_chain_step():
    rng = np.random.default_rng(0)
    for trial in range(60):
        g = int(rng.integers(1, 6))
        V = int(rng.integers(2, 40))
        x = I.custom(1, g, 16, V, seed=int(rng.integers(1 << 30)), sigma=float(rng.uniform(0.2, 2)))
        chain = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
        tree = TR.verify_tree(x["hidden_bits"], x["W_bits"], list(range(-1, g - 1)), x["draft"],
                              x["q"], x["uniforms"], logits=chain.logits)
        np.testing.assert_array_equal(tree.out_tokens, chain.out_tokens)
        np.testing.assert_array_equal(tree.n_accepted, chain.n_accepted)
        assert tree.draw_margin[0] == chain.draw_margin[0]
        assert tree.draw_row[0] == chain.draw_row[0]
        np.testing.assert_array_equal(tree.draw_cdf[0], chain.draw_cdf[0])
        tested = [m for (_, _, m, _) in tree.tests[0]]
        n = int(chain.n_accepted[0])
        np.testing.assert_array_equal(tested, chain.accept_margin[0, :min(n + 1, g)])


# ---------------------------------------------------------------------------
# Exact enumeration of the emitted token's law at one fork
# ---------------------------------------------------------------------------
def _bisect(pred, iters=64):
    """Largest r in (0, 1] with pred(r) true, for pred true on (0, a] and false above."""
    if pred(1.0):
        return 1.0
    lo, hi = 0.0, 1.0
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return lo


def _fork_law(p_rows, q_rows, parent, v, depth_index, base_tokens, force_path):
    """Law of the token emitted at out[depth_index] when the walk is at node v
    (the forced path leads there): enumerate v's children's tokens (weights
    q at v's row), integrate their accept uniforms and the draw uniform."""
    T1, V = p_rows.shape
    T = T1 - 1
    kids = TR.children(parent, v)
    slot = TR.q_slots(parent)[v + 1]
    law = np.zeros(V)
    for combo in itertools.product(range(V), repeat=len(kids)):
        weight = np.prod([q_rows[slot, x] for x in combo])
        if weight == 0.0:
            continue
        tokens = np.array(base_tokens)
        for t, x in zip(kids, combo):
            tokens[t] = x

        def run(rs, u):
            uu = np.ones(T + 1)
            for t, r in zip(kids, rs):
                uu[t] = r
            uu[T] = u
            return _run(p_rows, q_rows, parent, tokens, uu, force_path)

        reach = 1.0
        rs = [1.0] * len(kids)
        for j, t in enumerate(kids):
            def kept(r, j=j, t=t):
                rr = list(rs)
                rr[j] = r
                res = run(rr, 0.5)
                return res.n_accepted[0] > depth_index and res.path_nodes[0, depth_index] == t
            a = _bisect(kept)
            law[combo[j]] += weight * reach * a
            reach *= 1.0 - a
            if reach == 0.0:
                break
        if reach > 0.0:
            # every child rejected (all r = 1): the draw's law, by bisecting u
            edges = np.zeros(V)
            for k in range(V):
                edges[k] = _bisect(lambda u: run(rs, u).out_tokens[0, depth_index] <= k)
            law += weight * reach * np.diff(np.concatenate([[0.0], edges]))
    return law


TREES = [
    [-1, -1],                    # two candidates at the root
    [-1, -1, -1],                # three
    [-1, -1, 0, 0, 1],           # two levels, uneven
    [-1, 0, 0, -1],
]


@pytest.mark.parametrize("parent", TREES)
def test_enumeration_first_token_is_p(parent):
    rng = np.random.default_rng(len(parent) * 7 + parent.count(-1))
    V = 4
    T = len(parent)
    P = int((TR.q_slots(parent) >= 0).sum())
    p_rows = np.array([_dist(rng, V) for _ in range(T + 1)])
    q_rows = np.array([_dist(rng, V, zeros=[3] if s == 0 else []) for s in range(P)])
    law = _fork_law(p_rows, q_rows, parent, -1, 0, np.zeros(T, dtype=np.int64), None)
    np.testing.assert_allclose(law, p_rows[0], atol=1e-12)


def test_enumeration_after_a_kept_node_is_p_of_its_row():
    parent = [-1, -1, 0, 0, 0, 1]
    rng = np.random.default_rng(5)
    V = 4
    p_rows = np.array([_dist(rng, V) for _ in range(7)])
    q_rows = np.array([_dist(rng, V) for _ in range(3)])
    # keep node 0 (forced), then node 0's three children compete
    law = _fork_law(p_rows, q_rows, parent, 0, 1, np.zeros(6, dtype=np.int64), [0])
    np.testing.assert_allclose(law, p_rows[1], atol=1e-12)
    # keep node 1: one child, whose row is a leaf
    law = _fork_law(p_rows, q_rows, parent, 1, 1, np.zeros(6, dtype=np.int64), [1])
    np.testing.assert_allclose(law, p_rows[2], atol=1e-12)


def test_enumeration_page_example_with_two_candidates():
    # the page's example, completed with a third token: p = (.32, .09, .59), q = (.13, .33, .54)
    p = np.array([0.32, 0.09, 0.59])
    q = np.array([0.13, 0.33, 0.54])
    parent = [-1, -1]
    law = _fork_law(np.array([p, p, p]), np.array([q]), parent, -1, 0, np.zeros(2, dtype=np.int64),
                    None)
    np.testing.assert_allclose(law, p, atol=1e-12)


# ---------------------------------------------------------------------------
def test_residual_closed_form():
    """The oracle's residuals (renormalised at every step) against the closed
    form max(0, p - c_j q) with c_0 = 0, c_{j+1} = c_j + S_j, where S_j is the
    sum of the unnormalised closed form itself (S_0 = sum p = 1)."""
    rng = np.random.default_rng(3)
    for _ in range(200):
        V = int(rng.integers(2, 30))
        p = _dist(rng, V)
        q = _dist(rng, V, zeros=rng.choice(V, size=int(rng.integers(0, V // 2 + 1)), replace=False))
        cur, c, S_j = p, 0.0, 1.0
        for j in range(6):
            res, S = TR.residual(cur, q)
            c = c + S_j
            closed = np.maximum(0.0, p - c * q)
            if not S > 0:
                assert closed.sum() <= 1e-12
                break
            np.testing.assert_allclose(closed / closed.sum(), res / S, atol=1e-12)
            cur, S_j = res / S, float(closed.sum())


def _walk_rounds_brute_force(parent):
    """Max over every keep/reject sequence of (sums needed + the draw)."""
    best = 0

    def go(v, sums):
        nonlocal best
        kids = TR.children(parent, v)
        if not kids:
            best = max(best, sums + 1)
            return
        for kept_at in range(len(kids) + 1):       # len(kids): every child rejected
            if kept_at == len(kids):
                best = max(best, sums + (len(kids) - 1) + 1)
            else:
                go(kids[kept_at], sums + kept_at)

    go(-1, 0)
    return best


def test_worst_case_rounds_brute_force():
    rng = np.random.default_rng(4)
    assert TR.worst_case_rounds([0 - 1]) == 1
    assert TR.worst_case_rounds(list(range(-1, 7))) == 1          # a chain: one draw
    for _ in range(300):
        T = int(rng.integers(1, 12))
        parent = [int(rng.integers(-1, t)) for t in range(T)]
        assert TR.worst_case_rounds(parent) == _walk_rounds_brute_force(parent), parent


# ---------------------------------------------------------------------------
# Planted mistakes in the sibling step must fail the enumeration.
# ---------------------------------------------------------------------------
def _law_with(monkeypatch, fake):
    monkeypatch.setattr(TR, "residual", fake)
    rng = np.random.default_rng(11)
    p_rows = np.array([_dist(rng, 4) for _ in range(4)])
    q_rows = np.array([_dist(rng, 4)])
    law = _fork_law(p_rows, q_rows, [-1, -1, -1], -1, 0, np.zeros(3, dtype=np.int64), None)
    return law, p_rows[0]


@pytest.mark.parametrize("mistake", ["no_update", "sign", "no_clip"])
def test_planted_sibling_mistakes_are_caught(monkeypatch, mistake):
    real = TR.residual

    def fake(cur, q_row):
        if mistake == "no_update":        # later siblings tested against p again
            return cur * 1.0, 1.0
        if mistake == "sign":             # max(0, q - cur)
            w = np.maximum(0.0, q_row - cur)
            return w, float(w.sum())
        w = cur - 0.5 * q_row             # wrong residual, not clipped
        w = np.abs(w)
        return w, float(w.sum())

    law, p0 = _law_with(monkeypatch, fake)
    assert np.abs(law - p0).max() > 1e-3, mistake
    monkeypatch.setattr(TR, "residual", real)
    law, p0 = _law_with(monkeypatch, real)
    np.testing.assert_allclose(law, p0, atol=1e-12)
