"""Pins of the greedy-verification oracle to facts fixed outside it.

Greedy (match) verification keeps drafts while they equal the target's own
greedy token and emits the target's token at the first mismatch, so that the
output is exactly what the target alone would have written (the
maxstudionews.com article 1664 on multi-token prediction for Gemini Nano,
paragraphs on the draft / verify split and on bit-identical output).  The pins:

  * hand-built rows with known maxima, ties and NaN;
  * the low-temperature limit of the sampling rule ("推测解码", section
    通过的规则): with p one-hot at the greedy token, keep-with-probability
    min(1, p/q) keeps exactly the matching drafts and the residual
    max(0, p - q) puts all its weight on the greedy token -- so the
    independently pinned sampling oracle, fed logits / T with T -> 0, must
    reproduce the greedy oracle for every q and every uniform;
  * exhaustive enumeration of all drafts on a tiny vocabulary against the
    "target alone" statement: the emitted tokens are the target's greedy
    tokens of rows 0..n and n is the length of the common prefix.
"""

import numpy as np
import pytest

from oracle import greedy_ref as G
from oracle import verify_ref as R
from synth import inputs as I


def _hidden_W(rng, g1, d, V):
    h = I.f32_to_bf16_bits(rng.standard_normal((1, g1, d)).astype(np.float32))
    W = I.f32_to_bf16_bits((0.3 * rng.standard_normal((V, d))).astype(np.float32))
    return h, W


def test_greedy_token_hand_cases():
    nan, inf = float("nan"), float("inf")
    cases = [([1.0, 3.0, 3.0, 2.0], 1), ([5.0], 0), ([nan, 2.0, 2.0], 1), ([2.0, nan, 7.0], 2),
             ([-inf, -inf], -1), ([nan, nan], -1), ([-inf, nan, -3.0], 2), ([inf, inf, 1.0], 0),
             ([0.0, -0.0], 0), ([-1e300, -1e299], 1)]
    for row, want in cases:
        a = np.array(row)
        assert G.greedy_token(a) == want, row
        assert G.greedy_tokens(a[None])[0] == want, row


def test_vectorised_matches_scan_random_with_ties():
    rng = np.random.default_rng(11)
    L = rng.integers(-3, 4, size=(200, 9)).astype(np.float64)   # many exact ties
    L[rng.random(L.shape) < 0.05] = np.nan
    for r in range(L.shape[0]):
        assert G.greedy_tokens(L[r:r + 1])[0] == G.greedy_token(L[r])


def test_top_gap_and_near_ties():
    row = np.array([0.5, 2.0, 2.00005, -1.0, 1.9])
    y = G.greedy_token(row)
    assert y == 2
    assert G.top_gap(row, y) == pytest.approx(5e-5, abs=1e-12)
    assert list(G.near_ties(row)) == [1, 2]
    assert list(G.near_ties(row, band=0.2)) == [1, 2, 4]


def test_emitted_tokens_are_the_targets_own_all_drafts():
    """Every draft sequence over a 4-token vocabulary, gamma = 3."""
    rng = np.random.default_rng(12)
    g, d, V = 3, 8, 4
    h, W = _hidden_W(rng, g + 1, d, V)
    L = R.lmhead_logits(h.reshape(g + 1, d), W)
    t = [int(np.argmax(L[i])) for i in range(g + 1)]
    for code in range(V ** g):
        draft = [(code // V ** i) % V for i in range(g)]
        res = G.verify_greedy(h, W, np.array([draft]))
        n = 0
        while n < g and draft[n] == t[n]:
            n += 1
        assert res.n_accepted[0] == n
        assert list(res.out_tokens[0]) == t[:n + 1] + [-1] * (g - n)


def test_low_temperature_sampling_rule_is_greedy():
    rng = np.random.default_rng(13)
    g, d, V, B = 4, 16, 12, 1
    checked = 0
    for trial in range(60):
        h, W = _hidden_W(rng, g + 1, d, V)
        L = R.lmhead_logits(h.reshape(g + 1, d), W)
        gaps = [G.top_gap(L[i], G.greedy_token(L[i])) for i in range(g + 1)]
        if min(gaps) < 1e-3:
            continue
        T = min(gaps) / 2000.0          # every non-maximal p underflows to exactly 0
        tgt = G.greedy_tokens(L)
        draft = np.array([[tgt[i] if rng.random() < 0.7 else int(rng.integers(V)) for i in range(g)]])
        q = rng.dirichlet(np.ones(V), size=(B, g))
        for _ in range(5):
            u = 1.0 - rng.random((B, g + 1))
            samp = R.verify(h, W, draft, q, u, logits=L / T)
            assert np.array_equal(samp.p, (np.arange(V)[None] == tgt[:, None]).astype(float))
            gr = G.verify_greedy(h, W, draft, logits=L)
            assert samp.n_accepted[0] == gr.n_accepted[0]
            assert list(samp.out_tokens[0]) == list(gr.out_tokens[0])
            checked += 1
    assert checked >= 100


def test_bad_draft_never_matches_and_nan_row_is_flagged():
    rng = np.random.default_rng(14)
    g, d, V = 3, 8, 6
    h, W = _hidden_W(rng, g + 1, d, V)
    L = R.lmhead_logits(h.reshape(g + 1, d), W)
    t = G.greedy_tokens(L)
    res = G.verify_greedy(h, W, np.array([[t[0], V + 3, t[2]]]))
    assert res.n_accepted[0] == 1 and res.bad_draft[0, 1] and not res.bad_draft[0, 0]
    assert list(res.out_tokens[0]) == [t[0], t[1], -1, -1]
    # a NaN hidden entry makes every logit of its row NaN
    h2 = h.copy()
    h2[0, 0, 0] = 0x7FC0
    res = G.verify_greedy(h2, W, np.array([[t[0], t[1], t[2]]]))
    assert res.target[0, 0] == -1 and res.n_accepted[0] == 0
    assert res.nonfinite[0] and res.out_tokens[0, 0] == 0


def test_exact_tie_goes_to_lowest_id():
    rng = np.random.default_rng(15)
    g, d, V = 2, 8, 10
    h, W = _hidden_W(rng, g + 1, d, V)
    L = R.lmhead_logits(h.reshape(g + 1, d), W)
    y = int(np.argmax(L[1]))
    W2 = np.concatenate([W[:y], W[y:y + 1], W[y:]])   # duplicate row y at y and y+1
    res = G.verify_greedy(h, W2, np.array([[0, 0]]))
    assert res.target[0, 1] == y and res.gap[0, 1] == 0.0 and res.flagged[0, 1]


def test_random_config_invariants():
    x = I.custom(3, 5, 40, 300, seed=16)
    rng = np.random.default_rng(16)
    L = R.lmhead_logits(x["hidden_bits"].reshape(-1, 40), x["W_bits"])
    tgt = G.greedy_tokens(L).reshape(3, 6)
    draft = np.where(rng.random((3, 5)) < 0.8, tgt[:, :5], x["draft"])
    res = G.verify_greedy(x["hidden_bits"], x["W_bits"], draft)
    for b in range(3):
        n = int(res.n_accepted[b])
        assert list(res.out_tokens[b, :n + 1]) == list(tgt[b, :n + 1])
        assert all(v == -1 for v in res.out_tokens[b, n + 1:])
        assert n == 5 or draft[b, n] != tgt[b, n]
    forced = G.verify_greedy(x["hidden_bits"], x["W_bits"], draft, force_n=np.array([0, 5, 2]),
                             logits=L)
    assert [int(forced.out_tokens[b, k]) for b, k in enumerate([0, 5, 2])] == \
        [int(tgt[0, 0]), int(tgt[1, 5]), int(tgt[2, 2])]
