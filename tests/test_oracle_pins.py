"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something the pages print, a closed form,
a brute-force enumeration on a tiny input, or a special case that reduces to a
textbook routine -- chosen so that a dropped term, a wrong sign, a wrong index
or a transposed operand anywhere in the oracle fails at least one of them.

Pages: "推测解码" (Speculative decoding, world.lapla.si/zh/specdec) and
"多詞元預測視覺化指南" (A visual guide to multi-token prediction).
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import verify_ref as R
from synth import inputs as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# bf16 decode and the LM-head GEMM
# ---------------------------------------------------------------------------
def _bf16_value_by_fields(bits: int) -> float:
    """Decode bf16 from its sign / 8-bit exponent / 7-bit fraction fields."""
    sign = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_bf16_decode_known_patterns():
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x3F00: 0.5, 0x0001: 2.0 ** -133,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0x8000: -0.0, 0x3FC0: 1.5}
    got = R.bf16_to_f64(np.array(list(cases), dtype=np.uint16))
    assert list(got) == list(cases.values())


def test_bf16_decode_all_finite_patterns_by_fields():
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite].astype(np.uint16)
    got = R.bf16_to_f64(bits)
    ref = np.array([_bf16_value_by_fields(int(b)) for b in bits[::97]])
    np.testing.assert_array_equal(got[::97], ref)


def test_gemm_against_exact_triple_loop():
    rng = np.random.default_rng(11)
    Rr, d, V = 3, 24, 7                    # non-square so a transposed operand fails
    hb = I.f32_to_bf16_bits(rng.standard_normal((Rr, d)).astype(np.float32))
    wb = I.f32_to_bf16_bits(rng.standard_normal((V, d)).astype(np.float32))
    got = R.lmhead_logits(hb, wb)
    assert got.shape == (Rr, V)
    for r in range(Rr):
        for v in range(V):
            exact = sum(Fraction(_bf16_value_by_fields(int(hb[r, k]))) *
                        Fraction(_bf16_value_by_fields(int(wb[v, k]))) for k in range(d))
            assert abs(got[r, v] - float(exact)) <= 1e-13 * max(1.0, abs(float(exact)))


def test_gemm_chunking_is_exact():
    x = I.custom(2, 3, 40, 1000, seed=3)
    H = x["hidden_bits"].reshape(-1, 40)
    a = R.lmhead_logits(H, x["W_bits"])
    b = R.lmhead_logits(H, x["W_bits"], chunk_rows=77)
    np.testing.assert_array_equal(a, b)


# ---------------------------------------------------------------------------
# softmax
# ---------------------------------------------------------------------------
def test_softmax_sums_to_one_and_shift_invariant():
    L = np.random.default_rng(1).standard_normal((6, 5000)) * 4
    p, m, lse = R.softmax_rows(L)
    assert np.all(np.abs(p.sum(-1) - 1) < 1e-12)
    p2, _, lse2 = R.softmax_rows(L + 123.25)
    np.testing.assert_allclose(p2, p, rtol=1e-12, atol=0)   # L + c itself rounds
    np.testing.assert_allclose(lse2 - lse, 123.25, rtol=0, atol=1e-11)
    np.testing.assert_array_equal(m, L.max(-1))


def test_softmax_two_tokens_is_logistic():
    for a, b in [(0.0, 0.0), (1.5, -0.25), (-3.0, 7.0), (700.0, 650.0)]:
        p, _, lse = R.softmax_rows(np.array([[a, b]]))
        assert abs(p[0, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
        assert abs(lse[0] - (max(a, b) + math.log1p(math.exp(-abs(a - b))))) < 1e-12


def test_log_sum_exp_matches_fsum():
    L = np.random.default_rng(2).standard_normal((1, 300)) * 3
    _, _, lse = R.softmax_rows(L)
    assert abs(lse[0] - math.log(math.fsum(math.exp(v) for v in L[0]))) < 1e-12


# ---------------------------------------------------------------------------
# accept test, first rejection
# ---------------------------------------------------------------------------
def _accept_measure(p_x, q_x):
    """Measure of r in (0, 1] the oracle accepts, found by bisection."""
    if R.accept_draft(p_x, q_x, 1.0):
        return 1.0
    lo, hi = 0.0, 1.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        if R.accept_draft(p_x, q_x, mid):
            lo = mid
        else:
            hi = mid
    return lo


def test_page_example_keep_probabilities():
    g = _golden("page_accept_example.json")
    di, man = g["printed"]
    # Underestimated by the drafter (q < p): always kept.
    assert _accept_measure(di["p"], di["q"]) == g["keep_probability"]["地"]
    assert R.accept_draft(di["p"], di["q"], 1.0)
    # Overestimated (q > p): kept with probability p/q = 3/11.
    want = g["keep_probability"]["慢_num"] / g["keep_probability"]["慢_den"]
    assert abs(_accept_measure(man["p"], man["q"]) - want) < 1e-15


def test_accept_tie_and_zero_q():
    assert R.accept_draft(0.25, 0.5, 0.5)          # r == p/q exactly keeps
    assert not R.accept_draft(0.25, 0.5, 0.5 + 2 ** -20)
    assert R.accept_draft(0.0, 0.0, 1.0)           # q == 0 keeps
    assert R.accept_margin(0.1, 0.0, 0.5) == math.inf
    assert abs(R.accept_margin(0.09, 0.33, 0.5) - abs(0.5 - 0.09 / 0.33)) < 1e-16


@pytest.mark.parametrize("gamma", range(1, 9))
def test_first_rejection_all_patterns(gamma):
    for code in range(1 << gamma):
        flags = [bool((code >> i) & 1) for i in range(gamma)]
        text = "".join("1" if f else "0" for f in flags) + "0"
        assert R.first_rejection(flags) == text.index("0")


# ---------------------------------------------------------------------------
# residual and inverse CDF
# ---------------------------------------------------------------------------
def test_residual_sum_is_one_minus_alpha():
    rng = np.random.default_rng(5)
    for _ in range(20):
        p = rng.dirichlet(np.ones(50) * 0.3)
        q = rng.dirichlet(np.ones(50) * 0.3)
        S = R.draw_weights(p, q).sum()
        assert abs(S - (1.0 - R.acceptance_rate(p, q))) < 1e-12


def test_page_example_completed_residual():
    c = _golden("page_accept_example.json")["completed"]
    p, q = np.array(c["p"]), np.array(c["q"])
    assert abs(R.acceptance_rate(p, q) - c["alpha"]) < 1e-15
    w = R.draw_weights(p, q)
    np.testing.assert_allclose(w, c["residual"], atol=1e-15)
    assert abs(w.sum() - c["residual_sum"]) < 1e-15
    assert w[1] == 0.0        # the overestimated token can never be the replacement


def _first_reaching(w, t):
    run = 0.0
    for j, v in enumerate(w):
        run += v
        if run >= t:
            return j
    return None


def test_inverse_cdf_brute_force():
    rng = np.random.default_rng(9)
    for trial in range(50):
        w = rng.random(13)
        w[rng.random(13) < 0.4] = 0.0
        w[rng.integers(13)] = 0.5
        for u in rng.random(20):
            u = 1.0 - u
            y, C, S, t = R.inverse_cdf(w, u)
            assert y == _first_reaching(w, t)
            assert w[y] > 0


def test_inverse_cdf_boundaries_and_u_one():
    w = np.array([0.25, 0.25, 0.5])
    assert R.inverse_cdf(w, 0.25)[0] == 0      # t == C_0 lands on token 0 (smallest j with C_j >= t)
    assert R.inverse_cdf(w, 0.25 + 2 ** -30)[0] == 1
    assert R.inverse_cdf(w, 0.5)[0] == 1
    assert R.inverse_cdf(w, 1.0)[0] == 2
    z = np.array([0.5, 0.0, 0.5, 0.0, 0.0])
    assert R.inverse_cdf(z, 0.5)[0] == 0        # zero-weight token 1 is never drawn
    assert R.inverse_cdf(z, 1.0)[0] == 2        # u = 1 draws the last positive token
    a, b = 0.3, 0.7
    for u in np.linspace(0.01, 1.0, 100):
        assert R.inverse_cdf(np.array([a, b]), u)[0] == (0 if u * (a + b) <= a else 1)


def test_sample_margin_and_admissible():
    w = np.array([0.25, 0.25, 0.5])
    y, C, S, t = R.inverse_cdf(w, 0.3)
    assert y == 1 and abs(R.sample_margin(C, S, t, y) - 0.05) < 1e-15
    assert R.draw_admissible(C, S, 0.3, 1)
    assert not R.draw_admissible(C, S, 0.3, 0)
    assert R.draw_admissible(C, S, 0.25 + 5e-6, 0)     # within the band of the edge


# ---------------------------------------------------------------------------
# the whole step, driven with chosen target probabilities
# ---------------------------------------------------------------------------
def _verify_p(p_rows, q_rows, draft, uniforms):
    """Run the oracle's whole step with target probabilities given directly.

    logits = log p gives softmax(logits) = p; the GEMM inputs are dummies.
    """
    g1, V = p_rows.shape
    hidden = np.zeros((1, g1, 8), dtype=np.uint16)
    W = np.zeros((V, 8), dtype=np.uint16)
    with np.errstate(divide="ignore"):
        L = np.log(p_rows)
    return R.verify(hidden, W, np.asarray(draft, dtype=np.int64)[None], q_rows[None],
                    np.asarray(uniforms, dtype=np.float64)[None], logits=L)


def _prefix_drafts(p_rows, q_rows, upto):
    """Drafts for positions < upto that every r accepts (q <= p there)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        return [int(np.nanargmax(np.where(q_rows[j] > 0, p_rows[j] / q_rows[j], np.inf)))
                for j in range(upto)]


def _emission_by_enumeration(p_rows, q_rows, i):
    """Exact law of the token the whole step emits at position i, given i is reached.

    Enumerates the draft token x (weight q_i(x)); integrates the accept uniform
    and the draw uniform by bisecting the step's own decisions.
    """
    g = q_rows.shape[0]
    V = p_rows.shape[1]
    prefix = _prefix_drafts(p_rows, q_rows, i)
    base_u = np.ones(g + 1)

    def run(draft_i, r_i, u=0.5):
        draft = prefix + [draft_i] + [0] * (g - i - 1) if i < g else prefix
        uu = base_u.copy()
        if i < g:
            uu[i] = r_i
        uu[g] = u
        res = _verify_p(p_rows, q_rows, draft, uu)
        return int(res.n_accepted[0]), int(res.out_tokens[0, i])

    def draw_law(draft_i, r_i):
        # u -> token is a nondecreasing step map; bisect each interval's right edge.
        edges = np.zeros(V)
        for k in range(V):
            lo, hi = 0.0, 1.0
            if run(draft_i, r_i, 1.0)[1] <= k:
                edges[k] = 1.0
                continue
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                if run(draft_i, r_i, mid)[1] <= k:
                    lo = mid
                else:
                    hi = mid
            edges[k] = lo
        return np.diff(np.concatenate([[0.0], edges]))

    if i == g:   # every draft accepted: the bonus token
        return draw_law(None, 1.0)

    law = np.zeros(V)
    rejected_law = None
    for x in range(V):
        if q_rows[i, x] == 0:
            continue
        # accept measure for x at position i
        if run(x, 1.0)[0] > i:
            a = 1.0
        else:
            lo, hi = 0.0, 1.0
            for _ in range(60):
                mid = 0.5 * (lo + hi)
                if run(x, mid)[0] > i:
                    lo = mid
                else:
                    hi = mid
            a = lo
            if rejected_law is None:
                rejected_law = draw_law(x, 1.0)
        law[x] += q_rows[i, x] * a
        if a < 1.0:
            law += q_rows[i, x] * (1.0 - a) * rejected_law
    return law


def test_enumeration_page_example_emits_p():
    c = _golden("page_accept_example.json")["completed"]
    p = np.array([c["p"], c["p"]])
    q = np.array([c["q"]])
    law0 = _emission_by_enumeration(p, q, 0)
    np.testing.assert_allclose(law0, c["p"], atol=1e-12)
    np.testing.assert_allclose(_emission_by_enumeration(p, q, 1), c["p"], atol=1e-12)


@pytest.mark.slow
def test_enumeration_tiny_config_emits_p_at_every_position():
    x = I.generate(I.CONFIGS["tiny"])
    res = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    p_rows = res.p                       # [gamma+1, V] of the one sequence
    q_rows = x["q"][0].astype(np.float64)
    for i in range(q_rows.shape[0] + 1):
        law = _emission_by_enumeration(p_rows, q_rows, i)
        np.testing.assert_allclose(law, p_rows[i], atol=1e-12)


# ---------------------------------------------------------------------------
# Monte Carlo on the tiny config
# ---------------------------------------------------------------------------
def _chi2_pvalue(counts, probs):
    from scipy import stats
    n = counts.sum()
    exp = probs / probs.sum() * n
    order = np.argsort(exp)
    c, e = counts[order].astype(float), exp[order]
    # merge the smallest expected bins until every bin expects >= 5
    k = 0
    while k < len(e) - 1 and e[:k + 1].sum() < 5:
        k += 1
    c = np.concatenate([[c[:k + 1].sum()], c[k + 1:]])
    e = np.concatenate([[e[:k + 1].sum()], e[k + 1:]])
    return stats.chisquare(c, e).pvalue


@pytest.mark.slow
@pytest.mark.parametrize("seed", [101, 202, 303])
def test_monte_carlo_chi_square_tiny(seed):
    base = I.generate(I.CONFIGS["tiny"])
    t = I.repeated_trials(base, 100_000, seed)
    res = R.verify(t["hidden_bits"], t["W_bits"], t["draft"], t["q"], t["uniforms"])
    g = t["draft"].shape[1]
    p_rows = res.p[: g + 1]
    for i in range(g + 1):
        reached = res.n_accepted >= i
        if reached.sum() < 2000:
            continue
        counts = np.bincount(res.out_tokens[reached, i], minlength=p_rows.shape[1])
        assert _chi2_pvalue(counts, p_rows[i]) >= 1e-3, (seed, i)


@pytest.mark.slow
def test_monte_carlo_detects_a_planted_bias():
    """The chi-square check has power: draws from q instead of p fail it."""
    base = I.generate(I.CONFIGS["tiny"])
    res = R.verify(base["hidden_bits"], base["W_bits"], base["draft"], base["q"], base["uniforms"])
    q0 = base["q"][0, 0].astype(np.float64)
    draws = np.random.default_rng(0).choice(q0.shape[0], size=100_000, p=q0 / q0.sum())
    counts = np.bincount(draws, minlength=q0.shape[0])
    assert _chi2_pvalue(counts, res.p[0]) < 1e-6


@pytest.mark.slow
def test_alpha_formula_iid_positions():
    n = 100_000
    x = I.iid_positions(32, 16, 4, n, seed=7)
    res = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    alpha = res.alpha[0, 0]
    assert np.allclose(res.alpha, alpha)
    tokens = res.n_accepted + 1
    se = tokens.std(ddof=1) / math.sqrt(n)
    want = R.expected_tokens_per_step(alpha, 4)
    assert abs(tokens.mean() - want) < 4 * se, (tokens.mean(), want, se)


# ---------------------------------------------------------------------------
# the pages' printed formula values
# ---------------------------------------------------------------------------
def test_page_formula_values():
    g = _golden("page_formula_values.json")
    e = g["expected_tokens"][0]
    v = R.expected_tokens_per_step(e["alpha"], e["gamma"])
    assert round(v, e["printed_digits"]) == e["printed"]
    assert abs(v - 2.4887) < 1e-4
    b = g["best_gamma"][0]
    sp = {gm: R.speedup(b["alpha"], gm, b["c"]) for gm in range(1, 16)}
    best = max(sp, key=sp.get)
    assert best == b["best_gamma"]
    assert round(sp[best], b["printed_digits"]) == b["printed_speedup"]
    a = g["arithmetic_vs_speed"][0]
    tok = R.expected_tokens_per_step(a["alpha"], a["gamma"])
    assert round((tok - 1) * 100) == a["printed_extra_speed_pct"]
    assert round(((a["gamma"] + 1) / tok - 1) * 100) == a["printed_extra_arithmetic_pct"]
    assert R.expected_tokens_per_step(1.0, 4) == 5.0
    assert R.expected_tokens_per_step(0.0, 4) == 1.0


# ---------------------------------------------------------------------------
# special cases of the whole step
# ---------------------------------------------------------------------------
def _rand_dist(rng, V, zeros=None):
    p = rng.dirichlet(np.ones(V))
    if zeros is not None:
        p[zeros] = 0.0
        p /= p.sum()
    return p


def test_q_equal_p_accepts_everything():
    rng = np.random.default_rng(3)
    g, V = 4, 16
    p = np.array([_rand_dist(rng, V) for _ in range(g + 1)])
    for _ in range(200):
        draft = [int(rng.integers(V)) for _ in range(g)]
        u = 1.0 - rng.random(g + 1)
        res = _verify_p(p, p[:g].copy(), draft, u)
        assert res.n_accepted[0] == g
        C = np.cumsum(p[g])
        assert res.out_tokens[0, g] == np.searchsorted(C, u[g] * C[-1], side="left")


def test_disjoint_supports_reject_first_and_draw_from_p():
    rng = np.random.default_rng(4)
    g, V = 3, 16
    p = np.array([_rand_dist(rng, V, zeros=slice(8, 16)) for _ in range(g + 1)])
    q = np.array([_rand_dist(rng, V, zeros=slice(0, 8)) for _ in range(g)])
    for _ in range(100):
        draft = [int(rng.integers(8, 16)) for _ in range(g)]
        u = 1.0 - rng.random(g + 1)
        res = _verify_p(p, q, draft, u)
        assert res.n_accepted[0] == 0
        C = np.cumsum(p[0])
        assert res.out_tokens[0, 0] == np.searchsorted(C, u[g] * C[-1], side="left")
        assert list(res.out_tokens[0, 1:]) == [-1] * g


def test_one_hot_target_is_greedy_match():
    rng = np.random.default_rng(6)
    g, V = 4, 10
    hot = [3, 7, 7, 0, 5]
    p = np.zeros((g + 1, V))
    p[np.arange(g + 1), hot] = 1.0
    q = np.array([_rand_dist(rng, V) for _ in range(g)])
    for _ in range(200):
        draft = [hot[i] if rng.random() < 0.6 else int(rng.integers(V)) for i in range(g)]
        u = 1.0 - rng.random(g + 1)
        res = _verify_p(p, q, draft, u)
        n = next((i for i in range(g) if draft[i] != hot[i]), g)
        assert res.n_accepted[0] == n
        assert list(res.out_tokens[0, :n + 1]) == draft[:n] + [hot[n]]


def test_one_hot_drafter():
    rng = np.random.default_rng(8)
    g, V, x = 1, 12, 5
    p = np.array([_rand_dist(rng, V), _rand_dist(rng, V)])
    q = np.zeros((g, V)); q[0, x] = 1.0
    assert abs(_accept_measure(p[0, x], 1.0) - p[0, x]) < 1e-15
    law = _emission_by_enumeration(p, q, 0)
    np.testing.assert_allclose(law, p[0], atol=1e-12)
    res = _verify_p(p, q, [x], [1.0, 0.5])        # r = 1 rejects unless p(x) = 1
    w = R.draw_weights(p[0], q[0])
    want = p[0].copy(); want[x] = 0.0
    np.testing.assert_allclose(w, want, atol=1e-16)
    assert res.n_accepted[0] == 0 and res.out_tokens[0, 0] != x


def test_out_of_range_draft_is_rejected_and_flagged():
    rng = np.random.default_rng(10)
    g, V = 2, 8
    p = np.array([_rand_dist(rng, V) for _ in range(g + 1)])
    q = np.array([_rand_dist(rng, V) for _ in range(g)])
    for bad in (V, -1, 10 ** 6):
        res = _verify_p(p, q, [bad, 0], [0.001, 0.5, 0.5])
        assert res.n_accepted[0] == 0 and res.bad_draft[0, 0] and not res.accept[0, 0]


def test_residual_fallback_when_q_dominates():
    rng = np.random.default_rng(12)
    g, V = 1, 8
    p = np.array([_rand_dist(rng, V), _rand_dist(rng, V)])
    q = 2.0 * p[:1]                        # not normalised: p - q < 0 everywhere
    x = int(np.argmax(p[0]))
    res = _verify_p(p, q, [x], [0.9, 0.7])  # 0.9 * 2p > p: rejected
    assert res.n_accepted[0] == 0 and res.draw_fallback[0]
    C = np.cumsum(p[0])
    assert res.out_tokens[0, 0] == np.searchsorted(C, 0.7 * C[-1], side="left")


def test_force_n_draws_at_the_forced_row():
    x = I.custom(2, 3, 16, 64, seed=21)
    a = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    for n in range(4):
        f = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"],
                     force_n=np.array([n, n]))
        assert list(f.n_accepted) == [n, n]
        assert list(f.draw_row) == [n, 4 + n]
        for b in range(2):
            if a.n_accepted[b] == n:
                assert list(f.out_tokens[b]) == list(a.out_tokens[b])


def test_output_shape_invariants_random():
    x = I.custom(64, 5, 24, 300, seed=5, sigma=1.5)
    res = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    for b in range(64):
        n = res.n_accepted[b]
        assert 0 <= n <= 5
        assert list(res.out_tokens[b, :n]) == list(x["draft"][b, :n])
        assert 0 <= res.out_tokens[b, n] < 300
        assert all(v == -1 for v in res.out_tokens[b, n + 1:])
        assert res.accept[b, :n].all() and (n == 5 or not res.accept[b, n])
