"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in the oracle (on the CPU, by replacing one of its
step functions for the duration of the test) and checks that at least one pin
from test_oracle_pins fails.  Nothing here touches the GPU path.
"""

import numpy as np
import pytest

from oracle import verify_ref as R
from tests import test_oracle_pins as P


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


MUTANTS = {
    # keep iff r <= q/p instead of r <= p/q
    "accept_inverted_ratio": ("accept_draft", lambda p, q, r: bool(r * p <= q)),
    # strict inequality: ties reject
    "accept_strict": ("accept_draft", lambda p, q, r: bool(r * q < p)),
    # residual with the wrong sign
    "residual_sign": ("draw_weights",
                      lambda p, q: p.copy() if q is None else np.maximum(0.0, q.astype(float) - p)),
    # replacement drawn from p instead of the residual
    "residual_dropped": ("draw_weights", lambda p, q: p.copy()),
    # bonus drawn from the residual of the last draft row is not expressible
    # here; a count of all accepts instead of the leading ones is:
    "count_not_prefix": ("first_rejection", lambda flags: int(sum(bool(f) for f in flags))),
    # inverse CDF that takes the first C_j > t (other boundary convention)
    "cdf_right": ("inverse_cdf",
                  lambda w, u: (lambda C: (int(np.searchsorted(C, float(u) * C[-1], "right")),
                                           C, float(C[-1]), float(u) * C[-1]))(np.cumsum(w))),
    # inverse CDF without the normalisation by S
    "cdf_unnormalised": ("inverse_cdf",
                         lambda w, u: (lambda C: (min(int(np.searchsorted(C, float(u), "left")),
                                                      len(w) - 1), C, float(C[-1]), float(u)))(np.cumsum(w))),
    # softmax that forgets to subtract the log-normaliser
    "softmax_unnormalised": ("softmax_rows",
                             lambda L: (np.exp(L - L.max(-1, keepdims=True)), L.max(-1), L.max(-1))),
    # transposed GEMM operand order (hidden against W's columns)
    "gemm_wrong_rows": ("lmhead_logits",
                        lambda h, W, chunk_rows=8192: R.bf16_to_f64(h) @ R.bf16_to_f64(W)[::-1].T),
}

PINS = [
    (P.test_page_example_keep_probabilities, ()),
    (P.test_accept_tie_and_zero_q, ()),
    (P.test_first_rejection_all_patterns, (4,)),
    (P.test_page_example_completed_residual, ()),
    (P.test_inverse_cdf_brute_force, ()),
    (P.test_inverse_cdf_boundaries_and_u_one, ()),
    (P.test_enumeration_page_example_emits_p, ()),
    (P.test_one_hot_target_is_greedy_match, ()),
    (P.test_disjoint_supports_reject_first_and_draw_from_p, ()),
    (P.test_residual_fallback_when_q_dominates, ()),
    (P.test_softmax_sums_to_one_and_shift_invariant, ()),
    (P.test_softmax_two_tokens_is_logistic, ()),
    (P.test_gemm_against_exact_triple_loop, ()),
    (P.test_output_shape_invariants_random, ()),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    caught = []
    for pin, args in PINS:
        try:
            if _fails(pin, *args):
                caught.append(pin.__name__)
        except Exception:            # a crash under the mutant also counts as caught
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"


# --------------------------------------------------------------------------
# Greedy verification oracle.
# --------------------------------------------------------------------------
from oracle import greedy_ref as G          # noqa: E402
from tests import test_oracle_greedy_pins as GP   # noqa: E402


def _last_max(L):
    M = np.where(np.isnan(L), -np.inf, L)
    flipped = np.argmax(M[..., ::-1], axis=-1)
    arg = (M.shape[-1] - 1 - flipped).astype(np.int64)
    arg[~(M.max(axis=-1) > -np.inf)] = -1
    return arg


_ORIG_GT = G.greedy_tokens

GREEDY_MUTANTS = {
    # ties resolved to the highest id
    "argmax_last": ("greedy_tokens", _last_max),
    # each row judged by the next row's greedy token
    "argmax_next_row": ("greedy_tokens", lambda L: np.roll(_ORIG_GT(L), -1)),
    # argmin instead of argmax
    "argmin": ("greedy_tokens", lambda L: np.argmin(np.where(np.isnan(L), np.inf, L), axis=-1)),
    # a count of all matches instead of the leading ones
    "count_not_prefix": ("first_rejection", lambda flags: int(sum(bool(f) for f in flags))),
    # transposed GEMM operand order
    "gemm_wrong_rows": ("lmhead_logits",
                        lambda h, W, chunk_rows=8192: R.bf16_to_f64(h) @ R.bf16_to_f64(W)[::-1].T),
}
GREEDY_PINS = [
    (GP.test_greedy_token_hand_cases, ()),
    (GP.test_emitted_tokens_are_the_targets_own_all_drafts, ()),
    (GP.test_low_temperature_sampling_rule_is_greedy, ()),
    (GP.test_exact_tie_goes_to_lowest_id, ()),
    (GP.test_random_config_invariants, ()),
]


@pytest.mark.parametrize("name", sorted(GREEDY_MUTANTS))
def test_some_greedy_pin_catches(name, monkeypatch):
    attr, fn = GREEDY_MUTANTS[name]
    monkeypatch.setattr(G, attr, fn)
    caught = []
    for pin, args in GREEDY_PINS:
        try:
            if _fails(pin, *args):
                caught.append(pin.__name__)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"


# --------------------------------------------------------------------------
# Clustered sparse head oracle.
# --------------------------------------------------------------------------
from oracle import sparse_ref as S            # noqa: E402
from tests import test_oracle_sparse_pins as SP   # noqa: E402

_ORIG_SEL = S.selected_tokens

SPARSE_MUTANTS = {
    # the k smallest cluster logits
    "topk_smallest": ("top_clusters", lambda s, k: np.sort(np.argsort(s, kind="stable")[:k])),
    # ties to the higher index
    "topk_ties_high": ("top_clusters",
                       lambda s, k: np.sort(len(s) - 1 - np.argsort(-s[::-1], kind="stable")[:k])),
    # members of the neighbouring clusters
    "wrong_members": ("selected_tokens",
                      lambda m, c: _ORIG_SEL(m, (c + 1) % m.shape[0])),
    # centroid table transposed against the hidden rows (rows reversed)
    "cluster_scores_reversed": ("cluster_logits",
                                lambda h, c: R.bf16_to_f64(h) @ R.bf16_to_f64(c)[::-1].T),
}

SPARSE_PINS = [
    (SP.test_top_clusters_hand_cases, ()),
    (SP.test_top_clusters_brute_force, ()),
    (SP.test_all_clusters_is_the_full_softmax, ()),
    (SP.test_singleton_clusters_select_top_tokens, ()),
    (SP.test_values_follow_exact_logit_ratios, ()),
]


@pytest.mark.parametrize("name", sorted(SPARSE_MUTANTS))
def test_some_sparse_pin_catches(name, monkeypatch):
    attr, fn = SPARSE_MUTANTS[name]
    monkeypatch.setattr(S, attr, fn)
    caught = []
    for pin, args in SPARSE_PINS:
        try:
            if _fails(pin, *args):
                caught.append(pin.__name__)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
