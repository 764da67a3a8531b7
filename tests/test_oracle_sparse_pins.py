"""Pins of the clustered sparse-head oracle ("多詞元預測視覺化指南", section
高效嵌入器) to facts fixed outside it:

  * selecting every cluster turns the sparse head into the plain softmax
    over the whole vocabulary, which the dense oracle pins independently;
  * one token per cluster with the token's own row as its embedding turns
    cluster selection into top-k over the exact token logits;
  * the top-k rule against a brute-force tuple sort, with ties;
  * q values against ratios of exact token logits computed on the full W.
"""

import numpy as np
import pytest

from oracle import sparse_ref as S
from oracle import verify_ref as R
from synth import inputs as I


def _bits(rng, shape, scale=1.0):
    return I.f32_to_bf16_bits((scale * rng.standard_normal(shape)).astype(np.float32))


def _clusters(rng, V, M):
    return rng.permutation(V).reshape(V // M, M)


def test_top_clusters_hand_cases():
    s = np.array([0.5, 2.0, 2.0, -1.0, 2.0, 0.7])
    assert list(S.top_clusters(s, 1)) == [1]
    assert list(S.top_clusters(s, 2)) == [1, 2]
    assert list(S.top_clusters(s, 4)) == [1, 2, 4, 5]
    assert list(S.top_clusters(s, 6)) == [0, 1, 2, 3, 4, 5]
    assert S.topk_margin(s, 2) == 0.0 and S.topk_margin(s, 3) == pytest.approx(1.3)
    assert S.topk_margin(s, 6) == float("inf")


def test_top_clusters_brute_force():
    rng = np.random.default_rng(21)
    for _ in range(300):
        C = int(rng.integers(1, 12))
        k = int(rng.integers(1, C + 1))
        s = rng.integers(-3, 4, size=C).astype(float)      # frequent ties
        want = sorted(i for _, i in sorted((-float(v), i) for i, v in enumerate(s))[:k])
        assert list(S.top_clusters(s, k)) == want


def test_all_clusters_is_the_full_softmax():
    rng = np.random.default_rng(22)
    N, d, V, M = 3, 24, 96, 8
    h, W = _bits(rng, (N, d)), _bits(rng, (V, d), 0.3)
    members = _clusters(rng, V, M)
    cent = _bits(rng, (V // M, d), 0.3)
    res = S.sparse_head(h, W, cent, members, k=V // M)
    p, _, _ = R.softmax_rows(R.lmhead_logits(h, W))
    for n in range(N):
        assert list(res.idx[n]) == list(range(V))
        np.testing.assert_allclose(res.val[n], p[n], rtol=1e-12, atol=0)


def test_singleton_clusters_select_top_tokens():
    rng = np.random.default_rng(23)
    N, d, V, k = 4, 16, 50, 7
    h, W = _bits(rng, (N, d)), _bits(rng, (V, d), 0.3)
    members = np.arange(V)[:, None]
    res = S.sparse_head(h, W, W, members, k)
    L = R.lmhead_logits(h, W)
    for n in range(N):
        top = np.sort(np.argsort(-L[n], kind="stable")[:k])
        assert list(res.idx[n]) == list(top)
        e = np.exp(L[n, top] - L[n, top].max())
        np.testing.assert_allclose(res.val[n], e / e.sum(), rtol=1e-12)


def test_values_follow_exact_logit_ratios():
    rng = np.random.default_rng(24)
    N, d, V, M, k = 3, 32, 256, 16, 4
    h, W = _bits(rng, (N, d)), _bits(rng, (V, d), 0.3)
    members = _clusters(rng, V, M)
    cent = _bits(rng, (V // M, d), 0.3)
    res = S.sparse_head(h, W, cent, members, k)
    L = R.lmhead_logits(h, W)
    scores = R.bf16_to_f64(h) @ R.bf16_to_f64(cent).T
    for n in range(N):
        assert res.idx.shape[1] == k * M and np.all(np.diff(res.idx[n]) > 0)
        # every chosen cluster scores at least as high as every other
        chosen = set(res.clusters[n].tolist())
        lo = min(scores[n, c] for c in chosen)
        assert all(scores[n, c] <= lo for c in range(V // M) if c not in chosen)
        # the selected ids are exactly the chosen clusters' members
        assert set(res.idx[n].tolist()) == set(members[list(chosen)].ravel().tolist())
        assert abs(res.val[n].sum() - 1.0) < 1e-12
        j0 = res.idx[n, 0]
        np.testing.assert_allclose(res.val[n] / res.val[n, 0], np.exp(L[n, res.idx[n]] - L[n, j0]),
                                   rtol=1e-11)


def test_densify_and_verify_with_sparse_q():
    rng = np.random.default_rng(25)
    B, g, d, V, M, k = 2, 3, 16, 64, 8, 2
    hid = _bits(rng, (B, g + 1, d))
    W = _bits(rng, (V, d), 0.3)
    members = _clusters(rng, V, M)
    cent = _bits(rng, (V // M, d), 0.3)
    res = S.sparse_head(hid[:, :g].reshape(-1, d), W, cent, members, k)
    q = S.densify(res.idx.reshape(B, g, -1), res.val.reshape(B, g, -1), V)
    assert q.shape == (B, g, V)
    np.testing.assert_allclose(q.sum(-1), 1.0, atol=1e-12)
    for b in range(B):
        for i in range(g):
            r = b * g + i
            off = np.setdiff1d(np.arange(V), res.idx[r])
            assert np.all(q[b, i, off] == 0.0)
            assert np.array_equal(q[b, i, res.idx[r]], res.val[r])
    # drafts from the sparse q, then the dense oracle on the densified q
    draft = np.array([[int(rng.choice(res.idx[b * g + i], p=res.val[b * g + i])) for i in range(g)]
                      for b in range(B)])
    u = 1.0 - rng.random((B, g + 1))
    out = R.verify(hid, W, draft, q.astype(np.float32), u)
    assert np.all(out.q_draft > 0)           # every drafted id lies in its row's support
