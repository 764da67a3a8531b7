"""The seeded input generator: determinism, bf16 rounding and the config recipes."""

import numpy as np
import pytest
import torch

from synth import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200_000).astype(np.float32) * s for s in (1e-3, 1, 1e3)])
    # exact ties: low 16 bits 0x8000, both parities of bit 16
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32) + 0x3F800000
    x = np.concatenate([x, ties.view(np.float32)])
    ours = I.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_deterministic_and_shapes():
    a = I.custom(3, 4, 40, 500, seed=7)
    b = I.custom(3, 4, 40, 500, seed=7)
    c = I.custom(3, 4, 40, 500, seed=8)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["W_bits"], c["W_bits"])
    assert a["hidden_bits"].shape == (3, 5, 40) and a["hidden_bits"].dtype == np.uint16
    assert a["W_bits"].shape == (500, 40) and a["W_bits"].dtype == np.uint16
    assert a["draft"].shape == (3, 4) and a["draft"].dtype == np.int32
    assert a["q"].shape == (3, 4, 500) and a["q"].dtype == np.float32
    assert a["uniforms"].shape == (3, 5) and a["uniforms"].dtype == np.float32
    assert np.all(a["uniforms"] > 0) and np.all(a["uniforms"] <= 1)
    assert np.all((a["draft"] >= 0) & (a["draft"] < 500))
    np.testing.assert_allclose(a["q"].sum(-1), 1.0, atol=1e-5)


def test_tensor_streams_independent_of_other_shapes():
    a = I.custom(2, 4, 40, 500, seed=7)
    b = I.custom(2, 4, 40, 600, seed=7)
    # W rows of the shared chunk and the hidden states do not depend on V
    np.testing.assert_array_equal(a["W_bits"], b["W_bits"][:500])
    np.testing.assert_array_equal(a["hidden_bits"], b["hidden_bits"])
    np.testing.assert_array_equal(a["uniforms"], b["uniforms"])


def test_weight_std_recipe():
    x = I.custom(1, 1, 256, 4096, w_std=0.02, seed=1)
    w = I.bf16_bits_to_f32(x["W_bits"])
    assert abs(w.std() - 0.02) < 0.0005 and abs(w.mean()) < 0.0005


def test_gumbel_drafts_follow_q():
    rng = np.random.default_rng(0)
    q = rng.dirichlet(np.ones(8)).astype(np.float32)
    base = {"hidden_bits": np.zeros((1, 2, 8), np.uint16), "W_bits": np.zeros((8, 8), np.uint16),
            "draft": np.zeros((1, 1), np.int32), "q": q[None, None, :], "uniforms": np.ones((1, 2), np.float32)}
    t = I.repeated_trials(base, 200_000, seed=3)
    freq = np.bincount(t["draft"][:, 0], minlength=8) / 200_000
    np.testing.assert_allclose(freq, q, atol=0.004)


def test_sparse_q_structure():
    cfg = I.Config("sparse_small", 2, 3, 32, 64 * 16, 0.5, 1.0, 0.5, sparse=(64, 16, 4), seed=2)
    x = I.generate(cfg)
    nz = (x["q"] > 0).sum(-1)
    assert np.all(nz == 4 * 16)
    for b in range(2):
        for i in range(3):
            assert x["q"][b, i, x["draft"][b, i]] > 0


def test_config_registry_shapes():
    c = I.CONFIGS
    assert (c["tiny"].V, c["tiny"].d, c["tiny"].gamma, c["tiny"].B) == (32, 16, 4, 1)
    assert (c["gemma_e2b"].V, c["gemma_e2b"].d, c["gemma_e2b"].R) == (262144, 1536, 5)
    assert c["llama8b_g8_b4"].R == 36 and c["sweep_b256_s1.0"].R == 1280
    assert c["sparse_q"].sparse == (2048, 128, 32) and c["sparse_q"].R == 40


def test_to_sparse_q_lists_every_nonzero_once_with_repeats_and_padding():
    x = I.truncate_q(I.custom(2, 3, 32, 300, seed=3), 20, 4)
    ids, vals = I.to_sparse_q(x["q"], pad=3, dup=2, shuffle_seed=1)
    assert ids.shape == vals.shape == (2, 3, 20 + 2 + 3)
    assert ids.dtype == np.int32 and vals.dtype == np.float32
    for b in range(2):
        for i in range(3):
            live = ids[b, i] >= 0
            assert np.count_nonzero(~live) == 3 and np.all(vals[b, i, ~live] == 0)
            dense = np.zeros(300, dtype=np.float32)
            np.maximum.at(dense, ids[b, i, live], vals[b, i, live])   # a repeated id keeps its larger value
            np.testing.assert_array_equal(dense, x["q"][b, i])
            assert np.unique(ids[b, i, live]).size == 20


def test_truncate_q_keeps_k_entries_and_draws_from_them():
    x = I.custom(3, 4, 32, 500, seed=5)
    y = I.truncate_q(x, 17, 6)
    assert np.all((y["q"] != 0).sum(-1) == 17)
    np.testing.assert_allclose(y["q"].sum(-1), 1.0, atol=1e-6)
    for b in range(3):
        for i in range(4):
            assert y["q"][b, i, y["draft"][b, i]] > 0
            top = np.argsort(-x["q"][b, i], kind="stable")[:17]
            assert set(np.flatnonzero(y["q"][b, i])) == set(top)


def test_clustered_head_inputs():
    x = I.clustered_head(5, 24, 1000, 30, 20, w_std=0.3, seed=2)
    m = x["members"]
    assert m.shape == (30, 20) and m.dtype == np.int32
    assert np.unique(m).size == m.size and m.min() >= 0 and m.max() < 1000
    cent = I.bf16_bits_to_f32(x["centroid_bits"])
    W = I.bf16_bits_to_f32(x["W_bits"])
    for c in (0, 17, 29):
        np.testing.assert_allclose(cent[c], W[m[c]].mean(axis=0), rtol=1e-2, atol=1e-3)
    y = I.drafter_chain(2, 3, 24, 1024, 32, 32, 4, seed=3)
    assert y["h_draft_bits"].shape == (6, 24) and y["hidden_bits"].shape == (2, 4, 24)
    for r in range(6):
        # drafts are members of some cluster
        assert np.isin(y["draft"][r // 3, r % 3], y["members"])


def test_tree_inputs_draw_every_node_from_its_parents_q():
    parent = [-1, -1, 0, 0, 2]
    x = I.tree_inputs(3, parent, 16, 60, seed=4)
    assert x["hidden_bits"].shape == (3, 6, 16) and x["tokens"].shape == (3, 5)
    assert list(I.tree_rows_with_children(parent)) == [0, 1, 3]
    assert x["q"].shape == (3, 3, 60) and x["uniforms"].shape == (3, 6)
    np.testing.assert_allclose(x["q"].sum(-1), 1.0, atol=1e-5)
    y = I.tree_repeated_trials(x, 2000, seed=5)
    assert y["tokens"].shape == (2000, 5)
    # node 4's parent is node 2 (row 3, q slot 2): its tokens follow that row
    freq = np.bincount(y["tokens"][:, 4], minlength=60) / 2000
    assert np.abs(freq - x["q"][0, 2]).max() < 0.05
    for k, v in I.tree_inputs(3, parent, 16, 60, seed=4).items():
        np.testing.assert_array_equal(v, x[k])
