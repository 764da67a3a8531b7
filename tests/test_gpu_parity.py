"""HIP path vs the fp64 oracle, through the C ABI, on an MI355X.

Every case prints its name, seed and shape before touching the GPU.
"""

import math
import sys

import numpy as np
import pytest

from oracle import verify_ref as R
from synth import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu

_W_CACHE = {}


def _dev():
    import torch
    assert torch.cuda.is_available(), "no ROCm device"
    import draft_token_verification_02_amd as sv
    sv.library()                      # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def _gen(name):
    cfg = I.CONFIGS[name]
    key = (cfg.V, cfg.d, cfg.w_std, cfg.seed)
    x = I.generate(cfg, W_bits=_W_CACHE.get(key))
    _W_CACHE.clear()
    _W_CACHE[key] = x["W_bits"]
    return x


def _report(name, rep):
    _say(name, " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in rep.items()))


# ---------------------------------------------------------------------------
def test_tiny_config_full_parity():
    dev = _dev()
    _say("tiny config V=32 d=16 gamma=4 B=1 seed=0")
    x = I.generate(I.CONFIGS["tiny"])
    rep = parity.compare(x, parity.run_gpu(x, dev))
    _report("tiny", rep)
    assert rep["max_abs_dlogit"] < 1e-4


SMALL = [  # (B, gamma, d, V, seed): tiles, ragged tails, V % 4 != 0, R > 64, short d
    (3, 4, 200, 1000, 1),
    (2, 3, 1536, 5000, 2),
    (5, 2, 72, 777, 3),
    (1, 1, 8, 1, 4),
    (14, 4, 64, 4099, 5),      # R = 70: two row passes
    (4, 8, 136, 300, 6),
    (2, 32, 40, 513, 7),       # gamma at its maximum
    (40, 7, 24, 65, 8),        # R = 320
    (1, 4, 4096, 2048, 9),
    (300, 1, 16, 33, 10),
    (20, 4, 1024, 1000, 11),   # R = 100, the many-row GEMM's pipelined path, ragged V
    (30, 4, 512, 2050, 12),    # R = 150: two row tiles, shortest pipelined d, V % 4 != 0
    (1, 3, 16, 262143, 13),    # 64 chunks (one window of chunk totals), ragged last chunk
    (1, 4, 32, 300000, 14),    # 74 chunks: the split draw and the pick's multi-window search
    (2, 2, 24, 270001, 15),
    # several hidden fragments at small d
    (4, 4, 256, 5000, 16),     # R = 20, two fragments, a partial last vocab group
    (8, 4, 128, 3001, 17),     # R = 40, V % 4 != 0: per-element logit stores
    (12, 4, 512, 2048, 18),    # R = 60, four fragments
    (3, 7, 1536, 4096, 19),    # R = 24 at the Gemma-shaped d
    (16, 5, 512, 3000, 20),    # R = 96: the 128-row GEMM's 96-row blocks, pipelined path
    (49, 1, 512, 2003, 21),    # R = 98: its 128-row blocks, V % 4 != 0
]


@pytest.mark.parametrize("B,gamma,d,V,seed", SMALL)
def test_small_shapes_parity(B, gamma, d, V, seed):
    dev = _dev()
    _say(f"small B={B} gamma={gamma} d={d} V={V} seed={seed}")
    x = I.custom(B, gamma, d, V, seed=seed, sigma=0.8, w_std=parity.small_w_std(d))
    rep = parity.compare(x, parity.run_gpu(x, dev))
    _report("small", rep)


def test_stage_split_matches_whole_call():
    dev = _dev()
    _say("stage split B=6 gamma=4 d=256 V=3000 seed=11")
    x = I.custom(6, 4, 256, 3000, seed=11)
    a = parity.run_gpu(x, dev)
    b = parity.run_gpu(x, dev, split=True)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


FULL = ["gemma_e2b", "llama8b_g2_b1", "llama8b_g4_b1", "llama8b_g8_b1", "llama8b_g2_b4",
        "llama8b_g4_b4", "llama8b_g8_b4", "sweep_b16_s0.5", "sparse_q"]


@pytest.mark.parametrize("name", FULL)
def test_full_config_parity(name):
    dev = _dev()
    cfg = I.CONFIGS[name]
    _say(f"full {name} B={cfg.B} gamma={cfg.gamma} d={cfg.d} V={cfg.V} seed={cfg.seed}")
    x = _gen(name)
    rep = parity.compare(x, parity.run_gpu(x, dev))
    _report(name, rep)


@pytest.mark.parametrize("name", ["sweep_b64_s0.2", "sweep_b256_s1.0"])
def test_large_batch_sampled_parity(name):
    dev = _dev()
    cfg = I.CONFIGS[name]
    _say(f"large {name} B={cfg.B} gamma={cfg.gamma} d={cfg.d} V={cfg.V} seed={cfg.seed}")
    x = _gen(name)
    gpu = parity.run_gpu(x, dev)
    seqs = np.unique(np.concatenate([[0, cfg.B - 1], np.random.default_rng(1).choice(cfg.B, 10)]))
    rep = parity.compare(x, gpu, seqs=seqs)
    _report(name, rep)
    # every sequence: shape invariants
    n = gpu["n"]
    assert np.all((n >= 0) & (n <= cfg.gamma))
    for b in range(cfg.B):
        assert list(gpu["out"][b, :n[b]]) == list(x["draft"][b, :n[b]])
        assert 0 <= gpu["out"][b, n[b]] < cfg.V


def test_determinism_bitwise():
    dev = _dev()
    _say("determinism gemma_e2b twice")
    x = _gen("gemma_e2b")
    a = parity.run_gpu(x, dev)
    b = parity.run_gpu(x, dev)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_bad_draft_ids_are_rejected_and_flagged():
    dev = _dev()
    _say("bad draft ids B=4 gamma=3 d=64 V=500")
    x = I.custom(4, 3, 64, 500, seed=12)
    x["draft"] = x["draft"].copy()
    x["draft"][0, 0] = 500
    x["draft"][1, 1] = -7
    x["uniforms"] = x["uniforms"].copy()
    x["uniforms"][1, 0] = np.float32(1e-6)      # draft 0 of seq 1 is kept
    gpu = parity.run_gpu(x, dev)
    assert gpu["n"][0] == 0 and gpu["status"][0] & 1
    assert gpu["n"][1] <= 1 and gpu["status"][1] & 1
    parity.compare(x, gpu)


def test_residual_fallback_flagged():
    dev = _dev()
    _say("fallback q = 2p B=3 gamma=2 d=64 V=400")
    x = I.custom(3, 2, 64, 400, seed=13)
    ref = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    q = np.stack([2.0 * ref.p[b * 3:b * 3 + 2] for b in range(3)]).astype(np.float32)
    x["q"] = q
    x["uniforms"] = x["uniforms"].copy()
    x["uniforms"][:, 0] = np.float32(0.9)       # 0.9 * 2p > p: draft 0 rejected
    gpu = parity.run_gpu(x, dev)
    ref2 = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    assert ref2.draw_fallback.all()
    assert np.all(gpu["n"] == 0) and np.all(gpu["status"] & 2)
    parity.compare(x, gpu, ref=ref2)


def test_nan_hidden_completes_with_defined_output():
    dev = _dev()
    _say("NaN hidden B=2 gamma=2 d=64 V=300")
    x = I.custom(2, 2, 64, 300, seed=14)
    x["hidden_bits"] = x["hidden_bits"].copy()
    x["hidden_bits"][0, :, 5] = 0x7FC0              # NaN in every row of sequence 0
    gpu = parity.run_gpu(x, dev)
    n = gpu["n"]
    assert 0 <= n[0] <= 2 and 0 <= gpu["out"][0, n[0]] < 300
    assert gpu["status"][0] & 4                     # no finite weights
    parity.compare(parity.subset(x, [1]), {k: (v[1:] if k in ("out", "n", "status") else v[3:])
                                           for k, v in gpu.items()})


def test_tiny_distribution_on_gpu():
    """1e5 trials of the tiny config in one call: each position's law is p."""
    from tests.test_oracle_pins import _chi2_pvalue
    dev = _dev()
    _say("distribution tiny B=100000")
    base = I.generate(I.CONFIGS["tiny"])
    t = I.repeated_trials(base, 100_000, seed=404)
    gpu = parity.run_gpu(t, dev)
    ref = R.verify(t["hidden_bits"], t["W_bits"], t["draft"], t["q"], t["uniforms"])
    g = t["draft"].shape[1]
    for i in range(g + 1):
        reached = gpu["n"] >= i
        if reached.sum() < 2000:
            continue
        counts = np.bincount(gpu["out"][reached, i], minlength=32)
        assert _chi2_pvalue(counts, ref.p[i]) >= 1e-3, i
    rep = parity.compare(t, gpu, ref=ref)
    _report("distribution", rep)


def test_alpha_formula_on_gpu():
    dev = _dev()
    _say("alpha formula iid B=100000")
    n = 100_000
    x = I.iid_positions(32, 16, 4, n, seed=7)
    gpu = parity.run_gpu(x, dev)
    ref = R.verify(x["hidden_bits"][:1], x["W_bits"], x["draft"][:1], x["q"][:1], x["uniforms"][:1])
    alpha = ref.alpha[0, 0]
    tokens = gpu["n"] + 1
    se = tokens.std(ddof=1) / math.sqrt(n)
    want = R.expected_tokens_per_step(alpha, 4)
    _say(f"alpha={alpha:.4f} mean_tokens={tokens.mean():.4f} formula={want:.4f} se={se:.4f}")
    assert abs(tokens.mean() - want) < 4 * se
