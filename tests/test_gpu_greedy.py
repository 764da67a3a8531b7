"""Greedy (match) verification: HIP path vs the fp64 greedy oracle, through the
C ABI, on an MI355X.  Every case prints its name, seed and shape first."""

import sys

import numpy as np
import pytest

from oracle import greedy_ref as G
from oracle import verify_ref as R
from synth import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu

_W_CACHE = {}


def _dev():
    import torch
    assert torch.cuda.is_available(), "no ROCm device"
    import draft_token_verification_02_amd as sv
    sv.library()
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


def _case(x, seed, p_match=0.75, seqs=None, logits=None):
    """Oracle logits (only for ``seqs`` if given; ``logits``: all rows' oracle
    logits if already known), drafts, oracle result."""
    B, g1, d = x["hidden_bits"].shape
    rows = np.arange(B) if seqs is None else np.asarray(seqs)
    L = R.lmhead_logits(x["hidden_bits"][rows].reshape(-1, d), x["W_bits"]) if logits is None \
        else logits[(rows[:, None] * g1 + np.arange(g1)[None, :]).ravel()]
    tgt = np.full((B, g1), 0, dtype=np.int64)
    tgt[rows] = G.greedy_tokens(L).reshape(len(rows), g1)
    draft = parity.greedy_drafts(x, tgt, p_match, seed)
    ref = G.verify_greedy(x["hidden_bits"][rows], x["W_bits"], draft[rows], logits=L)
    return draft, ref


def _report(name, rep):
    _say(name, " ".join(f"{k}={v:.3g}" if isinstance(v, float) else f"{k}={v}" for k, v in rep.items()))


def test_greedy_tiny():
    dev = _dev()
    _say("greedy tiny V=32 d=16 gamma=4 B=1")
    x = I.generate(I.CONFIGS["tiny"])
    draft, ref = _case(x, 1)
    for split in (False, True):
        rep = parity.compare_greedy(x, draft, parity.run_gpu_greedy(x, draft, dev, split=split), ref)
    _report("tiny", rep)


SMALL = [(3, 4, 200, 1000, 1), (2, 3, 1536, 5000, 2), (5, 2, 72, 777, 3), (1, 1, 8, 1, 4),
         (14, 4, 64, 4099, 5), (4, 8, 136, 300, 6), (2, 32, 40, 513, 7), (40, 7, 24, 65, 8),
         (1, 4, 4096, 2048, 9), (300, 1, 16, 33, 10),
         (4, 4, 256, 5000, 16), (8, 4, 128, 3001, 17)]   # several hidden fragments


@pytest.mark.parametrize("B,gamma,d,V,seed", SMALL)
def test_greedy_small_shapes(B, gamma, d, V, seed):
    dev = _dev()
    _say(f"greedy small B={B} gamma={gamma} d={d} V={V} seed={seed}")
    x = I.custom(B, gamma, d, V, seed=seed, sigma=0.8)
    draft, ref = _case(x, seed)
    a = parity.run_gpu_greedy(x, draft, dev)
    b = parity.run_gpu_greedy(x, draft, dev, split=True)
    for k in ("out", "n", "target", "status"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
    rep = parity.compare_greedy(x, draft, b, ref)
    _report("small", rep)


SWEEP = [f"sweep_b{b}_s{s}" for b in (16, 64, 256) for s in (0.2, 0.5, 1.0)]
FULL = ["gemma_e2b", "llama8b_g2_b1", "llama8b_g4_b1", "llama8b_g8_b1", "llama8b_g2_b4",
        "llama8b_g4_b4", "llama8b_g8_b4", "sparse_q"] + SWEEP


@pytest.mark.parametrize("name", FULL)
def test_greedy_full_config(name):
    """Every sequence of every named workload (the batch sweep's nine runs too)."""
    dev = _dev()
    cfg = I.CONFIGS[name]
    _say(f"greedy full {name} B={cfg.B} gamma={cfg.gamma} d={cfg.d} V={cfg.V} seed={cfg.seed}")
    x = _gen(name)
    draft, ref = _case(x, 17, logits=parity.oracle_logits(cfg, x))
    gpu = parity.run_gpu_greedy(x, draft, dev)
    rep = parity.compare_greedy(x, draft, gpu, ref)
    _report(name, rep)
    assert rep["seqs"] == cfg.B


def test_greedy_all_drafts_match_gives_bonus():
    dev = _dev()
    _say("greedy all-match B=8 gamma=5 d=128 V=3000 seed=19")
    x = I.custom(8, 5, 128, 3000, seed=19)
    draft, ref = _case(x, 19, p_match=1.0)
    gpu = parity.run_gpu_greedy(x, draft, dev, split=True)
    parity.compare_greedy(x, draft, gpu, ref)
    ok = ~ref.flagged.any(axis=1)
    assert np.all(gpu["n"][ok] == 5)
    assert np.array_equal(gpu["out"][ok], ref.target[ok])


def test_greedy_exact_tie_lowest_id():
    """Duplicated W rows inside one 64-row group give bit-equal logits; the
    lower id must win, on the oracle and on the GPU's own logits."""
    dev = _dev()
    _say("greedy tie B=2 gamma=2 d=64 V=600 seed=20")
    x = I.custom(2, 2, 64, 600, seed=20)
    L = R.lmhead_logits(x["hidden_bits"].reshape(-1, 64), x["W_bits"])
    W = x["W_bits"].copy()
    for b in range(2):
        y = int(np.argmax(L[b * 3]))
        z = y + 1 if y % 64 != 63 else y - 1
        W[z] = W[y]
    x["W_bits"] = W
    draft, ref = _case(x, 20)
    gpu = parity.run_gpu_greedy(x, draft, dev, split=True)
    parity.compare_greedy(x, draft, gpu, ref)
    for b in range(2):
        r = b * 3
        row = gpu["logits"][r]
        top = np.flatnonzero(row == row.max())
        assert gpu["target"][b, 0] == top[0]


def test_greedy_bad_drafts_and_nan_rows():
    dev = _dev()
    _say("greedy bad drafts and NaN B=3 gamma=3 d=64 V=500 seed=21")
    x = I.custom(3, 3, 64, 500, seed=21)
    x["hidden_bits"] = x["hidden_bits"].copy()
    x["hidden_bits"][2, :, 3] = 0x7FC0               # every row of sequence 2 is NaN
    draft, ref = _case(x, 21, p_match=1.0)
    draft[0, 0] = 500
    draft[1, 1] = -3
    ref = G.verify_greedy(x["hidden_bits"], x["W_bits"], draft)
    gpu = parity.run_gpu_greedy(x, draft, dev)
    assert gpu["n"][0] == 0 and gpu["status"][0] & 1
    assert gpu["n"][1] <= 1 and gpu["status"][1] & 1
    assert gpu["n"][2] == 0 and gpu["status"][2] & 4
    assert gpu["out"][2, 0] == 0 and np.all(gpu["target"][2] == -1)
    assert ref.nonfinite[2] and np.all(ref.target[2] == -1)
    parity.compare_greedy(x, draft, gpu, ref, seqs=[0, 1])


def test_greedy_determinism_bitwise():
    dev = _dev()
    _say("greedy determinism gemma_e2b twice")
    x = _gen("gemma_e2b")
    draft = x["draft"]
    a = parity.run_gpu_greedy(x, draft, dev)
    b = parity.run_gpu_greedy(x, draft, dev)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)
