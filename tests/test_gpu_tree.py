"""Tree verification: HIP path vs the fp64 oracle, through the C ABI, on an
MI355X.  Every case prints its name, seed and shape before touching the GPU.
"""

import sys

import numpy as np
import pytest

from oracle import tree_ref as TR
from synth import inputs as I
from tests import parity

pytestmark = pytest.mark.gpu


def _dev():
    import torch
    assert torch.cuda.is_available(), "no ROCm device"
    import draft_token_verification_02_amd as sv
    sv.library()
    return torch.device("cuda:0")


def _say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def test_path_tree_is_the_chain_bitwise():
    dev = _dev()
    _say("path tree vs chain B=7 T=4 d=128 V=5000 seed=1")
    x = I.custom(7, 4, 128, 5000, seed=1, sigma=0.8)
    chain = parity.run_gpu(x, dev)
    tx = {"hidden_bits": x["hidden_bits"], "W_bits": x["W_bits"], "parent": np.arange(-1, 3),
          "tokens": x["draft"], "q": x["q"], "uniforms": x["uniforms"]}
    tree = parity.run_gpu_tree(tx, dev)
    for k in ("out", "n", "logits", "row_max", "row_sumexp", "status"):
        np.testing.assert_array_equal(tree[k], chain[k], err_msg=k)
    np.testing.assert_array_equal(tree["path"][np.arange(7)[:, None], np.arange(4)[None, :]] >= 0,
                                  np.arange(4)[None, :] < chain["n"][:, None])


SMALL = [  # (B, parent, d, V, sigma, seed)
    (5, [-1, -1], 64, 700, 0.8, 2),
    (9, [-1, -1, -1, 0, 0, 1, 3, 3, 6], 128, 3000, 1.0, 3),
    (3, I.EAGLE_LIKE_TREE, 200, 9000, 0.8, 4),
    (40, [-1, -1, 0, 1, 1], 32, 5000, 1.5, 5),      # many sequences
    (2, [-1] * 12, 48, 300, 2.0, 6),                # one wide fork
    (4, list(range(-1, 19)) + [0, 1], 64, 777, 0.5, 7),   # deep, two side branches
    (1, [-1, -1, 0, 0], 32, 280000, 1.0, 8),       # 69 chunks: split rounds, multi-window S
    # the largest tree: 64 nodes, a 32-wide fork at the root and a 32-deep
    # chain under its first child (one lane per node in the kernels' tables)
    (6, [-1] * 32 + [0] + list(range(32, 63)), 48, 600, 0.7, 9),
]


@pytest.mark.parametrize("B,parent,d,V,sigma,seed", SMALL)
def test_tree_small_parity(B, parent, d, V, sigma, seed):
    dev = _dev()
    _say(f"tree small B={B} T={len(parent)} d={d} V={V} sigma={sigma} seed={seed}")
    x = I.tree_inputs(B, parent, d, V, sigma=sigma, seed=seed)
    rep = parity.compare_tree(x, parity.run_gpu_tree(x, dev))
    _say("tree small", rep)


def test_tree_bad_tokens_are_rejected_and_flagged():
    dev = _dev()
    _say("tree bad tokens B=3 T=3 d=32 V=400 seed=8")
    x = I.tree_inputs(3, [-1, -1, 0], 32, 400, sigma=0.3, seed=8)
    x["tokens"][1, 0] = 400
    x["tokens"][2, 0] = -5
    x["tokens"][2, 1] = 10 ** 6
    gpu = parity.run_gpu_tree(x, dev)
    parity.compare_tree(x, gpu)
    assert gpu["status"][1] & 1 and gpu["status"][2] & 1


@pytest.mark.parametrize("B,d,V,seed", [(1, 1536, 262144, 0), (4, 4096, 128256, 1),
                                        (16, 4096, 128256, 2)])   # R = 104 and 416: tiled GEMM
def test_tree_full_shape_parity(B, d, V, seed):
    dev = _dev()
    _say(f"tree full B={B} T={len(I.EAGLE_LIKE_TREE)} d={d} V={V} seed={seed}")
    x = I.tree_inputs(B, I.EAGLE_LIKE_TREE, d, V, w_std=0.02, sigma=0.5, seed=seed)
    rep = parity.compare_tree(x, parity.run_gpu_tree(x, dev))
    _say("tree full", rep)


def _chi2_pvalue(counts, probs):
    from scipy.stats import chi2
    n = counts.sum()
    exp = probs * n
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    stat = ((c - e) ** 2 / e).sum()
    return chi2.sf(stat, len(e) - 1)


def test_tree_first_token_is_distributed_as_p_on_the_gpu():
    dev = _dev()
    parent = [-1, -1, -1, 0, 0, 1]
    _say("tree distribution B=100000 T=6 d=16 V=24 seed=9")
    base = I.tree_inputs(1, parent, 16, 24, w_std=0.6, sigma=1.5, seed=9)
    x = I.tree_repeated_trials(base, 100000, seed=10)
    gpu = parity.run_gpu_tree(x, dev)
    ref = TR.verify_tree(base["hidden_bits"], base["W_bits"], parent, base["tokens"], base["q"],
                         base["uniforms"])
    p0 = ref.p[0]
    counts = np.bincount(gpu["out"][:, 0], minlength=24).astype(float)
    pv = _chi2_pvalue(counts, p0)
    _say("first token chi-square p-value", pv)
    assert pv > 1e-3
    # after a kept node 0, the next token follows p of node 0's row
    sel = gpu["path"][:, 0] == 0
    counts = np.bincount(gpu["out"][sel, 1], minlength=24).astype(float)
    pv = _chi2_pvalue(counts, ref.p[1])
    _say("after node 0: chi-square p-value", pv, "trials", int(sel.sum()))
    assert pv > 1e-3
