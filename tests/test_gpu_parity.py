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
    (14, 4, 64, 4099, 5),      # R = 70: the tiled GEMM's 128-row blocks, three-stage ring
    (4, 8, 136, 300, 6),
    (2, 32, 40, 513, 7),       # gamma at its maximum
    (40, 7, 24, 65, 8),        # R = 320
    (1, 4, 4096, 2048, 9),
    (300, 1, 16, 33, 10),
    (20, 4, 1024, 1000, 11),   # R = 100, ragged V (a partial last vocab block)
    (30, 4, 512, 2050, 12),    # R = 150: one 192-row block, four-stage ring, V % 4 != 0
    (1, 3, 16, 262143, 13),    # 64 chunks (one window of chunk totals), ragged last chunk
    (1, 4, 32, 300000, 14),    # 74 chunks: the split draw and the pick's multi-window search
    (2, 2, 24, 270001, 15),
    # several hidden fragments at small d
    (4, 4, 256, 5000, 16),     # R = 20, two fragments, a partial last vocab group
    (8, 4, 128, 3001, 17),     # R = 40, V % 4 != 0: per-element logit stores
    (12, 4, 512, 2048, 18),    # R = 60, four fragments
    (3, 7, 1536, 4096, 19),    # R = 24 at the Gemma-shaped d
    (16, 5, 512, 3000, 20),    # R = 96
    (49, 1, 512, 2003, 21),    # R = 98, V % 4 != 0
    (13, 4, 200, 3000, 22),    # R = 65, d % 32 != 0: the ragged last k step
    (25, 4, 1544, 1031, 23),   # R = 125 at d = 1544 (ragged k), V % 4 != 0
    (43, 2, 200, 3000, 24),    # R = 129: 192-row blocks
    (172, 4, 64, 700, 25),     # R = 860: 128-row blocks with the four-stage ring
    (200, 4, 40, 900, 26),     # R = 1000: 256-row blocks, ragged k
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


@pytest.mark.parametrize("B,gamma,d,V,seed", [(6, 4, 256, 3000, 11), (40, 7, 64, 5000, 12)])
def test_lmhead_ex_split_matches_whole_calls(B, gamma, d, V, seed):
    """sv_lmhead_ex with the logits only, then stage 2, is spec_verify bit for
    bit; with the argmax partials only, then the greedy stage, it is
    spec_verify_greedy (R = 30 and R = 320: both LM-head paths)."""
    import torch
    import draft_token_verification_02_amd as sv
    dev = _dev()
    _say(f"sv_lmhead_ex split B={B} gamma={gamma} d={d} V={V} seed={seed}")
    x = I.custom(B, gamma, d, V, seed=seed, w_std=parity.small_w_std(d))
    whole = parity.run_gpu(x, dev)
    t = parity.to_device(x, dev)
    dims = sv.dims_of(t["hidden_bits"], t["W_bits"])
    ws = sv.new_workspace(dims, dev)
    out = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    n = torch.empty((B,), dtype=torch.int32, device=dev)
    sv.lmhead(t["hidden_bits"], t["W_bits"], ws, argmax=False)
    sv.accept_and_draw(dims, t["draft"], t["q"], t["uniforms"], out, n, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), whole["out"])
    np.testing.assert_array_equal(n.cpu().numpy(), whole["n"])
    np.testing.assert_array_equal(sv.debug_views(ws, dims)["logits"].cpu().numpy(), whole["logits"])
    g_out, g_n, g_t = sv.verify_greedy(t["hidden_bits"], t["W_bits"], t["draft"])
    tgt = torch.empty((B, gamma + 1), dtype=torch.int32, device=dev)
    sv.lmhead(t["hidden_bits"], t["W_bits"], ws, logits=False)
    sv.accept_greedy(dims, t["draft"], out, n, ws, target_tokens=tgt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), g_out.cpu().numpy())
    np.testing.assert_array_equal(tgt.cpu().numpy(), g_t.cpu().numpy())


SWEEP = [f"sweep_b{b}_s{s}" for b in (16, 64, 256) for s in (0.2, 0.5, 1.0)]
FULL = ["gemma_e2b", "llama8b_g2_b1", "llama8b_g4_b1", "llama8b_g8_b1", "llama8b_g2_b4",
        "llama8b_g4_b4", "llama8b_g8_b4", "sparse_q"] + SWEEP


@pytest.mark.parametrize("name", FULL)
def test_full_config_parity(name):
    """Every sequence of every named workload, element by element (the batch
    sweep's nine B x sigma runs included: up to 1280 rows x 128256 logits)."""
    dev = _dev()
    cfg = I.CONFIGS[name]
    _say(f"full {name} B={cfg.B} gamma={cfg.gamma} d={cfg.d} V={cfg.V} seed={cfg.seed}")
    x = _gen(name)
    gpu = parity.run_gpu(x, dev)
    rep = parity.compare(x, gpu, logits=parity.oracle_logits(cfg, x))
    _report(name, rep)
    assert rep["seqs"] == cfg.B


@pytest.mark.parametrize("d", [8200, 8192])
def test_lmhead_w_near_4gib(d):
    """The many-row GEMM's copies are buffer loads with 32-bit byte offsets
    while W is under 4 GiB, 64-bit pointer loads from 4 GiB on.  At
    262000 x 8192 bf16 (4.29 GB) the buffer offsets reach within 3 MB of
    2^32; at 262000 x 8200 (4.30 GB) the pointer form runs, with a ragged
    last k step (8200 = 256 * 32 + 8).  Sampled logits against the oracle's
    exact dot products -- the first and last rows of W and the partial last
    vocab block (262000 = 1023 * 256 + 112) included -- to the stated fp32
    summation bound, and each sampled row's normaliser against the GPU's own
    logits."""
    import torch
    import draft_token_verification_02_amd as sv
    dev = _dev()
    B, gamma, V, seed = 16, 4, 262000, 91
    assert (V * d * 2 >= 1 << 32) == (d == 8200)
    _say(f"W near 4 GiB B={B} gamma={gamma} d={d} V={V} seed={seed}")
    g = torch.Generator(device=dev).manual_seed(seed)
    W = torch.randn((V, d), generator=g, device=dev, dtype=torch.bfloat16).mul_(0.02)
    hidden = torch.randn((B, gamma + 1, d), generator=g, device=dev, dtype=torch.bfloat16)
    draft = torch.randint(0, V, (B, gamma), generator=g, device=dev, dtype=torch.int32)
    q = torch.rand((B, gamma, V), generator=g, device=dev) + 0.5
    q /= q.sum(dim=-1, keepdim=True)
    u = torch.rand((B, gamma + 1), generator=g, device=dev).clamp_(min=1e-6)
    dims = sv.dims_of(hidden, W)
    ws = sv.new_workspace(dims, dev)
    out, n = sv.verify(hidden, W, draft, q, u, workspace=ws)
    torch.cuda.synchronize()
    views = sv.debug_views(ws, dims)
    R_ = B * (gamma + 1)
    rows = [0, 1, 40, R_ - 1]
    rng = np.random.default_rng(seed)
    cols = sorted({0, 1, 255, 256, 131071, 200000, V - 112, V - 2, V - 1,
                   *rng.integers(0, V, 8).tolist()})
    h_bits = hidden.reshape(R_, d)[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    w_bits = W[cols].view(torch.int16).cpu().numpy().view(np.uint16)
    exact = R.lmhead_logits(h_bits, w_bits)
    absdot = R.bf16_to_f64(h_bits).__abs__() @ R.bf16_to_f64(w_bits).__abs__().T
    L = views["logits"][rows].double().cpu().numpy()
    got = L[:, cols]
    # the library's stated bound on a logit: an fp32 sum of exact bf16
    # products in any order, gamma_{d-1} sum_k |h_k W_jk|
    nu = (d - 1) * 2.0 ** -24
    bound = nu / (1 - nu) * absdot
    err = np.abs(got - exact)
    _say(f"max |dlogit| {err.max():.3e}, largest allowed {bound.max():.3e}")
    assert np.all(err <= bound), f"logit error {err.max()} beyond its bound"
    for i, r in enumerate(rows):
        m = L[i].max()
        assert float(views["row_max"][r]) == m
        s_ref = np.exp(L[i] - m).sum()
        assert abs(float(views["row_sumexp"][r]) - s_ref) <= 2e-5 * s_ref
    n_h = n.cpu().numpy()
    o_h = out.cpu().numpy()
    assert np.all((n_h >= 0) & (n_h <= gamma))
    for b in range(B):
        assert 0 <= o_h[b, n_h[b]] < V and np.all(o_h[b, n_h[b] + 1:] == -1)
    assert np.all(views["status"].cpu().numpy() == 0)
    del W, q, ws


def test_lmhead_hidden_rows_past_4gib():
    """Many rows at the largest hidden size: 32770 rows x 65536 bf16 (4.29 GB),
    whose tiled copy in the workspace (2049 x 2048 tiles, 4.297 GB) is past
    2^32 bytes, so the many-row GEMM copies the hidden rows through 64-bit
    pointers (192-row blocks; a ragged last row tile).  Sampled logits --
    first, last and ragged-tile rows -- against the oracle's exact dot
    products to the stated fp32 summation bound, each sampled row's
    normaliser against the GPU's own logits, and the outputs valid."""
    import torch
    import draft_token_verification_02_amd as sv
    from draft_token_verification_02_amd import _lib
    dev = _dev()
    B, gamma, d, V, seed = 6554, 4, 65536, 256, 92
    R_ = B * (gamma + 1)
    assert R_ * d * 2 >= 1 << 32 and -(-R_ // 16) * d * 2 * 16 >= 1 << 32
    _say(f"hidden rows past 4 GiB B={B} gamma={gamma} d={d} V={V} seed={seed}")
    g = torch.Generator(device=dev).manual_seed(seed)
    W = torch.randn((V, d), generator=g, device=dev, dtype=torch.bfloat16).mul_(0.004)
    hidden = torch.randn((B, gamma + 1, d), generator=g, device=dev, dtype=torch.bfloat16)
    draft = torch.randint(0, V, (B, gamma), generator=g, device=dev, dtype=torch.int32)
    q = torch.rand((B, gamma, V), generator=g, device=dev) + 0.5
    q /= q.sum(dim=-1, keepdim=True)
    u = torch.rand((B, gamma + 1), generator=g, device=dev).clamp_(min=1e-6)
    dims = sv.dims_of(hidden, W)
    ws = sv.new_workspace(dims, dev)
    out, n = sv.verify(hidden, W, draft, q, u, workspace=ws)
    torch.cuda.synchronize()
    views = sv.debug_views(ws, dims)
    rows = [0, 1, 17, 16383, 32767, 32768, R_ - 1]
    h_bits = hidden.reshape(R_, d)[rows].view(torch.int16).cpu().numpy().view(np.uint16)
    w_bits = W.view(torch.int16).cpu().numpy().view(np.uint16)
    exact = R.lmhead_logits(h_bits, w_bits)
    absdot = R.bf16_to_f64(h_bits).__abs__() @ R.bf16_to_f64(w_bits).__abs__().T
    L = views["logits"][rows].double().cpu().numpy()
    nu = (d - 1) * 2.0 ** -24
    bound = nu / (1 - nu) * absdot
    err = np.abs(L - exact)
    _say(f"max |dlogit| {err.max():.3e}, largest allowed {bound.max():.3e}")
    assert np.all(err <= bound), f"logit error {err.max()} beyond its bound"
    for i, r in enumerate(rows):
        m = L[i].max()
        assert float(views["row_max"][r]) == m
        s_ref = np.exp(L[i] - m).sum()
        assert abs(float(views["row_sumexp"][r]) - s_ref) <= 2e-5 * s_ref
    n_h = n.cpu().numpy()
    o_h = out.cpu().numpy()
    assert np.all((n_h >= 0) & (n_h <= gamma))
    ok = np.take_along_axis(o_h, n_h[:, None].astype(np.int64), axis=1)[:, 0]
    assert np.all((ok >= 0) & (ok < V))
    assert np.all(views["status"].cpu().numpy() == 0)
    del hidden, q, ws


def test_large_logits_stated_bound():
    """Logits near 90 (W std 0.5, d = 1536), where fp32 accumulation alone moves
    p by more than 1e-5: the error chain the library documents, checked link by
    link.  (1) Every logit is within the fp32 summation bound of its exact
    value: |dl| <= gamma_{d-1} * sum_k |h_k W_jk| (products of bf16 values are
    exact in fp32; any summation order).  (2) p follows from the GPU's own
    logit error: |dp_j| <= p_j * (2 eps + 4e-6) + 1e-12, eps the row's largest
    |dl| (the normaliser moves every p_j by the p-weighted mean of the dl, and
    the hardware exp2 and reciprocal add < 2e-6 each).  (3) Decisions: equal
    to the oracle's unless they lie inside the band that error implies
    (accept tests: |r - p/q| < (2 eps + 4e-6) p/q; draws: within 2 (2 eps +
    4e-6) / S of an edge of the normalised CDF, S the drawn weights' sum),
    and valid there."""
    dev = _dev()
    B, gamma, d, V = 6, 4, 1536, 6000
    _say(f"large logits B={B} gamma={gamma} d={d} V={V} w_std=0.5 seed=31")
    x = I.custom(B, gamma, d, V, seed=31, sigma=0.8, w_std=0.5)
    gpu = parity.run_gpu(x, dev)
    ref = R.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
    H = R.bf16_to_f64(x["hidden_bits"].reshape(-1, d))
    Wf = R.bf16_to_f64(x["W_bits"])
    absdot = np.abs(H) @ np.abs(Wf).T                          # sum_k |h_k W_jk|
    u = 2.0 ** -24
    gam = (d - 1) * u / (1 - (d - 1) * u)
    dl = np.abs(gpu["logits"].astype(np.float64) - ref.logits)
    assert np.all(dl <= gam * absdot), "a logit outside the fp32 summation bound"
    eps = dl.max(axis=1)                                       # per row
    gp = np.exp(gpu["logits"].astype(np.float64) - gpu["row_max"].astype(np.float64)[:, None]) / \
        gpu["row_sumexp"].astype(np.float64)[:, None]
    delta = 2 * eps + 4e-6                                     # relative error bound on p, per row
    dp = np.abs(gp - ref.p)
    assert np.all(dp <= ref.p * delta[:, None] + 1e-12), "p outside the bound its logits imply"
    g1 = gamma + 1
    dmax = float(delta.max())
    rows = np.arange(B)[:, None] * g1 + np.arange(gamma)[None, :]
    with np.errstate(divide="ignore"):
        ratio = np.where(ref.q_draft > 0, ref.p_draft / ref.q_draft, np.inf)
    acc_band = np.maximum(R.ACCEPT_BAND, delta[rows] * np.minimum(ratio, 1e30))
    rep = parity.compare(x, gpu, ref=ref, accept_band=acc_band,
                         sample_band=lambda res: np.maximum(R.SAMPLE_BAND, 2 * dmax / res.draw_S),
                         p_atol=float(dp.max()) + 1e-15)
    _say(f"large logits: max|l|={np.abs(ref.logits).max():.1f} max eps={eps.max():.3g} "
         f"(eps / (2^-24 sqrt(d) max|l|) = "
         f"{(eps / (u * np.sqrt(d) * np.abs(ref.logits).max(axis=1))).max():.3g}) "
         f"max|dp|={dp.max():.3g} accept_flagged={rep['accept_flagged']} "
         f"draw_flagged={rep['draw_flagged']}")
    assert dp.max() > 1e-6                    # the regime really is the large-logit one


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
