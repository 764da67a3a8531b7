"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--mode MODE]

One step is the whole path on one batch of resident synthetic inputs: the
LM-head GEMM over all B*(gamma+1) rows (one pass over W), the softmax
normalisers, the accept tests, the first rejection and the replacement/bonus
draw.  The timed loops call the library's two stage entry points back to back
(exactly the launches spec_verify makes).  The first loop gives the
throughput; a second loop with HIP events around each LM-head launch gives
that kernel's average duration for the roofline.  (Stage 1 is launched as
spec_verify launches it: sv_lmhead_ex keeping the logits, without the argmax
partials only greedy verification reads.)  Prints one JSON line.

Default workload: the batch sweep's largest single-GPU case, sweep_b256_s0.5
(d=4096, V=128256, gamma=4, B=256: 1280 rows, MFMA-bound), with the
Gemma-4-E2B-shaped head at B=1 (d=1536, V=262144: HBM-bound) measured the
same way as an extra entry.  Other named workloads are in
synth.inputs.CONFIGS.

Other modes (same JSON line):
  --mode greedy  greedy (match) verification: spec_verify_greedy, whose LM-head
                 launch keeps only argmax/softmax partials (no logits in HBM),
                 then the per-sequence greedy kernel; events bracket the call.
  --mode sparse  verification with q given as (id, value) entries of its
                 nonzeros (spec_verify_sparse_q); meant for --config sparse_q.
  --mode tree    tree verification of a 25-node draft tree at the config's
                 head shape and B (spec_verify_tree); events time the LM head.
  --mode head    the drafter's clustered sparse head at the config's shape
                 (sparse_q: B*gamma = 32 rows); value is rows/s.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import perfmodel  # noqa: E402

PROFILES = os.path.join(ROOT, "profiles")


def code_text(src: str) -> str:
    """C/C++/HIP source with its comments removed and whitespace runs folded
    to one space (string and character literals kept as written), so that a
    comment edit does not count as a change of the kernel."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(files) -> str:
    """Hash of the code (comments and layout aside) of the given sources."""
    h = hashlib.sha256()
    for p in files:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def traffic_from_counters(cfg_name: str):
    """HBM bytes per LM-head launch from committed rocprofv3 counter runs.

    The summaries (profiles/*_counters.json) were taken with the default mode
    (dense q) of one workload each; each records a hash of its kernel's
    sources.  None when there is no summary for this workload or the kernel
    source has changed since the counters were taken.
    """
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_counters.json"))):
        with open(path) as f:
            c = json.load(f)
        if c.get("workload") != cfg_name:
            continue
        if c.get("kernel_hash") != source_hash(c.get("kernel_sources", [])):
            return None
        return c.get("hbm_bytes_per_launch")
    return None


def counter_calibration(cfg_name: str):
    """How the committed counter summary of a workload turns counts into
    bytes: the scales that make FETCH_SIZE and WRITE_SIZE read 1 GiB for a
    1 GiB device copy, and the file they come from."""
    import glob
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_counters.json"))):
        with open(path) as f:
            c = json.load(f)
        if c.get("workload") == cfg_name:
            return (f"FETCH_SIZE x {c['fetch_scale']:.3f} + WRITE_SIZE x {c['write_scale']:.3f} "
                    f"(KiB per dispatch; scales from a {c['copy_probe_bytes'] >> 20} MiB device "
                    f"copy), profiles/{os.path.basename(path)}")
    return None


def mfma_counters(cfg_name: str) -> dict:
    """Counter-based MFMA busy fraction of the tiled LM-head GEMM, and the
    shader clock it ran at.

    From committed rocprofv3 runs (profiles/*_mfma_util.json: the
    derived MfmaUtil counter, MFMA busy cycles over active cycles of every
    SIMD, and GRBM_GUI_ACTIVE per XCD over each dispatch's duration) of the
    default mode of one workload each; None for both when there is no
    summary for this workload or the kernel's sources have changed since.
    """
    import glob
    none = {"busy": None, "clock_ghz": None}
    for path in sorted(glob.glob(os.path.join(PROFILES, "*_mfma_util.json"))):
        with open(path) as f:
            c = json.load(f)
        if c.get("workload") != cfg_name:
            continue
        if c.get("kernel_hash") != source_hash(c.get("kernel_sources", [])):
            return none
        return {"busy": c.get("mfma_util_pct") / 100.0, "clock_ghz": c.get("shader_clock_ghz_median")}
    return none


def mfma_busy_from_counters(cfg_name: str):
    """The counter-based MFMA busy fraction alone (see mfma_counters)."""
    return mfma_counters(cfg_name)["busy"]


def copy_bandwidth(dev, mib: int = 1024, reps: int = 5) -> float:
    """Achievable HBM rate of a plain device copy: (read + write bytes) / time.

    Context for the roofline: the fraction of 8 TB/s that a trivial streaming
    kernel (torch's copy) reaches on this GPU, best of ``reps`` HIP-event-timed
    copies of ``mib`` MiB, measured after the timed regions.
    """
    import torch
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del a, b
    return 2 * n / best / 1e9


def _oracle_rate(x: dict, seqs: int, greedy: bool, budget_s: float, threads):
    """Rows per second of the fp64 oracle (as it stands) on the first ``seqs``
    sequences of the workload, with BLAS limited to ``threads`` (None: all);
    median of up to three runs within ``budget_s``."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import greedy_ref, verify_ref
    sub = {k: (v if k == "W_bits" else v[:seqs]) for k, v in x.items()}
    times = []
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        t_end = time.perf_counter() + budget_s
        while True:
            t0 = time.perf_counter()
            if greedy:
                greedy_ref.verify_greedy(sub["hidden_bits"], sub["W_bits"], sub["draft"])
            else:
                verify_ref.verify(sub["hidden_bits"], sub["W_bits"], sub["draft"], sub["q"],
                                  sub["uniforms"])
            times.append(time.perf_counter() - t0)
            if len(times) >= 3 or time.perf_counter() + times[-1] > t_end:
                break
    rows = seqs * x["hidden_bits"].shape[1]
    t = statistics.median(times)
    return rows / t, used, len(times), t


def cpu_baseline(x: dict, greedy: bool = False, gpu_value: float = None) -> dict:
    """The fp64 oracle (as it stands) timed on the host, on bounded samples of
    the same workload: the first sequences of the batch, all host cores
    (BLAS threads as the environment sets them), then one core.  The oracle
    works sequence by sequence over full rows, so rows per second is its
    positions/s on the whole batch."""
    B, g1, d = x["hidden_bits"].shape
    V = x["W_bits"].shape[0]
    # samples sized for ~3 s per run of fp64 GEMM on a 16-core host, ~2 s on
    # one core (three runs each: ~15 s of host work in all)
    per_seq = 2.0 * g1 * d * V
    s_all = max(1, min(B, int(1.0e12 / per_seq)))
    s_one = max(1, min(B, int(4.0e10 / per_seq)))
    v_all, c_all, n_all, t_all = _oracle_rate(x, s_all, greedy, 30.0, None)
    v_one, c_one, n_one, t_one = _oracle_rate(x, s_one, greedy, 30.0, 1)
    res = {"value": v_all, "unit": "positions/s", "cores": c_all, "kind": "oracle",
           "sample": f"first {s_all} of {B} sequences ({s_all * g1} rows x V={V}, d={d}), "
                     f"median of {n_all} runs, {t_all:.2f} s each; fp64 numpy, "
                     f"BLAS threads={c_all}, host cpus={os.cpu_count()}",
           "single_core": {"value": v_one, "unit": "positions/s", "cores": c_one,
                           "sample": f"first {s_one} sequences ({s_one * g1} rows), median of "
                                     f"{n_one} runs, {t_one:.2f} s each"}}
    if gpu_value:
        res["gpu_over_oracle"] = gpu_value / v_all
        res["gpu_over_oracle_single_core"] = gpu_value / v_one
    return res


def measure(cfg, mode: str, steps: int, warmup: int, dev, w_layout: str = "rows",
            x=None) -> tuple:
    """Time ``steps`` whole steps of workload ``cfg`` in ``mode`` after
    ``warmup`` untimed ones; returns (result dict, the host inputs).
    w_layout "tiled": the steps take W's SV_W_TILED copy, made once before
    the timed regions (its time is reported, not counted in the steps).
    x: the host inputs of an earlier call on the same workload (sample,
    greedy and sparse modes), instead of generating them again."""
    import numpy as np
    import torch

    import draft_token_verification_02_amd as sv
    from synth import inputs

    def upload(x):
        # Through pinned host copies.  (Where a large tensor lands in HBM can
        # move the LM-head time by ~10% at d = 4096; uploads from pageable
        # host memory landed on the slow side more often in our measurements.)
        return {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).pin_memory().to(dev)
                .view(torch.bfloat16) if v.dtype == np.uint16 else
                torch.from_numpy(np.ascontiguousarray(v)).pin_memory().to(dev)
                for k, v in x.items()}

    stream = torch.cuda.current_stream(dev)
    extra_cfg = {}
    tile_ms = None
    if w_layout == "tiled" and mode == "head":
        raise SystemExit("--w-layout tiled: the drafter's head reads W row-major")

    def lm_w(t):
        """W as the verification calls take it; tiles it once for "tiled"."""
        nonlocal tile_ms
        if w_layout != "tiled":
            return t["W_bits"]
        Wt = sv.tile_w(t["W_bits"], stream=stream)
        # timed on a second, warm call into the same buffer
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        sv.tile_w(t["W_bits"], out=Wt.data, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
        tile_ms = a.elapsed_time(b)
        return Wt

    if mode == "tree":
        parent = inputs.EAGLE_LIKE_TREE
        x = inputs.tree_inputs(cfg.B, parent, cfg.d, cfg.V, w_std=cfg.w_std, sigma=cfg.sigma,
                               seed=cfg.seed)
        t = upload({k: v for k, v in x.items() if k != "parent"})
        W = lm_w(t)
        T = len(parent)
        D, P, rounds = sv.tree_shape(parent)
        R = cfg.B * (T + 1)
        dims = sv.dims_of(t["hidden_bits"], W)
        ws = torch.empty(sv.tree_workspace_bytes(dims), dtype=torch.uint8, device=dev)
        out = torch.empty((cfg.B, D + 1), dtype=torch.int32, device=dev)
        n_acc = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
        path = torch.empty((cfg.B, D), dtype=torch.int32, device=dev)
        extra_cfg = {"tree_nodes": T, "tree_depth": D, "tree_rounds": rounds}

        def whole():
            sv.verify_tree(t["hidden_bits"], W, parent, t["tokens"], t["q"],
                           t["uniforms"], out_tokens=out, n_accepted=n_acc, path_nodes=path,
                           workspace=ws, stream=stream)

        def lm_only():
            sv.lmhead(t["hidden_bits"], W, ws, stream=stream, argmax=False)
    elif mode == "head":
        if cfg.sparse is None:
            raise SystemExit("--mode head needs a workload with clusters (e.g. --config sparse_q)")
        C, M, k = cfg.sparse
        N = cfg.B * cfg.gamma
        x = inputs.clustered_head(N, cfg.d, cfg.V, C, M, w_std=cfg.w_std, seed=cfg.seed)
        t = upload(x)
        R = N
        hd = sv.HeadDims(N, cfg.d, cfg.V, C, M, k)
        ws = torch.empty(sv.sparse_head_workspace_bytes(hd), dtype=torch.uint8, device=dev)
        qi = torch.empty((N, k * M), dtype=torch.int32, device=dev)
        qv = torch.empty((N, k * M), dtype=torch.float32, device=dev)
        cl = torch.empty((N, k), dtype=torch.int32, device=dev)
        n_acc = None
        extra_cfg = {"clusters": C, "cluster_size": M, "top_k": k, "head_rows": N}

        def whole():
            sv.sparse_head(t["h_bits"], t["W_bits"], t["centroid_bits"], t["members"], k,
                           q_ids=qi, q_vals=qv, clusters=cl, workspace=ws, stream=stream)

        lm_only = whole
    else:
        x = inputs.generate(cfg) if x is None else x
        if mode == "sparse" and "q" in x:
            ids, vals = inputs.to_sparse_q(x["q"])
            x = dict(x, q_ids=ids, q_vals=vals)
            del x["q"]
            extra_cfg = {"q_entries_per_row": int(ids.shape[-1])}
        t = upload(x)
        W = lm_w(t)
        R = cfg.R
        dims = sv.dims_of(t["hidden_bits"], W)
        ws = sv.new_workspace(dims, dev)
        out = torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev)
        n_acc = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
        tgt = torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev)

        def lm_only():
            if mode == "greedy":
                sv.verify_greedy(t["hidden_bits"], W, t["draft"], out_tokens=out,
                                 n_accepted=n_acc, target_tokens=tgt, workspace=ws, stream=stream)
            else:
                # what spec_verify launches: logits kept, no argmax partials
                sv.lmhead(t["hidden_bits"], W, ws, stream=stream, argmax=False)

        def stage2():
            if mode == "sample":
                sv.accept_and_draw(dims, t["draft"], t["q"], t["uniforms"], out, n_acc, ws,
                                   stream=stream)
            elif mode == "sparse":
                sv.accept_and_draw_sparse_q(dims, t["draft"], t["q_ids"], t["q_vals"],
                                            t["uniforms"], out, n_acc, ws, stream=stream)

        def whole():
            lm_only()
            stage2()

    # For the event-timed loop: the LM-head launch alone, then the rest.
    def event_step(e0, e1):
        e0.record(stream)
        lm_only()
        e1.record(stream)
        if mode in ("sample", "sparse"):
            stage2()
        elif mode == "tree":
            whole()

    for _ in range(warmup):
        whole()
    torch.cuda.synchronize()

    # Timed region 1: K whole steps back to back -> value.
    K = steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        whole()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Timed region 2: K more steps with HIP events around each LM-head launch
    # (on the stream it runs on) -> the kernel's average duration.  Events
    # between the stages cost a few microseconds per step, so region 1 alone
    # gives the throughput.  (Tree mode: the LM-head launch is timed on its
    # own, then the whole call runs, so region 2 is not a step time.)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        event_step(*ev[i])
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    lm_ms = [a.elapsed_time(b) for a, b in ev]
    lm_avg_s = statistics.mean(lm_ms) * 1e-3

    ms_per_step = elapsed * 1e3 / K
    B, g, d, V = cfg.B, cfg.gamma, cfg.d, cfg.V
    n_host = n_acc.cpu().numpy() if n_acc is not None else None
    if mode == "head":
        C, M, k = cfg.sparse
        step_bytes = lm_bytes = perfmodel.sparse_head_bytes(R, d, C, M, k)
        flops = perfmodel.sparse_head_flops(R, d, C, M, k)
        kernel = "scores_kernel + topk_kernel + gather_kernel + qfinal_kernel"
        passes = 1
        tiled = False
    else:
        rows_g = R // B - 1                       # gamma, or T for a tree
        lm_bytes = perfmodel.lmhead_bytes(B, rows_g, d, V)
        flops = perfmodel.lmhead_flops(B, rows_g, d, V)
        if mode == "greedy":
            step_bytes = lm_bytes = perfmodel.greedy_step_bytes(B, g, d, V)
        elif mode == "sparse":
            step_bytes = perfmodel.sparse_q_step_bytes(B, g, d, V, int(t["q_ids"].shape[-1]),
                                                       int((n_host < g).sum()))
        elif mode == "tree":
            path_h = path.cpu().numpy()
            ends = [int(path_h[b, n_host[b] - 1]) if n_host[b] > 0 else -1 for b in range(B)]
            n_res = sum(1 for e in ends if e in set(parent))   # last node has children
            step_bytes = perfmodel.tree_step_bytes(B, rows_g, d, V, n_res)
        else:
            step_bytes = perfmodel.step_bytes(B, g, d, V, int((n_host < g).sum()))
        # R <= 64 rows: the streaming kernel, one launch per 64 rows; more
        # rows: the hidden rows tiled into the workspace, then one launch of
        # the ping-pong GEMM of 256-entry x 128-320-row blocks (when their
        # partials fit, as in every named workload).  The event-timed LM-head
        # stage spans both launches.
        tiled = R > 64 and -(-V // 256) <= 1024
        passes = 1 if tiled else -(-R // 64)
        kernel = "tile_w_kernel (hidden rows) + lmhead_big_kernel" if tiled else "lmhead_kernel"
        if mode == "greedy":
            kernel += " + greedy_kernel"
    # Bound by whichever roofline takes longer for the algorithmic work.
    mfma_bound = flops / perfmodel.MI355X_BF16_DENSE_FLOPS > lm_bytes / perfmodel.MI355X_HBM_BYTES_PER_S
    if mfma_bound:
        roof = {"bound": "mfma", "kernel": kernel, "achieved": flops / lm_avg_s / 1e12,
                "peak": perfmodel.MI355X_BF16_DENSE_FLOPS / 1e12, "unit": "TFLOP/s"}
        roof["frac"] = roof["achieved"] * 1e12 / perfmodel.MI355X_BF16_DENSE_FLOPS
        roof["alg_flops_per_launch"] = flops // passes
    else:
        roof = {"bound": "hbm", "kernel": kernel, "achieved": lm_bytes / lm_avg_s / 1e9,
                "peak": perfmodel.MI355X_HBM_BYTES_PER_S / 1e9, "unit": "GB/s"}
        roof["frac"] = roof["achieved"] * 1e9 / perfmodel.MI355X_HBM_BYTES_PER_S
    # committed counter runs are keyed by workload, "+tiled_w" for the tiled W
    prof_key = cfg.name + ("+tiled_w" if w_layout == "tiled" else "")
    roof["traffic"] = traffic_from_counters(prof_key) if mode == "sample" else None
    if roof["traffic"] is not None:
        roof["traffic_calibration"] = counter_calibration(prof_key)
    roof["alg_bytes_per_launch"] = lm_bytes // passes
    roof["hbm_GBps_alg"] = lm_bytes / lm_avg_s / 1e9

    metric = ("verified positions/sec + achieved HBM GB/s (% roofline), fused LM-head+verify"
              if mode != "head" else "drafter head rows/sec (clustered sparse LM head)")
    res = {
        "metric": metric,
        "mode": mode,
        "value": R * K / elapsed,
        "unit": "positions/s" if mode != "head" else "rows/s",
        "n_gpus": 1, "steps": K, "warmup": warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_with_lmhead_events": elapsed_ev * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; W ~ N(0, 0.02^2), hidden ~ N(0, 1), q = softmax(logits + noise))"
                + {"greedy": "; greedy mode: the config's sampled drafts",
                   "sparse": "; q given as (id, value) entries of its nonzeros",
                   "tree": "; a 25-node draft tree, every node drawn from q at its parent",
                   "head": "; drafter hidden rows ~ N(0, 1), disjoint random clusters"}.get(mode, ""),
        "config": {"workload": f"{cfg.name}: LM head d={d} V={V}, gamma={g}, B={B}"
                               + (f", {mode}" if mode != "sample" else "")
                               + (", W tiled" if w_layout == "tiled" else ""),
                   "B": B, "gamma": g, "d": d, "V": V, "sigma": cfg.sigma,
                   "seed": cfg.seed, "rows": R, "w_layout": w_layout if mode != "head" else "rows",
                   "parallelism": "single GPU", **extra_cfg},
        "steps_per_s": K / elapsed,
        "step_alg_bytes": step_bytes,
        "step_GBps": step_bytes * K / elapsed / 1e9,
        "step_frac_hbm_peak": step_bytes * K / elapsed / perfmodel.MI355X_HBM_BYTES_PER_S,
        "lmhead_ms_avg": statistics.mean(lm_ms), "lmhead_ms_median": statistics.median(lm_ms),
        "lmhead_launches_per_step": passes,
        "mfma_frac": flops / lm_avg_s / perfmodel.MI355X_BF16_DENSE_FLOPS,
        "mfma_busy_frac_counters": mfma_busy_from_counters(prof_key) if mode == "sample" else None,
        "shader_clock_ghz_counters": mfma_counters(prof_key)["clock_ghz"] if mode == "sample" else None,
        "roofline": roof,
    }
    if tile_ms is not None:
        res["tile_w_ms_once"] = tile_ms
    if n_host is not None:
        res["emitted_tokens_per_s"] = float((n_host + 1).sum()) * K / elapsed
        res["n_accepted"] = n_host.tolist()[:16]
        if mode in ("sample", "greedy", "sparse"):
            # empirical acceptance rate: accepts over the accept tests the
            # batch actually ran (checking stops at the first rejection)
            tests = np.minimum(n_host + 1, g).sum()
            res["alpha_empirical"] = float(n_host.sum()) / float(tests) if tests else None
            res["mean_accepted_per_seq"] = float(n_host.mean())
    del t, ws
    if mode != "head":
        del W
    torch.cuda.synchronize()
    return res, x


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="sweep_b256_s0.5")
    ap.add_argument("--extra-config", default="gemma_e2b",
                    help="a second workload measured the same way, reported under 'extra' "
                         "('none' to skip)")
    ap.add_argument("--mode", choices=("sample", "greedy", "sparse", "tree", "head"),
                    default="sample")
    ap.add_argument("--w-layout", choices=("rows", "tiled"), default="rows",
                    help="W as the verification calls take it: [V][d] row-major, or its "
                         "SV_W_TILED copy made once before timing")
    ap.add_argument("--no-tiled-extra", action="store_true",
                    help="skip the second measurement of the workload with W tiled "
                         "(reported under 'tiled_w' when the main run takes W row-major)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the verification step here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    if args.copy_probe_mib:
        n = args.copy_probe_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
        return

    from synth import inputs

    res, x = measure(inputs.CONFIGS[args.config], args.mode, args.steps, args.warmup, dev,
                     args.w_layout)
    if args.w_layout == "rows" and args.mode == "sample" and not args.no_tiled_extra:
        # the same steps on the same inputs with W's tiled copy (made once,
        # before timing): what a deployment that tiles W at load time gets
        tw, _ = measure(inputs.CONFIGS[args.config], args.mode, args.steps, args.warmup, dev,
                        "tiled", x=x)
        res["tiled_w"] = {k: tw[k] for k in ("value", "unit", "ms_per_step", "lmhead_ms_avg",
                                             "mfma_frac", "roofline", "tile_w_ms_once")}
    if args.extra_config != "none" and args.extra_config != args.config:
        ex, _ = measure(inputs.CONFIGS[args.extra_config], args.mode, args.steps, args.warmup,
                        dev, args.w_layout)
        keep = ("value", "unit", "ms_per_step", "steps_per_s", "step_GBps",
                "step_frac_hbm_peak", "lmhead_ms_avg", "mfma_frac", "roofline", "config",
                "emitted_tokens_per_s")
        res["extra"] = {args.extra_config: {k: ex[k] for k in keep if k in ex}}
    res["achievable_copy_GBps"] = copy_bandwidth(dev)
    if not args.no_cpu_baseline and args.mode in ("sample", "greedy"):
        res["cpu_baseline"] = cpu_baseline(x, greedy=args.mode == "greedy",
                                           gpu_value=res["value"])
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
