"""Benchmark of the verification step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--mode sample|greedy]

One step is the whole path on one batch of resident synthetic inputs: the
LM-head GEMM over all B*(gamma+1) rows (one pass over W), the softmax
normalisers, the accept tests, the first rejection and the replacement/bonus
draw.  The timed loops call the library's two stage entry points back to back
(exactly the launches spec_verify makes).  The first loop gives the
throughput; a second loop with HIP events around each LM-head launch gives
that kernel's average duration for the roofline.  Prints one JSON line.

Default workload: the Gemma-4-E2B-shaped head (d=1536, V=262144, gamma=4,
B=1).  Other named workloads are in synth.inputs.CONFIGS.

--mode greedy times greedy (match) verification instead: spec_verify_greedy,
whose LM-head launch keeps only argmax/softmax partials (no logits in HBM),
then the per-sequence greedy kernel; events bracket the whole call.
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

COUNTERS = os.path.join(ROOT, "profiles", "lmhead_gemma_e2b_counters.json")
KERNEL_SOURCES = ["draft_token_verification_02_amd/csrc/lmhead.hip",
                  "draft_token_verification_02_amd/csrc/sv_common.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_counters(cfg_name: str):
    """HBM bytes per LM-head launch from committed rocprofv3 counter runs.

    None when there is no summary for this workload or the kernel source has
    changed since the counters were taken.
    """
    if not os.path.exists(COUNTERS):
        return None
    with open(COUNTERS) as f:
        c = json.load(f)
    if c.get("workload") != cfg_name or c.get("kernel_hash") != kernel_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def cpu_baseline(x: dict, budget_s: float = 20.0, greedy: bool = False) -> dict:
    """Time the fp64 oracle (as it stands) on the same inputs, on the host."""
    from threadpoolctl import threadpool_info
    from oracle import greedy_ref, verify_ref
    times = []
    t_end = time.perf_counter() + budget_s
    while True:
        t0 = time.perf_counter()
        if greedy:
            greedy_ref.verify_greedy(x["hidden_bits"], x["W_bits"], x["draft"])
        else:
            verify_ref.verify(x["hidden_bits"], x["W_bits"], x["draft"], x["q"], x["uniforms"])
        times.append(time.perf_counter() - t0)
        if len(times) >= 3 or time.perf_counter() + times[-1] > t_end:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    B, g1 = x["hidden_bits"].shape[:2]
    t = statistics.median(times)
    return {"value": B * g1 / t, "unit": "positions/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} full steps of the same workload (median {t:.2f} s per step, "
                      f"fp64 numpy, BLAS threads={threads}, host cpus={os.cpu_count()})"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="gemma_e2b")
    ap.add_argument("--mode", choices=("sample", "greedy"), default="sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the verification step here runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
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

    import draft_token_verification_02_amd as sv
    from synth import inputs

    cfg = inputs.CONFIGS[args.config]
    x = inputs.generate(cfg)
    # Upload through pinned host copies.  (Where a large tensor lands in HBM
    # can move the LM-head time by ~10% at d = 4096; uploads from pageable
    # host memory landed on the slow side more often in our measurements.)
    t = {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).pin_memory().to(dev).view(torch.bfloat16)
         if v.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(v)).pin_memory().to(dev)
         for k, v in x.items()}
    hidden, W = t["hidden_bits"], t["W_bits"]
    dims = sv.dims_of(hidden, W)
    ws = sv.new_workspace(dims, dev)
    out = torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev)
    n_acc = torch.empty((cfg.B,), dtype=torch.int32, device=dev)
    tgt = torch.empty((cfg.B, cfg.gamma + 1), dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    greedy = args.mode == "greedy"

    def stage1():
        if greedy:
            sv.verify_greedy(hidden, W, t["draft"], out_tokens=out, n_accepted=n_acc,
                             target_tokens=tgt, workspace=ws, stream=stream)
        else:
            sv.lmhead(hidden, W, ws, stream=stream)

    def stage2():
        if not greedy:
            sv.accept_and_draw(dims, t["draft"], t["q"], t["uniforms"], out, n_acc, ws, stream=stream)

    def step():
        stage1()
        stage2()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region 1: K whole steps back to back -> value.
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Timed region 2: K more steps with HIP events around each LM-head launch
    # (on the stream it runs on) -> the kernel's average duration.  Events
    # between the stages cost a few microseconds per step, so region 1 alone
    # gives the throughput.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        ev[i][0].record(stream)
        stage1()
        ev[i][1].record(stream)
        stage2()
    torch.cuda.synchronize()
    elapsed_ev = time.perf_counter() - t1
    lm_ms = [a.elapsed_time(b) for a, b in ev]

    n_host = n_acc.cpu().numpy()
    R = cfg.R
    ms_per_step = elapsed * 1e3 / K
    n_rejected = int((n_host < cfg.gamma).sum())
    if greedy:
        step_bytes = perfmodel.greedy_step_bytes(cfg.B, cfg.gamma, cfg.d, cfg.V)
        lm_bytes = step_bytes
    else:
        step_bytes = perfmodel.step_bytes(cfg.B, cfg.gamma, cfg.d, cfg.V, n_rejected)
        lm_bytes = perfmodel.lmhead_bytes(cfg.B, cfg.gamma, cfg.d, cfg.V)
    # R <= 64 rows: the streaming kernel, one launch per 64 rows; more rows:
    # the LDS-tiled GEMM in one launch (when its partials fit, as in every
    # named workload).  The achieved figure is the stage's algorithmic bytes
    # (or flops) over the whole stage's time.
    tiled = R > 64 and -(-cfg.V // 256) <= 1024
    passes = 1 if tiled else -(-R // 64)
    kernel = "lmhead_tiled_kernel" if tiled else "lmhead_kernel"
    if greedy:
        kernel += " + greedy_kernel"
    lm_avg_s = statistics.mean(lm_ms) * 1e-3
    flops = perfmodel.lmhead_flops(cfg.B, cfg.gamma, cfg.d, cfg.V)
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
    roof["traffic"] = None if greedy or tiled else traffic_from_counters(cfg.name)
    roof["alg_bytes_per_launch"] = lm_bytes // passes
    roof["hbm_GBps_alg"] = lm_bytes / lm_avg_s / 1e9

    res = {
        "metric": "verified positions/sec (fused LM-head + verify); LM-head HBM GB/s in roofline",
        "mode": args.mode,
        "value": R * K / elapsed,
        "unit": "positions/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_with_lmhead_events": elapsed_ev * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; W ~ N(0, 0.02^2), hidden ~ N(0, 1), q = softmax(logits + noise))"
                + ("; greedy mode: the config's sampled drafts" if greedy else ""),
        "config": {"workload": f"{cfg.name}: LM head d={cfg.d} V={cfg.V}, gamma={cfg.gamma}, B={cfg.B}",
                   "B": cfg.B, "gamma": cfg.gamma, "d": cfg.d, "V": cfg.V, "sigma": cfg.sigma,
                   "seed": cfg.seed, "rows": R, "parallelism": "single GPU"},
        "steps_per_s": K / elapsed,
        "emitted_tokens_per_s": float((n_host + 1).sum()) * K / elapsed,
        "step_alg_bytes": step_bytes,
        "step_GBps": step_bytes * K / elapsed / 1e9,
        "step_frac_hbm_peak": step_bytes * K / elapsed / perfmodel.MI355X_HBM_BYTES_PER_S,
        "lmhead_ms_avg": statistics.mean(lm_ms), "lmhead_ms_median": statistics.median(lm_ms),
        "lmhead_launches_per_step": passes,
        "mfma_frac": flops / (statistics.mean(lm_ms) * 1e-3) / perfmodel.MI355X_BF16_DENSE_FLOPS,
        "roofline": roof,
        "n_accepted": n_host.tolist()[:16],
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(x, greedy=greedy)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
