"""Byte/roofline accounting, pinned to the explainer's H100 paper arithmetic."""

import json
import os

import perfmodel as M

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "h100_paper_arithmetic.json")


def test_h100_paper_arithmetic():
    g = json.load(open(GOLDEN, encoding="utf-8"))
    i, pr = g["inputs"], g["printed"]
    one = M.paper_decode(i["params"], i["bytes_per_param"], i["hbm_bytes_per_s"], i["dense_ops_per_s"])
    assert round(one["weight_bytes"] / 1e9) == pr["model_gb"]
    assert round(one["step_s"] * 1e3, 1) == pr["ms_per_token"]
    assert round(one["tokens_per_s"]) == pr["tokens_per_s_batch1"]
    assert round(one["ops_per_step"] / 1e9) == pr["ops_per_token_g"]
    assert round(one["busy_frac"] * 100, 1) == pr["busy_pct_batch1"]
    assert round(one["ops_per_byte_peak"]) == pr["ops_per_byte"]
    b64 = M.paper_decode(i["params"], i["bytes_per_param"], i["hbm_bytes_per_s"], i["dense_ops_per_s"], batch=64)
    assert abs(b64["tokens_per_s"] - pr["tokens_per_s_batch64"]) / pr["tokens_per_s_batch64"] < 0.005
    assert round(b64["busy_frac"] * 100) == pr["busy_pct_batch64"]
    kv = M.paper_decode(i["params"], i["bytes_per_param"], i["hbm_bytes_per_s"], i["dense_ops_per_s"],
                        batch=64, kv_bytes_per_token=i["kv_bytes_per_token"], context_tokens=i["context_tokens"])
    assert round(kv["kv_bytes"] / 1e9) == pr["kv_extra_gb_batch64"]
    assert abs(kv["tokens_per_s"] - pr["tokens_per_s_batch64_kv"]) / pr["tokens_per_s_batch64_kv"] < 0.01
    assert round(kv["step_bytes"] / 1e9) == pr["gb_per_step_batch64_kv"]
    assert round(9 / one["ops_per_byte_peak"] * 100) == pr["lanes_9_busy_pct"]


def test_verify_step_bytes():
    # Gemma-shaped head, one sequence, gamma = 4, one rejected sequence.
    assert M.lmhead_bytes(1, 4, 1536, 262144) == 2 * 262144 * 1536 + 2 * 5 * 1536 + 4 * 5 * 262144
    b = M.step_bytes(1, 4, 1536, 262144, 1)
    assert abs(b / 1e6 - 812.7) < 0.1
    assert abs(M.step_bytes(256, 4, 4096, 128256, 256) / 1e6 - 1980.5) < 0.2
    assert M.lmhead_flops(1, 4, 1536, 262144) == 2 * 5 * 262144 * 1536
