"""Byte, flop and roofline accounting for the verification step.

Used by the benchmark to turn measured times into bandwidth and MFMA
fractions.  The paper-arithmetic helper reproduces the decode-cost reasoning of
the speculative-decoding explainer "推测解码" (world.lapla.si/zh/specdec,
sections 一次一个词元 "one token at a time", 几段话一起写 "batching" and
剖开读头 "the read head"): weights are read once per step, the step's time is
at least bytes / bandwidth, and arithmetic is busy for ops / peak of that time.
"""

from __future__ import annotations

# MI355X published peaks.
MI355X_HBM_BYTES_PER_S = 8.0e12
MI355X_BF16_DENSE_FLOPS = 2.5e15
MI355X_FP32_VECTOR_FLOPS = 157.3e12


def paper_decode(params: int, bytes_per_param: float, hbm_bytes_per_s: float,
                 dense_ops_per_s: float, batch: int = 1, kv_bytes_per_token: float = 0.0,
                 context_tokens: int = 0) -> dict:
    """Bandwidth-bound decode arithmetic for one step of ``batch`` sequences.

    Every step streams all weights once plus each sequence's own KV cache; one
    token per sequence comes out; 2 ops per parameter per token.
    """
    weight_bytes = params * bytes_per_param
    kv_bytes = batch * kv_bytes_per_token * context_tokens
    step_s = (weight_bytes + kv_bytes) / hbm_bytes_per_s
    ops = 2.0 * params * batch
    return {
        "weight_bytes": weight_bytes,
        "kv_bytes": kv_bytes,
        "step_bytes": weight_bytes + kv_bytes,
        "step_s": step_s,
        "tokens_per_s": batch / step_s,
        "ops_per_step": ops,
        "busy_frac": (ops / dense_ops_per_s) / step_s,
        "ops_per_byte_peak": dense_ops_per_s / hbm_bytes_per_s,
    }


def rows(B: int, gamma: int) -> int:
    """Rows scored per step: gamma drafted positions plus one, per sequence."""
    return B * (gamma + 1)


def lmhead_bytes(B: int, gamma: int, d: int, V: int) -> int:
    """Minimum HBM bytes of the LM-head stage: W and hidden read once, logits written once."""
    R = rows(B, gamma)
    return 2 * V * d + 2 * R * d + 4 * R * V


def step_bytes(B: int, gamma: int, d: int, V: int, n_rejected: int) -> int:
    """Minimum HBM bytes of the whole verification step.

    W + hidden + logits written once + the drawn row's logits read back per
    sequence + the drawn row's q for every rejected sequence + the small
    per-draft gathers, uniforms and outputs.
    """
    R = rows(B, gamma)
    small = 4 * B * gamma * 3 + 4 * B * (gamma + 1) * 2 + 4 * B
    return lmhead_bytes(B, gamma, d, V) + 4 * B * V + 4 * V * n_rejected + small


def lmhead_flops(B: int, gamma: int, d: int, V: int) -> int:
    return 2 * rows(B, gamma) * V * d


def greedy_step_bytes(B: int, gamma: int, d: int, V: int) -> int:
    """Minimum HBM bytes of greedy verification: W and hidden read once; the
    argmax needs no logits in memory.  Plus drafts and outputs."""
    R = rows(B, gamma)
    small = 4 * B * gamma + 4 * B * (gamma + 1) * 2 + 4 * B
    return 2 * V * d + 2 * R * d + small


def sparse_q_step_bytes(B: int, gamma: int, d: int, V: int, K: int, n_rejected: int) -> int:
    """Minimum HBM bytes of verification with sparse q: as step_bytes, but a
    rejected sequence reads its q row's K (id, value) entries instead of V
    floats, and the accept tests' lookups read each drafted row's K entries."""
    R = rows(B, gamma)
    small = 4 * B * gamma * 2 + 4 * B * (gamma + 1) * 2 + 4 * B
    return (lmhead_bytes(B, gamma, d, V) + 4 * B * V + 8 * K * (B * gamma + n_rejected)
            + small)


def tree_lmhead_bytes(B: int, T: int, d: int, V: int) -> int:
    """LM-head bytes of tree verification: one row per node plus the root."""
    return lmhead_bytes(B, T, d, V)


def tree_step_bytes(B: int, T: int, d: int, V: int, n_residual: int) -> int:
    """Minimum HBM bytes of tree verification: the LM head over B*(T+1) rows,
    the drawn row's logits per sequence and its q row when the draw is from a
    residual (n_residual sequences), plus the per-node gathers and outputs.
    Sums for rejected siblings before the last are extra passes over a row
    that this lower bound leaves out."""
    small = 4 * B * T * 3 + 4 * B * (T + 1) + 8 * B
    return lmhead_bytes(B, T, d, V) + 4 * B * V + 4 * V * n_residual + small


def sparse_head_bytes(N: int, d: int, C: int, M: int, k: int) -> int:
    """Minimum HBM bytes of the clustered head for N rows: the cluster table
    once, every chosen token's W row once per row that chose it, the hidden
    rows, the members of the chosen clusters, and the (id, q) outputs."""
    K = k * M
    return 2 * C * d + 2 * N * K * d + 2 * N * d + 4 * N * K + 8 * N * K


def sparse_head_flops(N: int, d: int, C: int, M: int, k: int) -> int:
    return 2 * N * d * (C + k * M)
