"""fp64 CPU oracle for the target-side verification step of speculative decoding.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and it never imports the
product path.  It shares no code with the GPU side: the only common module is
the seeded input generator, which holds none of this arithmetic.

What is computed, and where the pages state it
----------------------------------------------
[SD]  "推测解码" (Speculative decoding), world.lapla.si/zh/specdec:
      - section 先让小模型猜 ("let the small model guess"): the target scores the
        gamma drafted positions plus one more in a single read of its weights;
      - section 通过的规则 ("the acceptance rule"): with target probability p and
        drafter probability q of a drafted token, keep it outright when q <= p,
        otherwise keep it only when a uniform draw r in [0, 1] satisfies
        r <= p/q (keep probability min(1, p/q)); on rejection the replacement
        is drawn from max(0, p - q) renormalised;
      - section 留下对的，换掉错的 ("keep the right, replace the wrong"): checking
        stops at the first rejected draft, every later draft is discarded, and
        when all gamma drafts pass the already-computed (gamma+1)-th position
        yields one bonus token, so each step emits 1..gamma+1 tokens;
      - section 和大模型写的一样 ("the same as the big model"): the emitted token
        is distributed exactly as p, because min(p, q) + (p - min(p, q)) = p;
      - section 接受率 α ("acceptance rate"): alpha = sum_x min(p, q) and the
        expected tokens per weight read (1 - alpha^(gamma+1)) / (1 - alpha);
      - section 快多少 ("how much faster"): the speedup model with drafter cost c.
[MTP] "多詞元預測視覺化指南" (A visual guide to multi-token prediction),
      gemma.gh.miniasp.com, section 高效嵌入器 ("efficient embedder"): the LM
      head multiplies the final hidden states by the (tied) embedding matrix to
      get logits, i.e. token probabilities after a softmax.

Readings taken where the pages are silent (each is listed in the design notes):
  * inputs are the bf16 tensors themselves; the oracle decodes them exactly;
  * W is [V, d] row-major (the embedding table), logits = hidden @ W^T;
  * p = softmax(logits) at temperature 1;
  * the accept test is evaluated as r * q <= p (ties accept, no division);
  * an out-of-range draft id is rejected with p = 0 and flagged;
  * uniforms[b, i] for i < gamma feed the accept tests, uniforms[b, gamma]
    is the single replacement/bonus draw;
  * the draw is an inverse CDF over ascending token id: the smallest j with
    C_j >= u * S, where C is the running sum of the weights and S = C[-1];
  * if the residual sums to S <= 0 the replacement is drawn from p instead
    (flagged);
  * q is used exactly as supplied (not renormalised).

Everything is float64 unless stated.  Loops over sequences are plain Python;
each step is one numpy operation over the vocabulary.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

ACCEPT_BAND = 1e-5   # decision-boundary band for the accept test, |r - p/q|
SAMPLE_BAND = 1e-5   # decision-boundary band for the draw, in normalised-CDF units
GEMM_CHUNK_ROWS = 8192


# --------------------------------------------------------------------------
# Step 0: exact bf16 decode.
# --------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64.

    bfloat16 is the top half of an IEEE binary32, so placing the 16 bits in
    the high half of a 32-bit word gives the same number as a binary32, which
    float64 represents exactly.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Step 1: LM-head logits ([MTP] 高效嵌入器; [SD] 先让小模型猜).
# --------------------------------------------------------------------------
def lmhead_logits(hidden_bits: np.ndarray, W_bits: np.ndarray,
                  chunk_rows: int = GEMM_CHUNK_ROWS) -> np.ndarray:
    """logits[r, v] = sum_k hidden[r, k] * W[v, k], in float64.

    hidden_bits: uint16 [R, d]; W_bits: uint16 [V, d].  W is decoded a chunk of
    rows at a time so the fp64 copy never exceeds chunk_rows * d * 8 bytes.
    The products of bf16 values are exact in float64 and the sums carry only
    float64 rounding.
    """
    X = bf16_to_f64(hidden_bits)
    V = W_bits.shape[0]
    out = np.empty((X.shape[0], V), dtype=np.float64)
    for v0 in range(0, V, chunk_rows):
        v1 = min(V, v0 + chunk_rows)
        out[:, v0:v1] = X @ bf16_to_f64(W_bits[v0:v1]).T
    return out


# --------------------------------------------------------------------------
# Step 2: target probabilities p = softmax(logits) (temperature 1).
# --------------------------------------------------------------------------
def softmax_rows(L: np.ndarray):
    """Return (p, m, lse) with m = max_j L_j, lse = m + log sum_j exp(L_j - m)."""
    m = L.max(axis=-1)
    z = np.exp(L - m[..., None]).sum(axis=-1)
    lse = m + np.log(z)
    p = np.exp(L - lse[..., None])
    return p, m, lse


# --------------------------------------------------------------------------
# Step 3: the accept test ([SD] 通过的规则).
# --------------------------------------------------------------------------
def accept_draft(p_x: float, q_x: float, r: float) -> bool:
    """Keep the drafted token iff r * q <= p.

    For q <= p this holds for every r in (0, 1] (kept outright); for q > p it
    holds iff r <= p/q, so the keep probability is min(1, p/q).  A tie
    r = p/q keeps.  q = 0 (impossible for a token drawn from q) keeps.
    """
    return bool(float(r) * float(q_x) <= float(p_x))


def accept_margin(p_x: float, q_x: float, r: float) -> float:
    """Distance of r from the decision boundary p/q (inf when q == 0)."""
    if q_x == 0.0:
        return float("inf")
    return abs(float(r) - float(p_x) / float(q_x))


# --------------------------------------------------------------------------
# Step 4: stop at the first rejection ([SD] 留下对的，换掉错的).
# --------------------------------------------------------------------------
def first_rejection(flags) -> int:
    """Number of leading accepted drafts: min{i : not flags[i]}, or len(flags)."""
    for i, f in enumerate(flags):
        if not f:
            return i
    return len(flags)


# --------------------------------------------------------------------------
# Step 5: weights of the replacement / bonus draw ([SD] 通过的规则, 留下对的).
# --------------------------------------------------------------------------
def draw_weights(p_row: np.ndarray, q_row: Optional[np.ndarray]) -> np.ndarray:
    """max(0, p - q) after a rejection; p itself for the bonus (q_row None)."""
    if q_row is None:
        return p_row.copy()
    return np.maximum(0.0, p_row - q_row.astype(np.float64))


# --------------------------------------------------------------------------
# Step 6: inverse-CDF draw over ascending token id.
# --------------------------------------------------------------------------
def inverse_cdf(w: np.ndarray, u: float):
    """Return (y, C, S, t): the smallest y with C_y >= t = u * S.

    C is the running (sequential) sum of w and S = C[-1].  With u in (0, 1]
    the draw lands on token y with probability w_y / S, and a zero-weight
    token can never be drawn.  y is clamped to the last positive-weight token.
    """
    C = np.cumsum(w)
    S = float(C[-1])
    t = float(u) * S
    y = int(np.searchsorted(C, t, side="left"))
    pos = np.flatnonzero(w > 0)
    if pos.size:
        y = min(y, int(pos[-1]))
    return y, C, S, t


def sample_margin(C: np.ndarray, S: float, t: float, y: int) -> float:
    """Distance of t from the nearer edge of y's CDF interval, divided by S."""
    lo = float(C[y - 1]) if y > 0 else 0.0
    hi = float(C[y])
    return min(t - lo, hi - t) / S


# --------------------------------------------------------------------------
# The acceptance rate and the pages' step-count formulas ([SD] 接受率 α, 快多少).
# --------------------------------------------------------------------------
def acceptance_rate(p_row: np.ndarray, q_row: np.ndarray) -> float:
    """alpha = sum_x min(p(x), q(x))."""
    return float(np.minimum(p_row, q_row.astype(np.float64)).sum())


def expected_tokens_per_step(alpha: float, gamma: int) -> float:
    """(1 - alpha^(gamma+1)) / (1 - alpha); gamma+1 when alpha == 1."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speedup(alpha: float, gamma: int, c: float) -> float:
    """Expected tokens per step divided by the step cost gamma * c + 1."""
    return expected_tokens_per_step(alpha, gamma) / (gamma * c + 1.0)


# --------------------------------------------------------------------------
# The whole step.
# --------------------------------------------------------------------------
@dataclasses.dataclass
class VerifyResult:
    out_tokens: np.ndarray      # int32 [B, gamma+1], -1 after the emitted tokens
    n_accepted: np.ndarray      # int32 [B]
    logits: np.ndarray          # float64 [R, V]
    p: np.ndarray               # float64 [R, V]
    row_max: np.ndarray         # float64 [R]
    lse: np.ndarray             # float64 [R]
    p_draft: np.ndarray         # float64 [B, gamma]  p at each drafted token (0 if out of range)
    q_draft: np.ndarray         # float64 [B, gamma]
    accept: np.ndarray          # bool [B, gamma]      every test, also those after the first rejection
    accept_margin: np.ndarray   # float64 [B, gamma]
    bad_draft: np.ndarray       # bool [B, gamma]      draft id outside [0, V)
    draw_row: np.ndarray        # int64 [B]            row (b*(gamma+1)+n) the draw used
    draw_S: np.ndarray          # float64 [B]          sum of the draw weights
    draw_t: np.ndarray          # float64 [B]          u * S
    draw_margin: np.ndarray     # float64 [B]
    draw_fallback: np.ndarray   # bool [B]             residual summed to <= 0; drew from p
    draw_cdf: list              # per sequence: the running sum C (float64 [V])
    alpha: np.ndarray           # float64 [B, gamma]   sum_x min(p, q) at each drafted position

    @property
    def accept_flagged(self) -> np.ndarray:
        return self.accept_margin < ACCEPT_BAND

    @property
    def draw_flagged(self) -> np.ndarray:
        return self.draw_margin < SAMPLE_BAND


def verify(hidden_bits: np.ndarray, W_bits: np.ndarray, draft: np.ndarray, q: np.ndarray,
           uniforms: np.ndarray, force_n: Optional[np.ndarray] = None,
           logits: Optional[np.ndarray] = None) -> VerifyResult:
    """Run the verification step for B sequences.

    hidden_bits uint16 [B, gamma+1, d]; W_bits uint16 [V, d]; draft int [B, gamma];
    q float32 [B, gamma, V]; uniforms float32 [B, gamma+1] in (0, 1].

    force_n (conditional mode): per-sequence accepted counts to use instead of
    the ones this call derives, so that a draw can be checked at the row a
    different (boundary-flagged) accept decision led to.  logits: precomputed
    float64 logits [B*(gamma+1), V] from lmhead_logits, to skip the GEMM.
    """
    B, g1, d = hidden_bits.shape
    g = g1 - 1
    V = W_bits.shape[0]
    assert draft.shape == (B, g) and q.shape == (B, g, V) and uniforms.shape == (B, g1)

    L = lmhead_logits(hidden_bits.reshape(B * g1, d), W_bits) if logits is None else logits
    p, m, lse = softmax_rows(L)

    out = np.full((B, g1), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    p_d = np.zeros((B, g)); q_d = np.zeros((B, g))
    acc = np.zeros((B, g), dtype=bool); acc_m = np.full((B, g), np.inf)
    bad = np.zeros((B, g), dtype=bool)
    row = np.zeros(B, dtype=np.int64); S_all = np.zeros(B); t_all = np.zeros(B)
    margin = np.zeros(B); fallback = np.zeros(B, dtype=bool); cdfs = []
    alpha = np.zeros((B, g))

    for b in range(B):
        r0 = b * g1
        for i in range(g):
            alpha[b, i] = acceptance_rate(p[r0 + i], q[b, i])
            x = int(draft[b, i])
            r = float(uniforms[b, i])
            if x < 0 or x >= V:
                bad[b, i] = True          # rejected with p = 0
                continue
            p_d[b, i] = p[r0 + i, x]
            q_d[b, i] = float(q[b, i, x])
            acc[b, i] = accept_draft(p_d[b, i], q_d[b, i], r)
            acc_m[b, i] = accept_margin(p_d[b, i], q_d[b, i], r)
        n = first_rejection(acc[b]) if force_n is None else int(force_n[b])
        n_acc[b] = n
        k = r0 + n
        row[b] = k
        w = draw_weights(p[k], q[b, n] if n < g else None)
        if not (w.sum() > 0.0):
            w = draw_weights(p[k], None)
            fallback[b] = True
        y, C, S, t = inverse_cdf(w, float(uniforms[b, g]))
        S_all[b], t_all[b] = S, t
        margin[b] = sample_margin(C, S, t, y)
        cdfs.append(C)
        out[b, :n] = draft[b, :n]
        out[b, n] = y

    return VerifyResult(out, n_acc, L, p, m, lse, p_d, q_d, acc, acc_m, bad, row, S_all,
                        t_all, margin, fallback, cdfs, alpha)


def draw_admissible(C: np.ndarray, S: float, u: float, y: int, band: float = SAMPLE_BAND) -> bool:
    """Whether token y is within ``band`` (normalised-CDF units) of u's interval.

    Used for draws flagged as lying near a CDF boundary: another token is an
    acceptable answer there only if u sits within the band of its interval.
    """
    if y < 0 or y >= C.shape[0]:
        return False
    lo = (float(C[y - 1]) if y > 0 else 0.0) / S
    hi = float(C[y]) / S
    return lo - band <= float(u) <= hi + band
