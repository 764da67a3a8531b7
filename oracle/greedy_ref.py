"""fp64 CPU oracle for greedy (match) verification of drafted tokens.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; it shares no
code with the HIP path and never imports it.

What is computed, and where the pages state it
----------------------------------------------
[ND]   the maxstudionews.com article 1664 on multi-token prediction for the
       on-device Gemini Nano model (no title in its extracted text), the
       paragraph on the draft / verify split: the large model checks the
       drafted tokens in one parallel pass, keeps those that agree with its
       own prediction and falls back to the first point of disagreement; the
       paragraph after the frozen-backbone description: because wrong drafts
       are discarded, the output stays bit-for-bit the main model's own.
[SD]   "推测解码" (world.lapla.si/zh/specdec), section 先让小模型猜: checking a
       guess against the large model was possible before the sampling rule,
       but only for greedy decoding; section 留下对的，换掉错的: stop at the
       first failed draft, replace it with the large model's own token, or
       emit one bonus token when every draft passes.

Readings taken where the pages are silent:
  * the large model's "prediction" at a position is its greedy token, the
    argmax of that row's logits (equivalently of p; softmax is monotone);
  * ties in the maximum go to the lowest token id;
  * NaN logits never win; a row with no entry above -inf has no greedy token
    (flagged; the emitted token is 0, as for a non-finite sampling row);
  * an out-of-range draft id never matches (flagged).

The fp64 logits come from the same exact bf16 decode and GEMM as the sampling
oracle.  A GPU computing in fp32 may pick another token only where the top two
logits of a row lie within ARGMAX_BAND of each other; such rows are flagged,
and the tokens within the band of the maximum are all admissible there.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from oracle.verify_ref import first_rejection, lmhead_logits

# Logit-gap band for near-ties.  The GPU sums d bf16 products in fp32; over the
# workloads here its logits differ from the exact ones by ~1e-5 at most, well
# inside this band, and a random pair of top logits falls this close in well
# under one row in a thousand.
ARGMAX_BAND = 1e-4


def greedy_token(row: np.ndarray) -> int:
    """Lowest token id attaining the row maximum; -1 if no entry is above -inf.

    Written as the scan it is: ascending ids, replace only on a strictly larger
    value, so the first maximum stays and NaN (never larger) never wins.
    """
    best, arg = -np.inf, -1
    for j, v in enumerate(row.tolist()):
        if v > best:
            best, arg = v, j
    return arg


def greedy_tokens(L: np.ndarray) -> np.ndarray:
    """greedy_token for every row, vectorised: numpy's argmax returns the first
    maximum; NaN entries are masked to -inf first and an all-(-inf) row gives -1."""
    M = np.where(np.isnan(L), -np.inf, L)
    arg = np.argmax(M, axis=-1).astype(np.int64)
    arg[~(M.max(axis=-1) > -np.inf)] = -1
    return arg


def top_gap(row: np.ndarray, y: int) -> float:
    """row[y] minus the largest other entry (inf for a single-entry row)."""
    if y < 0:
        return 0.0
    M = np.where(np.isnan(row), -np.inf, row)
    other = np.delete(M, y)
    return float(M[y] - other.max()) if other.size else float("inf")


def near_ties(row: np.ndarray, band: float = ARGMAX_BAND) -> np.ndarray:
    """Token ids whose logit lies within ``band`` of the row maximum."""
    M = np.where(np.isnan(row), -np.inf, row)
    return np.flatnonzero(M >= M.max() - band)


@dataclasses.dataclass
class GreedyResult:
    out_tokens: np.ndarray      # int32 [B, gamma+1], -1 after the emitted tokens
    n_accepted: np.ndarray      # int32 [B]
    target: np.ndarray          # int64 [B, gamma+1]  greedy token of every row (-1: none)
    gap: np.ndarray             # float64 [B, gamma+1] top-1 minus top-2 logit
    match: np.ndarray           # bool [B, gamma]     draft i equals the row-i greedy token
    bad_draft: np.ndarray       # bool [B, gamma]     draft id outside [0, V)
    nonfinite: np.ndarray       # bool [B]            emitted row had no greedy token
    logits: np.ndarray          # float64 [R, V]

    @property
    def flagged(self) -> np.ndarray:
        """Rows whose greedy token an fp32 computation may legitimately change."""
        return self.gap < ARGMAX_BAND


def verify_greedy(hidden_bits: np.ndarray, W_bits: np.ndarray, draft: np.ndarray,
                  force_n: Optional[np.ndarray] = None,
                  logits: Optional[np.ndarray] = None) -> GreedyResult:
    """Greedy verification of B sequences of gamma drafts.

    hidden_bits uint16 [B, gamma+1, d]; W_bits uint16 [V, d]; draft int [B, gamma].
    Draft i of sequence b is kept while it equals the greedy token of row i;
    the first mismatch n is replaced by row n's greedy token (n = gamma: the
    bonus token of the last row).  force_n and logits as in verify_ref.verify.
    """
    B, g1, d = hidden_bits.shape
    g = g1 - 1
    V = W_bits.shape[0]
    assert draft.shape == (B, g)
    L = lmhead_logits(hidden_bits.reshape(B * g1, d), W_bits) if logits is None else logits
    tgt = greedy_tokens(L).reshape(B, g1)
    gap = np.array([top_gap(L[r], int(t)) for r, t in enumerate(tgt.ravel())]).reshape(B, g1)

    out = np.full((B, g1), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    match = np.zeros((B, g), dtype=bool)
    bad = np.zeros((B, g), dtype=bool)
    nonfin = np.zeros(B, dtype=bool)
    for b in range(B):
        for i in range(g):
            x = int(draft[b, i])
            bad[b, i] = not (0 <= x < V)
            match[b, i] = (not bad[b, i]) and x == int(tgt[b, i])
        n = first_rejection(match[b]) if force_n is None else int(force_n[b])
        n_acc[b] = n
        out[b, :n] = draft[b, :n]
        y = int(tgt[b, n])
        nonfin[b] = y < 0
        out[b, n] = y if y >= 0 else 0
    return GreedyResult(out, n_acc, tgt, gap, match, bad, nonfin, L)
