"""fp64 CPU oracle for the drafter's clustered sparse LM head and the sparse-q
form of verification.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; it shares no
code with the HIP path and never imports it.

What is computed, and where the pages state it
----------------------------------------------
[MTP] "多詞元預測視覺化指南" (gemma.gh.miniasp.com), section 高效嵌入器: the
      drafter's output head does not score every token.  The tokens' embeddings
      are grouped offline into clusters of similar tokens, each with one
      embedding of its own; multiplying the hidden state by that small table
      gives cluster logits, the clusters most likely to hold the next token are
      chosen, and token logits are computed only for the tokens of the chosen
      clusters.
[SD]  "推测解码" (world.lapla.si/zh/specdec), section 通过的规则: the verifier
      needs the drafter's probability q of each drafted token and, after a
      rejection, max(0, p - q) over the vocabulary.

Readings taken where the pages are silent:
  * the clustering is an input: `members` [C][M] lists the token ids of each
    cluster (every id in [0, V) at most once); the cluster embedding table
    `centroids` [C][d] is an input too (the synthetic workloads use the mean
    of the member rows, rounded to bf16);
  * "the most likely clusters" are the k with the largest cluster logits,
    ties to the lower cluster index;
  * the drafter's q is the softmax, at temperature 1, of the token logits
    h . W[j] over the selected tokens only, and exactly 0 elsewhere;
  * the sparse q row is handed over as (ids ascending, values); verification
    with it is verification with the dense row that has those values at those
    ids and 0 elsewhere, so the verifier's oracle is verify_ref.verify on the
    densified q.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from oracle.verify_ref import bf16_to_f64, lmhead_logits

# Cluster-score band: a row whose k-th and (k+1)-th cluster logits lie closer
# than this may select a different set in fp32; such rows are flagged.
TOPK_BAND = 1e-4


def cluster_logits(h_bits: np.ndarray, centroid_bits: np.ndarray) -> np.ndarray:
    """scores[n, c] = h[n] . centroid[c] in float64 (exact products, fp64 sums)."""
    return bf16_to_f64(h_bits) @ bf16_to_f64(centroid_bits).T


def top_clusters(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the lower index, ascending.

    A stable sort on the negated scores keeps equal scores in index order, so
    its first k entries are exactly the k largest with lower indices first.
    """
    order = np.argsort(-scores, kind="stable")
    return np.sort(order[:k])


def topk_margin(scores: np.ndarray, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest scores (inf if k == C)."""
    if k >= scores.shape[0]:
        return float("inf")
    s = np.sort(scores)[::-1]
    return float(s[k - 1] - s[k])


def selected_tokens(members: np.ndarray, clusters: np.ndarray) -> np.ndarray:
    """Token ids of the chosen clusters, ascending."""
    return np.sort(members[clusters].ravel())


@dataclasses.dataclass
class SparseHeadResult:
    idx: np.ndarray          # int64 [N, K]  selected token ids, ascending per row
    val: np.ndarray          # float64 [N, K] q at those ids (each row sums to 1)
    clusters: np.ndarray     # int64 [N, k]  chosen clusters, ascending
    scores: np.ndarray       # float64 [N, C] cluster logits
    logits: np.ndarray       # float64 [N, K] token logits at idx
    margin: np.ndarray       # float64 [N]   k-th minus (k+1)-th cluster logit

    @property
    def flagged(self) -> np.ndarray:
        return self.margin < TOPK_BAND


def sparse_head(h_bits: np.ndarray, W_bits: np.ndarray, centroid_bits: np.ndarray,
                members: np.ndarray, k: int) -> SparseHeadResult:
    """The drafter's clustered head for N hidden rows.

    h_bits uint16 [N, d]; W_bits uint16 [V, d]; centroid_bits uint16 [C, d];
    members int [C, M].  Returns q over the k*M selected tokens of each row.
    """
    N = h_bits.shape[0]
    scores = cluster_logits(h_bits, centroid_bits)
    K = k * members.shape[1]
    idx = np.zeros((N, K), dtype=np.int64)
    val = np.zeros((N, K))
    lg = np.zeros((N, K))
    cl = np.zeros((N, k), dtype=np.int64)
    margin = np.zeros(N)
    for n in range(N):
        cl[n] = top_clusters(scores[n], k)
        margin[n] = topk_margin(scores[n], k)
        idx[n] = selected_tokens(members, cl[n])
        lg[n] = lmhead_logits(h_bits[n:n + 1], W_bits[idx[n]])[0]
        m = lg[n].max()
        e = np.exp(lg[n] - m)
        val[n] = e / e.sum()
    return SparseHeadResult(idx, val, cl, scores, lg, margin)


def densify(idx: np.ndarray, val: np.ndarray, V: int) -> np.ndarray:
    """Dense rows with val at idx and 0 elsewhere (leading dims kept)."""
    lead = idx.shape[:-1]
    out = np.zeros(lead + (V,))
    flat_i = idx.reshape(-1, idx.shape[-1])
    flat_v = val.reshape(-1, val.shape[-1])
    flat_o = out.reshape(-1, V)
    for r in range(flat_i.shape[0]):
        flat_o[r, flat_i[r]] = flat_v[r]
    return out
