"""fp64 CPU oracle of tree verification: several drafted candidates per
position, checked with the same keep-or-replace rule at every fork.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; it shares no
code with the HIP path and never imports it.

What the pages fix, and the reading taken where they stop
---------------------------------------------------------
[SD]  "推测解码" (world.lapla.si/zh/specdec):
      section 通过的规则 -- a drafted token x is kept with probability
        min(1, p(x)/q(x)); after a rejection the replacement comes from
        max(0, p - q) renormalised, and the emitted token is then distributed
        as p;
      section 留下对的，换掉错的 -- stop at the first rejection; when every
        draft passes, the target's own distribution at the next position
        gives one more token;
      section on later methods (Medusa / EAGLE) -- the guesses may form a
        tree that is checked in one pass, and EAGLE applies the same rule at
        every fork of its guess tree, which leaves the distribution unchanged.
The pages do not spell out how several siblings are checked.  The plainest
reading that keeps the distribution, taken here:
  * the tree is a static topology: node t (0..T-1) has parent[t] < t, or -1
    for a child of the root; the target scores one row per position -- row 0
    for the root (the last context position), row t+1 for node t;
  * the candidates at a fork are the children of one node, drawn from the
    drafter's q at that node's row; they are checked one after another in
    increasing node index, each with the rule above against the *current*
    target distribution: p of the node's row for the first child, and after
    each rejection the renormalised residual max(0, cur - q) / sum;
  * a kept child is emitted and the walk continues at its row with its own
    children (a fresh p; its own q);
  * when every child of a node is rejected, the token is drawn from the
    residual left after the last rejection; at a node without children the
    bonus token is drawn from p of its row;
  * the draw is the inverse CDF over ascending token id of the chain oracle;
  * q is given only for rows that have children, in row order ("q slots");
    uniforms[b][t] is node t's accept test, uniforms[b][T] the one draw;
  * a residual with no mass (sum <= 0: only through rounding or an
    unnormalised q) stops the checking and draws from p of the node's row,
    flagged -- the chain oracle's fallback;
  * a path topology (parent[t] = t - 1) is exactly the chain step.
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np

from oracle.verify_ref import (ACCEPT_BAND, SAMPLE_BAND, accept_draft, accept_margin,
                               inverse_cdf, lmhead_logits, sample_margin, softmax_rows)


# --------------------------------------------------------------------------
# Topology
# --------------------------------------------------------------------------
def children(parent, v: int) -> List[int]:
    """Children of node v (v = -1 for the root), in increasing node index."""
    return [t for t in range(len(parent)) if int(parent[t]) == v]


def check_topology(parent) -> None:
    for t, a in enumerate(parent):
        if not (-1 <= int(a) < t):
            raise ValueError(f"parent[{t}] = {a}: parents must precede their children")


def depth_of(parent) -> np.ndarray:
    """Depth of every node (1 for the root's children)."""
    d = np.zeros(len(parent), dtype=np.int64)
    for t, a in enumerate(parent):
        d[t] = 1 if a < 0 else d[a] + 1
    return d


def max_depth(parent) -> int:
    return int(depth_of(parent).max()) if len(parent) else 0


def q_slots(parent) -> np.ndarray:
    """q slot of every row (0 = root, t+1 = node t): its rank among the rows
    with children, in row order; -1 for rows without children."""
    T = len(parent)
    has = np.zeros(T + 1, dtype=bool)
    for a in parent:
        has[int(a) + 1] = True
    slots = np.full(T + 1, -1, dtype=np.int64)
    slots[has] = np.arange(int(has.sum()))
    return slots


# --------------------------------------------------------------------------
# The sibling step ([SD] 通过的规则, applied at a fork)
# --------------------------------------------------------------------------
def residual(cur: np.ndarray, q_row: np.ndarray):
    """After a rejection against the current target ``cur``: (max(0, cur - q), its sum)."""
    w = np.maximum(0.0, cur - q_row)
    return w, float(w.sum())


@dataclasses.dataclass
class TreeResult:
    out_tokens: np.ndarray      # int32 [B, D+1]: the kept path's tokens, then the drawn one, -1 after
    n_accepted: np.ndarray      # int32 [B]
    path_nodes: np.ndarray      # int32 [B, D]: node index of every kept token, -1 after
    logits: np.ndarray          # float64 [B*(T+1), V]
    p: np.ndarray               # float64 [B*(T+1), V]
    tests: list                 # per sequence: [(node, ratio, margin, kept)] in test order
    draw_row: np.ndarray        # int64 [B]  row the draw used
    draw_S: np.ndarray          # float64 [B]
    draw_margin: np.ndarray     # float64 [B]
    draw_fallback: np.ndarray   # bool [B]
    draw_cdf: list              # per sequence: running sum of the draw weights
    bad_token: np.ndarray       # bool [B]: a tested node's token lay outside [0, V)

    @property
    def accept_flagged(self) -> np.ndarray:
        """Per sequence: some test of the walk lay within the band of its boundary."""
        return np.array([any(m < ACCEPT_BAND for (_, _, m, _) in ts) for ts in self.tests])

    @property
    def draw_flagged(self) -> np.ndarray:
        return self.draw_margin < SAMPLE_BAND


def verify_tree(hidden_bits: np.ndarray, W_bits: np.ndarray, parent, tokens: np.ndarray,
                q: np.ndarray, uniforms: np.ndarray, logits: Optional[np.ndarray] = None,
                force_path: Optional[list] = None) -> TreeResult:
    """Tree verification for B sequences.

    hidden_bits uint16 [B, T+1, d]; W_bits uint16 [V, d]; parent int [T];
    tokens int [B, T]; q float32 [B, P, V] (P = rows with children, q_slots);
    uniforms float [B, T+1] in (0, 1].  logits: precomputed float64
    [B*(T+1), V] to skip the GEMM.  force_path (conditional mode): per
    sequence, the list of nodes to keep, followed without testing; the walk
    then continues normally from the last of them -- used to check a draw at
    the node a boundary-flagged test led the GPU to.
    """
    check_topology(parent)
    B, T1, d = hidden_bits.shape
    T = T1 - 1
    assert len(parent) == T and tokens.shape == (B, T) and uniforms.shape == (B, T1)
    slots = q_slots(parent)
    assert q.shape[:2] == (B, int((slots >= 0).sum()))
    V = W_bits.shape[0]
    D = max_depth(parent)

    L = lmhead_logits(hidden_bits.reshape(B * T1, d), W_bits) if logits is None else logits
    p, _, _ = softmax_rows(L)

    out = np.full((B, D + 1), -1, dtype=np.int32)
    path_nodes = np.full((B, D), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    tests = []
    row_used = np.zeros(B, dtype=np.int64)
    S_all = np.zeros(B)
    margin = np.zeros(B)
    fallback = np.zeros(B, dtype=bool)
    bad = np.zeros(B, dtype=bool)
    cdfs = []

    for b in range(B):
        r0 = b * T1
        v = -1                       # current node (-1 = root), its row is v + 1
        kept: List[int] = []
        ts = []
        forced = list(force_path[b]) if force_path is not None else []
        while True:
            kids = children(parent, v)
            prow = p[r0 + v + 1]
            if forced:
                t = forced.pop(0)
                assert t in kids, "forced path must follow the tree"
                kept.append(t)
                v = t
                continue
            if not kids:             # a leaf: the bonus token from p
                w = prow.copy()
                break
            q_row = q[b, slots[v + 1]].astype(np.float64)
            cur = prow
            taken = None
            w = None
            for t in kids:
                x = int(tokens[b, t])
                r = float(uniforms[b, t])
                if 0 <= x < V:
                    keep = accept_draft(cur[x], q_row[x], r)
                    ratio = cur[x] / q_row[x] if q_row[x] > 0 else np.inf
                    ts.append((t, ratio, accept_margin(cur[x], q_row[x], r), keep))
                else:
                    keep = False     # out of range: rejected with p = 0
                    bad[b] = True
                    ts.append((t, 0.0, np.inf, False))
                if keep:
                    taken = t
                    break
                res, S = residual(cur, q_row)
                if not (S > 0.0):    # no residual mass: draw from p at this row
                    fallback[b] = True
                    w = prow.copy()
                    break
                cur = res / S
                last = res
            if taken is not None:
                kept.append(taken)
                v = taken
                continue
            if w is None:
                w = last             # every child rejected: the last residual (the draw normalises)
            break
        row_used[b] = r0 + v + 1
        y, C, S, tt = inverse_cdf(w, float(uniforms[b, T]))
        S_all[b] = S
        margin[b] = sample_margin(C, S, tt, y)
        cdfs.append(C)
        n = len(kept)
        n_acc[b] = n
        for i, t in enumerate(kept):
            out[b, i] = tokens[b, t]
            path_nodes[b, i] = t
        out[b, n] = y
        tests.append(ts)

    return TreeResult(out, n_acc, path_nodes, L, p, tests, row_used, S_all, margin, fallback,
                      cdfs, bad)


def worst_case_rounds(parent) -> int:
    """Largest number of residual sums one walk can need, plus its draw.

    A walk at a node with children k_1..k_m tests k_1 against p (no sum
    needed); every rejection before the last child needs the sum of the new
    residual to test the next child; the draw needs the sum of its weights.
    So: m when every child is rejected, (j - 1) + rounds(k_j) when k_j is kept,
    and 1 at a leaf.  Used to size the GPU schedule; pinned by brute force
    over every decision sequence in the tests.
    """
    def rounds(v):
        kids = children(parent, v)
        if not kids:
            return 1
        best = len(kids)
        for j, t in enumerate(kids):
            best = max(best, j + rounds(t))
        return best
    return rounds(-1)
