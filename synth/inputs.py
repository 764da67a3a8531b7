"""Seeded synthetic inputs for the target-side verification step.

This module is shared by the fp64 oracle's tests and by the GPU-side tests and
benchmark.  It builds *inputs only* and holds none of the verification
arithmetic (no accept test, no residual, no inverse-CDF sampling):

* ``hidden`` and ``W`` are Gaussian draws rounded to bfloat16 (round to
  nearest, ties to even) and stored as raw uint16 bit patterns.  Both sides of
  the parity check read these exact bf16 values.
* ``q`` (the drafter's distribution at each drafted position) is built from an
  fp32 approximation of the target logits plus Gaussian noise, softmaxed.  The
  approximation only shapes the input: neither side's logits come from here.
* draft tokens are drawn from ``q`` with the Gumbel-max trick, a sampling
  method deliberately different from the inverse CDF the verifier uses.
* ``uniforms`` are ``1 - U`` with ``U`` in [0, 1) from a Philox stream, so
  every uniform lies in (0, 1].  Slots ``0..gamma-1`` feed the accept tests,
  slot ``gamma`` the one replacement/bonus draw.

Every tensor has its own stream spawned from ``SeedSequence(seed)`` (SFC64
for the bulk Gaussian tensors, Philox for the uniforms and the cluster
permutation), so changing one shape never shifts another tensor's values.
"""

from __future__ import annotations

import dataclasses
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Optional, Tuple

import numpy as np

STREAMS = ("W", "hidden", "noise", "drafts", "uniforms", "clusters")
W_CHUNK_ROWS = 16384


@dataclasses.dataclass(frozen=True)
class Config:
    """Shape and value recipe of one synthetic verification workload."""

    name: str
    B: int          # sequences
    gamma: int      # drafted tokens per sequence
    d: int          # hidden size
    V: int          # vocabulary size
    w_std: float    # std of the LM-head weights
    h_std: float    # std of the hidden states
    sigma: float    # std of the noise added to the logits to form q
    sparse: Optional[Tuple[int, int, int]] = None  # (clusters, cluster size, top-k clusters)
    seed: int = 0

    @property
    def R(self) -> int:
        return self.B * (self.gamma + 1)


def _registry() -> Dict[str, Config]:
    reg = {}
    # Tiny check case: V=32, d=16, unit-variance weights and hidden states.
    reg["tiny"] = Config("tiny", 1, 4, 16, 32, 1.0, 1.0, 1.0)
    # Gemma-4-E2B-shaped head: d=1536, V=262144.
    reg["gemma_e2b"] = Config("gemma_e2b", 1, 4, 1536, 262144, 0.02, 1.0, 0.5)
    # Llama-3.1-8B-shaped head: d=4096, V=128256, gamma x B grid.
    for g in (2, 4, 8):
        for b in (1, 4):
            n = f"llama8b_g{g}_b{b}"
            reg[n] = Config(n, b, g, 4096, 128256, 0.02, 1.0, 0.5)
    # Batch sweep on the Llama-shaped head.
    for b in (16, 64, 256):
        for s in (0.2, 0.5, 1.0):
            n = f"sweep_b{b}_s{s}"
            reg[n] = Config(n, b, 4, 4096, 128256, 0.02, 1.0, s)
    # Sparse-q drafter: q nonzero only on the top-32 of 2048 random clusters.
    reg["sparse_q"] = Config("sparse_q", 8, 4, 1536, 262144, 0.02, 1.0, 0.5,
                             sparse=(2048, 128, 32))
    return reg


CONFIGS: Dict[str, Config] = _registry()


def streams(seed: int) -> Dict[str, np.random.Generator]:
    """One independent generator per tensor, spawned from ``SeedSequence(seed)``.

    The bulk Gaussian tensors use SFC64 for speed; the uniforms (and the
    cluster permutation) use Philox.
    """
    children = np.random.SeedSequence(seed).spawn(len(STREAMS))
    out = {}
    for n, c in zip(STREAMS, children):
        bitgen = np.random.Philox if n in ("uniforms", "clusters") else np.random.SFC64
        out[n] = np.random.Generator(bitgen(c))
    out["_W_seedseq"] = children[STREAMS.index("W")]
    return out


def _round_bf16_inplace(buf: np.ndarray, scratch: np.ndarray, out: np.ndarray) -> None:
    """Round fp32 ``buf`` to bf16 (nearest, ties to even) into uint16 ``out``.

    ``buf`` is overwritten; ``scratch`` is a uint32 array of the same shape.
    """
    u = buf.view(np.uint32)
    np.right_shift(u, np.uint32(16), out=scratch)
    scratch &= np.uint32(1)
    scratch += np.uint32(0x7FFF)
    u += scratch
    u >>= np.uint32(16)
    np.copyto(out, u, casting="unsafe")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bfloat16 (nearest, ties to even); return the uint16 bits.

    Inputs here are finite Gaussian draws, so NaN/Inf handling is not needed.
    """
    buf = np.array(x, dtype=np.float32, copy=True, order="C")
    out = np.empty(buf.shape, dtype=np.uint16)
    _round_bf16_inplace(buf, np.empty(buf.shape, dtype=np.uint32), out)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)).view(np.float32)


_tls = threading.local()


def _scratch(name: str, shape, dtype) -> np.ndarray:
    """Per-thread reusable buffer (fresh pages are slow to fault in)."""
    key = (name, np.dtype(dtype).str)
    store = getattr(_tls, "bufs", None)
    if store is None:
        store = _tls.bufs = {}
    n = int(np.prod(shape))
    buf = store.get(key)
    if buf is None or buf.size < n:
        buf = store[key] = np.empty(n, dtype=dtype)
    return buf[:n].reshape(shape)


def _pool_map(fn, items):
    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        return list(ex.map(fn, items))


def _gumbel_draw(rng: np.random.Generator, q_row: np.ndarray) -> int:
    """One draw from q_row by Gumbel-max: argmax_j log q_j + G_j."""
    u = rng.random(q_row.shape[0])  # [0, 1); u == 0 gives -inf and is never chosen
    with np.errstate(divide="ignore"):
        keys = np.log(q_row.astype(np.float64)) - np.log(-np.log(u))
    return int(np.argmax(keys))


def _softmax_f64(z: np.ndarray) -> np.ndarray:
    z = z.astype(np.float64)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def make_weights(cfg: Config, rs: Dict[str, np.random.Generator]) -> np.ndarray:
    """bf16 weights [V, d] ~ N(0, w_std^2), one SFC64 stream per 16384-row chunk."""
    n_chunks = -(-cfg.V // W_CHUNK_ROWS)
    seeds = rs["_W_seedseq"].spawn(n_chunks)
    W = np.empty((cfg.V, cfg.d), dtype=np.uint16)

    def work(ci):
        v0 = ci * W_CHUNK_ROWS
        v1 = min(cfg.V, v0 + W_CHUNK_ROWS)
        buf = _scratch("wf", (v1 - v0, cfg.d), np.float32)
        np.random.Generator(np.random.SFC64(seeds[ci])).standard_normal(out=buf, dtype=np.float32)
        buf *= np.float32(cfg.w_std)
        _round_bf16_inplace(buf, _scratch("wu", buf.shape, np.uint32), W[v0:v1])

    _pool_map(work, range(n_chunks))
    return W


def approx_target_logits(hidden_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
    """fp32 library matmul of the bf16 inputs, used only to shape q."""
    H = bf16_bits_to_f32(hidden_bits.reshape(-1, hidden_bits.shape[-1]))
    V, d = W_bits.shape
    out = np.empty((H.shape[0], V), dtype=np.float32)
    chunk = 4096

    def work(v0):
        v1 = min(V, v0 + chunk)
        wu = _scratch("au", (v1 - v0, d), np.uint32)
        np.copyto(wu, W_bits[v0:v1], casting="unsafe")
        wu <<= np.uint32(16)
        out[:, v0:v1] = H @ wu.view(np.float32).T

    _pool_map(work, range(0, V, chunk))
    return out


def generate(cfg: Config, W_bits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Build one batch of inputs for ``cfg``.

    Returns uint16 ``hidden_bits`` [B, gamma+1, d], uint16 ``W_bits`` [V, d],
    int32 ``draft`` [B, gamma], float32 ``q`` [B, gamma, V] and float32
    ``uniforms`` [B, gamma+1].  ``W_bits`` may be passed in to reuse a
    previously generated weight matrix of the same config and seed.
    """
    rs = streams(cfg.seed)
    B, g, d, V = cfg.B, cfg.gamma, cfg.d, cfg.V
    if W_bits is None:
        W_bits = make_weights(cfg, rs)
    assert W_bits.shape == (V, d) and W_bits.dtype == np.uint16
    hidden = f32_to_bf16_bits(
        rs["hidden"].standard_normal((B, g + 1, d), dtype=np.float32) * np.float32(cfg.h_std))

    # q is only needed at the gamma drafted positions of every sequence.
    lg = approx_target_logits(hidden[:, :g, :], W_bits).reshape(B, g, V)
    q = np.empty((B, g, V), dtype=np.float32)
    if cfg.sparse is None:
        for b in range(B):
            noise = rs["noise"].standard_normal((g, V), dtype=np.float32) * np.float32(cfg.sigma)
            q[b] = _softmax_f64(lg[b] + noise).astype(np.float32)
    else:
        n_clusters, size, top = cfg.sparse
        assert n_clusters * size == V
        members = rs["clusters"].permutation(V).reshape(n_clusters, size)
        centroids = np.empty((n_clusters, d), dtype=np.float32)
        for c in range(n_clusters):
            centroids[c] = bf16_bits_to_f32(W_bits[members[c]]).mean(axis=0)
        hf = bf16_bits_to_f32(hidden.reshape(-1, d)).reshape(B, g + 1, d)
        for b in range(B):
            noise = rs["noise"].standard_normal((g, V), dtype=np.float32) * np.float32(cfg.sigma)
            for i in range(g):
                score = centroids @ hf[b, i]
                chosen = np.argsort(-score, kind="stable")[:top]
                sel = np.sort(members[chosen].ravel())
                row = np.zeros(V, dtype=np.float32)
                row[sel] = _softmax_f64(lg[b, i, sel] + noise[i, sel]).astype(np.float32)
                q[b, i] = row

    draft = np.empty((B, g), dtype=np.int32)
    for b in range(B):
        for i in range(g):
            draft[b, i] = _gumbel_draw(rs["drafts"], q[b, i])
    uniforms = (np.float32(1.0) - rs["uniforms"].random((B, g + 1), dtype=np.float32)).astype(np.float32)
    return {"hidden_bits": hidden, "W_bits": W_bits, "draft": draft, "q": q, "uniforms": uniforms}


def custom(B: int, gamma: int, d: int, V: int, *, w_std: float = 0.5, h_std: float = 1.0,
           sigma: float = 0.7, seed: int = 0, sparse=None) -> Dict[str, np.ndarray]:
    """Inputs of an arbitrary (small) shape with the same recipe."""
    return generate(Config(f"custom_B{B}_g{gamma}_d{d}_V{V}", B, gamma, d, V, w_std, h_std,
                           sigma, sparse=sparse, seed=seed))


def repeated_trials(base: Dict[str, np.ndarray], n: int, seed: int, *,
                    row: int = 0) -> Dict[str, np.ndarray]:
    """``n`` independent trials of one sequence of ``base``.

    Every trial shares the hidden states, weights and q of sequence ``row``;
    the draft tokens (drawn from q) and the uniforms are fresh per trial.
    """
    rs = streams(seed)
    g = base["draft"].shape[1]
    hidden = np.repeat(base["hidden_bits"][row:row + 1], n, axis=0)
    q = np.repeat(base["q"][row:row + 1], n, axis=0)
    # Gumbel-max for all trials at once (small V only).
    V = q.shape[-1]
    u = rs["drafts"].random((n, g, V))
    with np.errstate(divide="ignore"):
        keys = np.log(q.astype(np.float64)) - np.log(-np.log(u))
    draft = np.argmax(keys, axis=-1).astype(np.int32)
    uniforms = (np.float32(1.0) - rs["uniforms"].random((n, g + 1), dtype=np.float32)).astype(np.float32)
    return {"hidden_bits": hidden, "W_bits": base["W_bits"], "draft": draft, "q": q,
            "uniforms": uniforms}


def iid_positions(V: int, d: int, gamma: int, n: int, seed: int, *, sigma: float = 1.0,
                  w_std: float = 0.25) -> Dict[str, np.ndarray]:
    """Trials in which every position is equally easy to guess.

    All gamma+1 hidden rows are the same vector and all gamma q rows are the
    same distribution, so every position has the same acceptance rate.
    """
    rs = streams(seed)
    W = f32_to_bf16_bits(rs["W"].standard_normal((V, d), dtype=np.float32) * np.float32(w_std))
    h = f32_to_bf16_bits(rs["hidden"].standard_normal((d,), dtype=np.float32))
    lg = approx_target_logits(h[None, :], W)[0]
    q1 = _softmax_f64(lg + rs["noise"].standard_normal(V, dtype=np.float32) * np.float32(sigma))
    q1 = q1.astype(np.float32)
    hidden = np.broadcast_to(h, (n, gamma + 1, d)).copy()
    q = np.broadcast_to(q1, (n, gamma, V)).copy()
    u = rs["drafts"].random((n, gamma, V))
    with np.errstate(divide="ignore"):
        keys = np.log(q.astype(np.float64)) - np.log(-np.log(u))
    draft = np.argmax(keys, axis=-1).astype(np.int32)
    uniforms = (np.float32(1.0) - rs["uniforms"].random((n, gamma + 1), dtype=np.float32)).astype(np.float32)
    return {"hidden_bits": hidden, "W_bits": W, "draft": draft, "q": q, "uniforms": uniforms}


# ---------------------------------------------------------------------------
# Sparse q and the clustered drafter head (inputs only).
# ---------------------------------------------------------------------------
def to_sparse_q(q: np.ndarray, *, pad: int = 0, dup: int = 0,
                shuffle_seed: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(ids, values) form of dense q rows [B, gamma, V] -> two [B, gamma, K] arrays.

    Every nonzero entry of a row is listed; ``dup`` entries per row repeat an
    id with half its value (the ABI keeps the larger value of a repeated id,
    so the row still means the same q); ``pad`` padding entries (id -1) fill
    every row to the same K.  With ``shuffle_seed`` each row's entries are put
    in a random order.  Pure data movement: no arithmetic on q besides the
    halving of the repeats.
    """
    B, g, V = q.shape
    nnz = (q != 0).sum(axis=-1)
    K = int(nnz.max()) + dup + pad
    ids = np.full((B, g, K), -1, dtype=np.int32)
    vals = np.zeros((B, g, K), dtype=np.float32)
    rng = np.random.default_rng(shuffle_seed) if shuffle_seed is not None else None
    for b in range(B):
        for i in range(g):
            nz = np.flatnonzero(q[b, i]).astype(np.int32)
            v = q[b, i, nz]
            if dup:
                pick = nz[:dup] if rng is None else rng.choice(nz, size=min(dup, nz.size), replace=False)
                nz = np.concatenate([nz, pick])
                v = np.concatenate([v, (q[b, i, pick] * np.float32(0.5)).astype(np.float32)])
            n = nz.size
            ids[b, i, :n] = nz
            vals[b, i, :n] = v
            if rng is not None:
                perm = rng.permutation(K)
                ids[b, i] = ids[b, i, perm]
                vals[b, i] = vals[b, i, perm]
    return ids, vals


def truncate_q(x: Dict[str, np.ndarray], K: int, seed: int) -> Dict[str, np.ndarray]:
    """Inputs whose q rows keep only their K largest entries (renormalised),
    with the drafts drawn again from the truncated rows (Gumbel-max)."""
    rs = streams(seed)
    q = x["q"].astype(np.float64)
    B, g, V = q.shape
    out = np.zeros_like(x["q"])
    draft = np.empty((B, g), dtype=np.int32)
    for b in range(B):
        for i in range(g):
            keep = np.argsort(-q[b, i], kind="stable")[:K]
            row = np.zeros(V)
            row[keep] = q[b, i, keep] / q[b, i, keep].sum()
            out[b, i] = row.astype(np.float32)
            draft[b, i] = _gumbel_draw(rs["drafts"], out[b, i])
    y = dict(x)
    y["q"] = out
    y["draft"] = draft
    return y


def clustered_head(N: int, d: int, V: int, C: int, M: int, *, w_std: float = 0.02,
                   seed: int = 0, W_bits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Inputs of the drafter's clustered head: N hidden rows, W [V, d], a
    members table [C, M] of disjoint clusters (the first C * M ids of a seeded
    random permutation of the vocabulary) and the cluster embeddings, each
    the mean of its members' rows (fp32) rounded to bf16."""
    rs = streams(seed)
    cfg = Config("clustered_head", 1, 1, d, V, w_std, 1.0, 0.0, seed=seed)
    if W_bits is None:
        W_bits = make_weights(cfg, rs)
    h = f32_to_bf16_bits(rs["hidden"].standard_normal((N, d), dtype=np.float32))
    assert C * M <= V, "clusters are disjoint: C * M tokens at most"
    members = rs["clusters"].permutation(V)[:C * M].reshape(C, M).astype(np.int32)
    cent = np.empty((C, d), dtype=np.float32)
    for c in range(C):
        cent[c] = bf16_bits_to_f32(W_bits[members[c]]).mean(axis=0)
    return {"h_bits": h, "W_bits": W_bits, "centroid_bits": f32_to_bf16_bits(cent),
            "members": members}


def drafter_chain(B: int, gamma: int, d: int, V: int, C: int, M: int, k: int, *,
                  w_std: float = 0.02, sigma_h: float = 0.5, seed: int = 0,
                  W_bits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Inputs of a drafter-then-verifier step with the clustered head.

    The target's hidden rows [B, gamma+1, d]; the drafter's hidden rows at the
    gamma drafted positions are the target's plus N(0, sigma_h^2) noise
    (rounded to bf16), [B*gamma, d].  Drafts are drawn (Gumbel-max) from an
    fp32 approximation of the drafter's sparse q -- top-k clusters by fp32
    scores, fp32 token logits -- which only shapes the input.
    """
    base = clustered_head(B * gamma, d, V, C, M, w_std=w_std, seed=seed, W_bits=W_bits)
    rs = streams(seed + 1)
    hidden = f32_to_bf16_bits(rs["hidden"].standard_normal((B, gamma + 1, d), dtype=np.float32))
    hf = bf16_bits_to_f32(hidden[:, :gamma].reshape(-1, d))
    hd = f32_to_bf16_bits(hf + rs["noise"].standard_normal(hf.shape, dtype=np.float32)
                          * np.float32(sigma_h))
    cent = bf16_bits_to_f32(base["centroid_bits"])
    hdf = bf16_bits_to_f32(hd)
    draft = np.empty((B, gamma), dtype=np.int32)
    for r in range(B * gamma):
        chosen = np.argsort(-(cent @ hdf[r]), kind="stable")[:k]
        sel = base["members"][chosen].ravel()
        sel = sel[(sel >= 0) & (sel < V)]
        lg = bf16_bits_to_f32(base["W_bits"][sel]) @ hdf[r]
        qa = np.zeros(V, dtype=np.float32)
        qa[sel] = _softmax_f64(lg).astype(np.float32)
        draft[r // gamma, r % gamma] = _gumbel_draw(rs["drafts"], qa)
    uniforms = (np.float32(1.0) - rs["uniforms"].random((B, gamma + 1), dtype=np.float32)).astype(np.float32)
    return {"hidden_bits": hidden, "W_bits": base["W_bits"], "h_draft_bits": hd,
            "centroid_bits": base["centroid_bits"], "members": base["members"], "draft": draft,
            "uniforms": uniforms}


# ---------------------------------------------------------------------------
# Draft trees (inputs only).
# ---------------------------------------------------------------------------
def tree_rows_with_children(parent) -> np.ndarray:
    """Rows (0 = root, t+1 = node t) that have children, in row order."""
    has = np.zeros(len(parent) + 1, dtype=bool)
    for a in parent:
        has[int(a) + 1] = True
    return np.flatnonzero(has)


def tree_inputs(B: int, parent, d: int, V: int, *, w_std: float = 0.5, sigma: float = 0.7,
                seed: int = 0, W_bits: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Inputs of tree verification with the recipe of ``generate``.

    hidden [B, T+1, d] (row 0 the root, row t+1 node t); q [B, P, V] at the
    rows with children, softmax of fp32 approximate logits plus N(0, sigma^2);
    every node's token drawn (Gumbel-max) from q at its parent's row, siblings
    independently; uniforms [B, T+1] = 1 - U.
    """
    T = len(parent)
    cfg = Config(f"tree_B{B}_T{T}_d{d}_V{V}", B, T, d, V, w_std, 1.0, sigma, seed=seed)
    rs = streams(seed)
    if W_bits is None:
        W_bits = make_weights(cfg, rs)
    hidden = f32_to_bf16_bits(rs["hidden"].standard_normal((B, T + 1, d), dtype=np.float32))
    rows = tree_rows_with_children(parent)
    slot = {int(r): i for i, r in enumerate(rows)}
    lg = approx_target_logits(hidden[:, rows, :], W_bits).reshape(B, rows.size, V)
    q = np.empty((B, rows.size, V), dtype=np.float32)
    for b in range(B):
        noise = rs["noise"].standard_normal((rows.size, V), dtype=np.float32) * np.float32(sigma)
        q[b] = _softmax_f64(lg[b] + noise).astype(np.float32)
    tokens = np.empty((B, T), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            tokens[b, t] = _gumbel_draw(rs["drafts"], q[b, slot[int(parent[t]) + 1]])
    uniforms = (np.float32(1.0) - rs["uniforms"].random((B, T + 1), dtype=np.float32)).astype(np.float32)
    return {"hidden_bits": hidden, "W_bits": W_bits, "parent": np.asarray(parent, dtype=np.int32),
            "tokens": tokens, "q": q, "uniforms": uniforms}


def tree_repeated_trials(base: Dict[str, np.ndarray], n: int, seed: int) -> Dict[str, np.ndarray]:
    """``n`` trials of sequence 0 of ``base``: hidden states, weights and q
    shared; every node's token (from q at its parent's row) and the uniforms
    fresh per trial.  Small V only."""
    rs = streams(seed)
    parent = base["parent"]
    T = len(parent)
    rows = tree_rows_with_children(parent)
    slot = {int(r): i for i, r in enumerate(rows)}
    q = np.repeat(base["q"][:1], n, axis=0)
    V = q.shape[-1]
    tokens = np.empty((n, T), dtype=np.int32)
    with np.errstate(divide="ignore"):
        for t in range(T):
            lq = np.log(base["q"][0, slot[int(parent[t]) + 1]].astype(np.float64))
            u = rs["drafts"].random((n, V))
            tokens[:, t] = np.argmax(lq[None, :] - np.log(-np.log(u)), axis=-1)
    uniforms = (np.float32(1.0) - rs["uniforms"].random((n, T + 1), dtype=np.float32)).astype(np.float32)
    return {"hidden_bits": np.repeat(base["hidden_bits"][:1], n, axis=0), "W_bits": base["W_bits"],
            "parent": parent, "tokens": tokens, "q": q, "uniforms": uniforms}


# A static tree of 25 nodes in the shape EAGLE-style drafters use: wide near
# the root, narrowing with depth (4 root candidates; their children 3, 2, 1, 1;
# and so on to depth 5).
EAGLE_LIKE_TREE = [-1, -1, -1, -1,          # depth 1: nodes 0-3
                   0, 0, 0, 1, 1, 2, 3,     # depth 2: nodes 4-10
                   4, 4, 5, 7, 9, 10,       # depth 3: nodes 11-16
                   11, 11, 13, 14, 16,      # depth 4: nodes 17-21
                   17, 19, 21]              # depth 5: nodes 22-24
