// Shared definitions of the verification-step kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <climits>
#include <stddef.h>
#include <stdint.h>

#include "specverify.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16 bytes = 8 bf16

constexpr int kWave = 64;
constexpr int kBlock = 256;              // threads per greedy and drafter-head workgroup

constexpr int kLmTile = 16;              // vocab rows (and hidden rows) per MFMA fragment
constexpr int kLmWaves = 4;              // waves per LM-head workgroup
constexpr int kLmMaxPartials = 1024;     // LM-head workgroups (softmax partials per row), at most
constexpr int kLmRowsPerPass = 64;       // hidden rows one LM-head launch handles
// Draw and tree kernels: 1024 threads (four waves per SIMD, so that one
// wave's dependent arithmetic hides behind the others') over 4096-token
// chunks, four tokens per thread.
constexpr int kDrawBlock = 1024;
constexpr int kDrawChunk = 4096;                                                // tokens per chunk
constexpr int kDrawPerThread = kDrawChunk / kDrawBlock;
constexpr int kDrawWaves = kDrawBlock / kWave;
// Each sequence's arrival counter sits on a 128-byte line of its own: the
// counters take one device-scope atomic per draw workgroup, and atomics on
// one line serialise (512 workgroups over 8 sequences sharing a line spent
// ~7 us there).
constexpr int kCounterStride = 32;
static_assert(kDrawPerThread % 4 == 0, "whole 16-byte runs of tokens per thread");

// LM-head workgroups worth launching for a vocabulary of V: at least one
// 16-row fragment per wave.
static inline int lmhead_useful_groups(int V) {
    const int ntiles = (V + kLmTile - 1) / kLmTile;
    const int g = (ntiles + kLmWaves - 1) / kLmWaves;
    return g < kLmMaxPartials ? g : kLmMaxPartials;
}

// Many-row LM-head path (an LDS-tiled MFMA GEMM, 256 x 256 blocks): used for
// R > 64 as long as its per-block softmax partials fit the bound.
constexpr int kLmTiledVocab = 256;
static inline int lmhead_tiled_partials(int V) { return (V + kLmTiledVocab - 1) / kLmTiledVocab; }
static inline bool lmhead_use_tiled(int R, int V) {
    return R > kLmRowsPerPass && lmhead_tiled_partials(V) <= kLmMaxPartials;
}

// Byte offsets of every array inside the caller's workspace.  The partial
// arrays have a row stride NPs (a multiple of 4, for 16-byte loads) that
// bounds the LM-head grid on any device.
struct Layout {
    int R, NPs, NC;
    size_t logits, part_max, part_sum, part_arg, row_max, row_sum, status, counters, csum, psum,
        cwave, pwave, tstate, htile, total;
};

// Bytes of a [N][d] bf16 matrix in 1 KB tiles of 16 rows x 32 columns (rows
// and columns padded with zeros to whole tiles).
__host__ __device__ inline size_t tiled_bytes(int N, int d) {
    return (size_t)((N + 15) / 16) * (size_t)((d + 31) / 32) * 1024;
}

// The draw's chunk totals, fp64: per (sequence, chunk) the sums of the draw
// weights (csum [B][NC]) and of p (psum), and the same per wave of the
// chunk's workgroup (cwave, pwave [B][NC][kDrawWaves]).
struct ChunkSums {
    double* csum;
    double* psum;
    double* cwave;
    double* pwave;
};

constexpr size_t kTreeStateBytes = 32;   // per-sequence walk state of tree verification

static inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static inline Layout make_layout(int B, int gamma, int d, int V) {
    Layout L;
    L.R = B * (gamma + 1);
    const int np_tiled = lmhead_tiled_partials(V);
    const int np = lmhead_use_tiled(L.R, V) && np_tiled > lmhead_useful_groups(V)
                       ? np_tiled : lmhead_useful_groups(V);
    L.NPs = (np + 3) / 4 * 4;
    L.NC = (V + kDrawChunk - 1) / kDrawChunk;
    size_t off = 0;
    L.logits = off;   off = align_up(off + (size_t)L.R * V * sizeof(float), 256);
    L.part_max = off; off = align_up(off + (size_t)L.R * L.NPs * sizeof(float), 256);
    L.part_sum = off; off = align_up(off + (size_t)L.R * L.NPs * sizeof(float), 256);
    L.part_arg = off; off = align_up(off + (size_t)L.R * L.NPs * sizeof(int32_t), 256);
    L.row_max = off;  off = align_up(off + (size_t)L.R * sizeof(float), 256);
    L.row_sum = off;  off = align_up(off + (size_t)L.R * sizeof(float), 256);
    L.status = off;   off = align_up(off + (size_t)B * sizeof(int32_t), 256);
    L.counters = off; off = align_up(off + (size_t)B * kCounterStride * sizeof(int32_t), 256);
    L.csum = off;     off = align_up(off + (size_t)B * L.NC * sizeof(double), 256);
    L.psum = off;     off = align_up(off + (size_t)B * L.NC * sizeof(double), 256);
    L.cwave = off;    off = align_up(off + (size_t)B * L.NC * kDrawWaves * sizeof(double), 256);
    L.pwave = off;    off = align_up(off + (size_t)B * L.NC * kDrawWaves * sizeof(double), 256);
    L.tstate = off;   off = align_up(off + (size_t)B * kTreeStateBytes, 256);
    // the hidden rows in tiles, for the many-row GEMM (written by stage 1)
    L.htile = off;    off = align_up(off + (lmhead_use_tiled(L.R, V) ? tiled_bytes(L.R, d) : 0), 256);
    L.total = off;
    return L;
}

// Byte offsets inside the workspace of the drafter's sparse head
// (make_head_layout, in sparse_head.hip).
struct HeadLayout {
    int G;                    // gather workgroups (softmax partials) per row
    size_t scores, tl, pmax, psum, total;
};
HeadLayout make_head_layout(int N, int C, int K);

// Static topology of a draft tree, passed to the tree kernels by value.
// Rows: 0 for the root, t + 1 for node t.
struct TreeTopo {
    int T;                                       // nodes
    int D;                                       // deepest node's depth
    int P;                                       // rows with children (q rows)
    int8_t first_child[SV_MAX_TREE_NODES + 1];   // per row: first child node, -1 for none
    int8_t next_sibling[SV_MAX_TREE_NODES];      // per node: next child of its parent, -1
    int8_t qslot[SV_MAX_TREE_NODES + 1];         // per row: its q row, -1 without children
};

// exp(x) for x <= 0 (or -inf) through the hardware exp2.
__device__ __forceinline__ float exp2_scaled(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// Merge of two (max, sum of exp(x - max)) pairs: the online-softmax step.
// Symmetric in its two arguments, so a butterfly gives every lane the same bits.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
    if (m2 == -INFINITY) return;
    if (m == -INFINITY) { m = m2; s = s2; return; }
    if (m2 > m) { s = s * expf(m - m2) + s2; m = m2; }
    else        { s = s + s2 * expf(m2 - m); }
}

// Merge of two (value, token id) candidates for a row's greedy token: the
// larger value wins, equal values go to the lower id, id -1 (no candidate)
// loses.  A total order on the candidates, so any merge order and any
// butterfly give the same answer on every lane.  Values are never NaN here:
// candidates are only taken by a strict '>' against -inf or a previous value.
__device__ __forceinline__ void arg_merge(float& v, int& i, float v2, int i2) {
    if (i2 < 0) return;
    if (i < 0 || v2 > v || (v2 == v && i2 < i)) { v = v2; i = i2; }
}

}  // namespace sv
