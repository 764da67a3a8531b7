// Tree verification: several drafted candidates per position, checked with
// the same keep-or-replace rule at every fork.
//
// Source: "推测解码" (world.lapla.si/zh/specdec): section 通过的规则 (keep x
// with probability min(1, p/q), else replace it from max(0, p - q)
// renormalised), section 留下对的，换掉错的 (stop at the first rejection; a
// bonus token after the last kept one), and the section on later methods,
// where EAGLE applies that rule at every fork of its guess tree and the
// distribution is unchanged.  The procedure at a fork: the children of the
// current node are tested in increasing node index, the first against p of
// the node's row and each later one against the renormalised residual the
// previous rejection left; a kept child is emitted and the walk moves to its
// row; when every child is rejected the token is drawn from the last
// residual, and at a node without children the bonus token from p.
//
// The residual after j rejected siblings has a closed form: with c_0 = 0,
// S_0 = 1, c_{j+1} = c_j + S_j and S_j = sum_v max(0, p_v - c_j q_v),
// it is max(0, p - c_j q) / S_j.  So each test needs only p(x), q(x) and
// the scalars c_j, S_j, and each rejection costs one sum over the row --
// the same per-chunk pass (with weight max(0, p - c q)) as the chain draw.
//
// Kernels, on the caller's stream after the LM head:
//   tree_init_kernel   one workgroup per sequence: the row normalisers of the
//                      sequence's T+1 rows, output padding, and the walk
//                      from the root as far as it goes without a sum.
//   then a fixed number of rounds (the most sums any walk of the topology
//   can need, plus the draw), each
//   tree_sums_kernel   one workgroup per (sequence, 4096-token chunk): fp64
//                      chunk totals of max(0, p - c q) and of p at the
//                      sequence's current row (nothing for finished ones);
//   tree_decide_kernel one workgroup per sequence: S from the totals, then
//                      either the pending sibling test and the walk onwards,
//                      or the inverse-CDF pick that ends the sequence;
//   or, with at most 64 chunk workgroups in all, tree_round_kernel: both in
//   one launch, the sequence's last chunk workgroup deciding.
// The state of each walk lives in the workspace between launches.

#include "draw_common.h"

namespace sv {

namespace {

enum : int32_t { kPhaseSum = 0, kPhaseDrawRes = 1, kPhaseDrawP = 2, kPhaseDone = 3 };

struct TreeState {
    double c;          // residual coefficient for the pending test or the draw
    int32_t row;       // row of the current node (0 = root, t + 1 = node t)
    int32_t kid;       // node whose test is pending
    int32_t j;         // its rank among its siblings
    int32_t phase;
    int32_t depth;     // kept nodes so far
    int32_t flags;     // SV_DEV_* bits
};

static_assert(sizeof(TreeState) == kTreeStateBytes, "workspace layout of the walk state");

struct TreeArgs {
    const float* logits;
    const float* row_max;
    const float* row_sum;
    const int32_t* tokens;     // [B][T]
    const float* q;            // [B][P][V]
    const float* uniforms;     // [B][T+1]
    int V;
    int32_t* out_tokens;       // [B][D+1]
    int32_t* path_nodes;       // [B][D] or null
    int8_t parent_row[SV_MAX_TREE_NODES];   // per node: its parent's row (0 = root)
};

__device__ __forceinline__ size_t grow(int b, const TreeTopo& tp, int row) {
    return (size_t)b * (tp.T + 1) + row;
}

// What the walk reads at node t: its token x, its uniform r, and p and q of x
// at its parent's row.  One wave gathers them for every node at once, lane t
// taking node t (at most 64 nodes), so that the walk -- one thread -- reads
// LDS instead of making two dependent trips to memory per node.  In two
// parts: node_keys issues the loads that need only the topology (token,
// uniform, the parent row's normaliser), node_table the gathers at the token.
struct NodeVal {
    float px, qx, r;
    int x;
};

struct NodeKeys {
    int x, prow;
    float r, m, s;
};

__device__ __forceinline__ NodeKeys node_keys(const TreeTopo& tp, int b, const TreeArgs& a,
                                              const float* rmax, const float* rsum) {
    const int lane = threadIdx.x & (kWave - 1);
    NodeKeys k{-1, 0, 0.f, 0.f, 0.f};
    if (lane < tp.T) {
        k.prow = a.parent_row[lane];
        k.x = a.tokens[(size_t)b * tp.T + lane];
        k.r = a.uniforms[(size_t)b * (tp.T + 1) + lane];
        k.m = rmax[k.prow];
        k.s = rsum[k.prow];
    }
    return k;
}

__device__ __forceinline__ void node_table(const NodeKeys& k, const TreeTopo& tp, int b,
                                           const TreeArgs& a, NodeVal* s_node) {
    const int lane = threadIdx.x & (kWave - 1);
    if (lane >= tp.T) return;
    NodeVal v{0.f, 0.f, k.r, k.x};
    if (k.x >= 0 && k.x < a.V) {
        const float lx = a.logits[grow(b, tp, k.prow) * a.V + k.x];
        v.qx = a.q[((size_t)b * tp.P + tp.qslot[k.prow]) * a.V + k.x];
        v.px = target_prob(lx, k.m, k.s);
    }
    s_node[lane] = v;
}

// Runs the walk of sequence b from its state until it needs a sum (or a
// draw).  S is the sum for a pending test of rank j >= 1.  One thread, after
// its wave has filled s_node (node_keys, node_table).
__device__ void tree_advance(TreeState& st, double S, const TreeTopo& tp, int b, const TreeArgs& a,
                             const NodeVal* s_node) {
    for (;;) {
        const int t = st.kid;
        const NodeVal nv = s_node[t];          // node t's values at its parent, st.row
        const int x = nv.x;
        const float r = nv.r;
        bool keep = false;
        if (x >= 0 && x < a.V) {
            const float px = nv.px;
            const float qx = nv.qx;
            if (st.j == 0) {
                keep = r * qx <= px;
            } else {
                // the residual's weight at x, as the chunk pass computes it
                const float wx = fmaxf(0.f, px - (float)st.c * qx);
                keep = (double)r * (double)qx * S <= (double)wx;
            }
        } else {
            st.flags |= SV_DEV_BAD_DRAFT;             // rejected with p = 0
        }
        if (keep) {
            a.out_tokens[(size_t)b * (tp.D + 1) + st.depth] = x;
            if (a.path_nodes) a.path_nodes[(size_t)b * tp.D + st.depth] = t;
            ++st.depth;
            st.row = t + 1;
            const int fc = tp.first_child[st.row];
            if (fc < 0) { st.phase = kPhaseDrawP; return; }     // a leaf: the bonus from p
            st.kid = fc;
            st.j = 0;
            st.c = 0.0;
            continue;
        }
        st.c += st.j == 0 ? 1.0 : S;                   // c_{j+1} = c_j + S_j, S_0 = 1
        const int nk = tp.next_sibling[t];
        if (nk < 0) { st.phase = kPhaseDrawRes; return; }       // every child rejected
        st.kid = nk;
        ++st.j;
        st.phase = kPhaseSum;
        return;
    }
}

__device__ __forceinline__ DrawRow tree_draw_row(const TreeState& st, const TreeTopo& tp, int b,
                                                 const TreeArgs& a) {
    DrawRow d;
    const size_t gr = grow(b, tp, st.row);
    d.lrow = a.logits + gr * a.V;
    d.qrow = st.phase == kPhaseDrawP ? nullptr
                                     : a.q + ((size_t)b * tp.P + tp.qslot[st.row]) * a.V;
    d.qids = nullptr;
    d.qvals = nullptr;
    d.K = 0;
    d.M = a.row_max[gr];
    d.S = a.row_sum[gr];
    d.c = (float)st.c;
    d.V = a.V;
    return d;
}

__global__ __launch_bounds__(kDrawBlock) void tree_init_kernel(
    const float* __restrict__ part_max, const float* __restrict__ part_sum, int NP, int NPs,
    TreeTopo tp, TreeArgs a, float* __restrict__ row_max, float* __restrict__ row_sum,
    TreeState* __restrict__ state, int32_t* __restrict__ n_accepted,
    int32_t* __restrict__ status) {
    __shared__ float r_m[SV_MAX_TREE_NODES + 1], r_s[SV_MAX_TREE_NODES + 1];
    const int b = blockIdx.x;
    const int T1 = tp.T + 1;
    merge_row_partials(part_max, part_sum, NP, NPs, (size_t)b * T1, T1, r_m, r_s);
    for (int i = threadIdx.x; i <= tp.D; i += kDrawBlock) {
        a.out_tokens[(size_t)b * (tp.D + 1) + i] = -1;
        if (a.path_nodes && i < tp.D) a.path_nodes[(size_t)b * tp.D + i] = -1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T1; i += kDrawBlock) {
        row_max[(size_t)b * T1 + i] = r_m[i];
        row_sum[(size_t)b * T1 + i] = r_s[i];
    }
    if (threadIdx.x >= kWave) return;
    __shared__ NodeVal s_node[SV_MAX_TREE_NODES];
    node_table(node_keys(tp, b, a, r_m, r_s), tp, b, a, s_node);
    // lane 0 reads the entries the other lanes of its wave just wrote
    __builtin_amdgcn_wave_barrier();
    if (threadIdx.x == 0) {
        TreeState st;
        st.c = 0.0;
        st.row = 0;
        st.kid = tp.first_child[0];
        st.j = 0;
        st.depth = 0;
        st.flags = 0;
        tree_advance(st, 1.0, tp, b, a, s_node);
        state[b] = st;
        n_accepted[b] = st.depth;
        status[b] = st.flags;
    }
}

// Chunk c's totals of the weights at the sequence's current row:
// max(0, p - c q) (the residual of a pending test, or the draw's), or p for a
// bonus draw, per wave and over the workgroup.  Every thread takes part.
__device__ void tree_chunk_totals(const TreeState& st, const TreeTopo& tp, int b, int c, int NC,
                                  const TreeArgs& a, const ChunkSums& cs) {
    const DrawRow d = tree_draw_row(st, tp, b, a);
    const int c0 = c * kDrawChunk;
    float w[kDrawPerThread], p[kDrawPerThread];
    draw_weights<false>(d, c0 + threadIdx.x * kDrawPerThread, nullptr, c0, w, p);
    double tw = 0.0, tp_ = 0.0;
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) { tw += (double)w[e]; tp_ += (double)p[e]; }
    store_chunk_totals(tw, tp_, cs, (size_t)b * NC + c);
}

// With every chunk total of the round in place: the sum S, then either the
// pending sibling test and the walk onwards (state updated for the next
// round), or the inverse-CDF pick that ends the sequence.  One whole wave
// (the pick is a wave operation; lane 0 updates the state).
__device__ void tree_decide(TreeState st, const TreeTopo& tp, int b, const TreeArgs& a, int NC,
                            const ChunkSums& cs, TreeState* __restrict__ state,
                            int32_t* __restrict__ n_accepted, int32_t* __restrict__ status) {
    const int lane = threadIdx.x & (kWave - 1);
    const DrawRow d = tree_draw_row(st, tp, b, a);
    __shared__ NodeVal s_node[SV_MAX_TREE_NODES];
    const size_t g0 = grow(b, tp, 0);
    const NodeKeys keys = node_keys(tp, b, a, a.row_max + g0, a.row_sum + g0);
    // S in the association the pick uses; every lane has it, so every lane
    // takes the same branch.
    const double S = chunk_total_sum(cs.csum + (size_t)b * NC, NC);
    bool draw = st.phase != kPhaseSum;
    if (!draw && !(S > 0.0 && S < INFINITY)) draw = true;   // no residual mass: the pick falls back to p
    if (!draw) {
        node_table(keys, tp, b, a, s_node);
        __builtin_amdgcn_wave_barrier();       // lane 0 reads the other lanes' entries
        if (lane == 0) {
            tree_advance(st, S, tp, b, a, s_node);
            state[b] = st;
            n_accepted[b] = st.depth;
            status[b] = st.flags;
        }
        return;
    }
    int pflags;
    const int tok = pick<false>(d, b, NC, cs, a.uniforms[(size_t)b * (tp.T + 1) + tp.T], nullptr,
                                &pflags);
    if (lane == 0) {
        a.out_tokens[(size_t)b * (tp.D + 1) + st.depth] = tok;
        n_accepted[b] = st.depth;
        status[b] = st.flags | pflags;
        st.phase = kPhaseDone;
        state[b] = st;
    }
}

// Split round, many sequences: chunk totals here, tree_decide_kernel next
// (the kernel boundary orders the totals before the decision).
__global__ __launch_bounds__(kDrawBlock) void tree_sums_kernel(
    TreeTopo tp, TreeArgs a, const TreeState* __restrict__ state, int NC, ChunkSums cs) {
    const int c = (int)(blockIdx.x % (unsigned)NC), b = (int)(blockIdx.x / (unsigned)NC);
    const TreeState st = state[b];
    if (st.phase == kPhaseDone) return;
    tree_chunk_totals(st, tp, b, c, NC, a, cs);
}

// One wave per sequence.
__global__ __launch_bounds__(kWave) void tree_decide_kernel(
    TreeTopo tp, TreeArgs a, TreeState* __restrict__ state, int NC, ChunkSums cs,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ status) {
    const int b = blockIdx.x;
    const TreeState st = state[b];
    if (st.phase == kPhaseDone) return;
    tree_decide(st, tp, b, a, NC, cs, state, n_accepted, status);
}

// Fused round, few sequences: the sequence's last chunk workgroup to finish
// (a per-sequence counter that the LM-head launch zeroes and this kernel
// resets) decides -- one launch per round.
__global__ __launch_bounds__(kDrawBlock) void tree_round_kernel(
    TreeTopo tp, TreeArgs a, TreeState* __restrict__ state, int NC, ChunkSums cs,
    int32_t* __restrict__ counters, int32_t* __restrict__ n_accepted,
    int32_t* __restrict__ status) {
    const int c = (int)(blockIdx.x % (unsigned)NC), b = (int)(blockIdx.x / (unsigned)NC);
    const TreeState st = state[b];
    if (st.phase == kPhaseDone) return;
    tree_chunk_totals(st, tp, b, c, NC, a, cs);
    if (!arrive_last(&counters[(size_t)b * kCounterStride], NC)) return;
    if (threadIdx.x >= kWave) return;          // the decision is one wave's
    if (threadIdx.x == 0) counters[(size_t)b * kCounterStride] = 0;   // ready for the next round
    tree_decide(st, tp, b, a, NC, cs, state, n_accepted, status);
}

}  // namespace

// One fused launch per round up to 64 chunk workgroups (moving the threshold
// to 256 or 1024 changed nothing measurable), two above.
constexpr int kTreeFuseMaxGroups = 64;

hipError_t launch_tree(const float* logits, const float* part_max, const float* part_sum, int NP,
                       int NPs, int B, int V, const TreeTopo& tp, int rounds,
                       const int32_t* tokens, const float* q, const float* uniforms, int NC,
                       const ChunkSums& cs, float* row_max, float* row_sum, void* state,
                       int32_t* counters, int32_t* out_tokens, int32_t* n_accepted,
                       int32_t* path_nodes, int32_t* status, hipStream_t stream) {
    TreeArgs a{logits, row_max, row_sum, tokens, q, uniforms, V, out_tokens, path_nodes, {}};
    for (int row = 0; row <= tp.T; ++row)
        for (int k = tp.first_child[row]; k >= 0; k = tp.next_sibling[k]) a.parent_row[k] = (int8_t)row;
    TreeState* st = static_cast<TreeState*>(state);
    tree_init_kernel<<<dim3(B), dim3(kDrawBlock), 0, stream>>>(part_max, part_sum, NP, NPs, tp, a,
                                                          row_max, row_sum, st, n_accepted,
                                                          status);
    hipError_t e = hipGetLastError();
    const unsigned groups = (unsigned)B * NC;
    // Few chunk workgroups: one fused launch per round (see draw_kernel for
    // why many sequences use the split form instead).
    const bool fused = groups <= kTreeFuseMaxGroups;
    for (int r = 0; r < rounds && e == hipSuccess; ++r) {
        if (fused) {
            tree_round_kernel<<<dim3(groups), dim3(kDrawBlock), 0, stream>>>(
                tp, a, st, NC, cs, counters, n_accepted, status);
            e = hipGetLastError();
            continue;
        }
        tree_sums_kernel<<<dim3(groups), dim3(kDrawBlock), 0, stream>>>(tp, a, st, NC, cs);
        e = hipGetLastError();
        if (e != hipSuccess) break;
        tree_decide_kernel<<<dim3(B), dim3(kWave), 0, stream>>>(tp, a, st, NC, cs, n_accepted,
                                                                status);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace sv
