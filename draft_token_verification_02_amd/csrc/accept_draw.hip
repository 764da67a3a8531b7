// Accept test, first rejection and the replacement / bonus draw.
//
// Source: "推测解码" (world.lapla.si/zh/specdec):
//   section 通过的规则 -- keep a drafted token outright when q <= p, else with
//     probability p/q against a uniform r; on rejection the replacement comes
//     from max(0, p - q) renormalised;
//   section 留下对的，换掉错的 -- stop at the first rejection and discard the
//     later drafts; when every draft passes, emit the target's own token at
//     the extra position, which the same weight read already scored.
//
// After the LM head, one 1024-thread workgroup per (sequence b, 4096-token
// chunk c) of draw_kernel, four tokens per thread.  For sequence b they
//   1. gather l[x_i], q[x_i] and r_i of the gamma drafts and, meanwhile,
//      merge each of the sequence's gamma+1 rows' LM-head partials (one
//      wave per row) into the row's softmax normaliser;
//   2. run the gamma accept tests r * q <= p and take n, the number of
//      leading accepts, from a wave ballot;
//   3. compute fp64 totals of the chunk's draw weights -- the residual
//      max(0, p - q) at row n, or p at row gamma for the bonus -- and of p.
// Then one wave scans the chunk totals, finds the chunk where the running sum
// reaches u * S, then the wave of that chunk from its wave totals, rescans
// that wave's tokens with the same code and picks the first token that
// reaches it: an inverse CDF over ascending ids.
//
// Three forms, by the number of draw workgroups.  Few: every chunk
// workgroup runs steps 1-2 itself (they read (gamma+1) * NP * 8 bytes,
// little next to the chunk) and the sequence's last workgroup to finish (a
// per-sequence counter that the LM-head launch zeroes) picks: one launch.
// More: the same, but pick_kernel picks (two launches).  Many: accept_kernel
// runs steps 1-2 once per sequence, the chunk workgroups (four chunks each
// with dense q) read n and the draw row's normaliser from memory, and
// pick_kernel follows (three launches).
//
// q comes in one of two forms.  Dense: a full [V] row per drafted position.
// Sparse: K (id, value) entries per row -- the drafter's clustered head
// ("多詞元預測視覺化指南", section 高效嵌入器) gives q only on the tokens of its
// chosen clusters and exactly 0 elsewhere.  With sparse q a drafted token's
// q is found by one wave scanning the row's ids, and a draw workgroup builds
// its chunk of the dense row in LDS (zeroed, then the row's entries that fall
// in the chunk scattered in), so the draw arithmetic is the same in both.

#include "draw_common.h"

namespace sv {

namespace {

// ---------------------------------------------------------------------------
// Steps 1-2: softmax normalisers of the sequence's rows (into r_m, r_s) and
// the accept tests.  Returns n; *flags gets SV_DEV_BAD_DRAFT when a draft id
// was out of range and SV_DEV_BAD_QID when a sparse q row lists an id >= V.
template <bool SPARSE>
__device__ int accept_tests(const float* __restrict__ logits, const float* __restrict__ part_max,
                            const float* __restrict__ part_sum, int NP, int NPs, int b, int gamma,
                            int V, const int32_t* __restrict__ draft, QArg q,
                            const float* __restrict__ uniforms, float* r_m, float* r_s, int* flags) {
    __shared__ int s_n, s_flags;
    __shared__ unsigned s_qx[SPARSE ? SV_MAX_GAMMA : 1];
    __shared__ int s_x[SPARSE ? SV_MAX_GAMMA : 1];
    __shared__ int s_badq;
    const int g1 = gamma + 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // Draft gathers, issued before the partial loads they do not depend on.
    float lx = 0.f, qx = 0.f, ux = 1.f;
    bool valid = false;
    if (wave == 0 && lane < gamma) {
        const int x = draft[(size_t)b * gamma + lane];
        valid = x >= 0 && x < V;
        ux = uniforms[(size_t)b * g1 + lane];
        if (valid) {
            lx = logits[((size_t)b * g1 + lane) * V + x];
            if (!SPARSE) qx = q.val[((size_t)b * gamma + lane) * V + x];
        }
    }
    if (SPARSE) {
        // Every drafted position's token is looked up in its q row by the
        // whole workgroup at once: the gamma rows' K ids are one flat range,
        // 8 loads in flight per thread, and a match merges its value into
        // s_qx by unsigned max on the (non-negative) value's bits.
        if (threadIdx.x < SV_MAX_GAMMA) {
            s_qx[threadIdx.x] = 0u;
            s_x[threadIdx.x] = threadIdx.x < gamma ? draft[(size_t)b * gamma + threadIdx.x] : -1;
        }
        if (threadIdx.x == 0) s_badq = 0;
        __syncthreads();
        const int32_t* ids = q.idx + (size_t)b * gamma * q.K;
        const float* vals = q.val + (size_t)b * gamma * q.K;
        bool badq = false;
        if ((q.K & 3) == 0) {
            const int K4 = q.K >> 2;
            const int total = gamma * K4;
            const int4* id4 = reinterpret_cast<const int4*>(ids);
            for (int e0 = 0; e0 < total; e0 += kDrawBlock * 8) {
                int4 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + threadIdx.x + u * kDrawBlock;
                    v[u] = e < total ? id4[e] : make_int4(-1, -1, -1, -1);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int e = e0 + threadIdx.x + u * kDrawBlock;
                    if (e >= total) continue;
                    const int i = e / K4;
                    const int x = s_x[i];
                    const int id[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        badq |= id[c] >= V;
                        if (id[c] == x)
                            atomicMax(&s_qx[i], __float_as_uint(sparse_value(vals[(size_t)e * 4 + c])));
                    }
                }
            }
        } else {
            const int total = gamma * q.K;
            for (int e = threadIdx.x; e < total; e += kDrawBlock) {
                const int id = ids[e];
                const int i = e / q.K;
                badq |= id >= V;
                if (id == s_x[i]) atomicMax(&s_qx[i], __float_as_uint(sparse_value(vals[e])));
            }
        }
        if (badq) atomicOr(&s_badq, 1);
    }
    merge_row_partials(part_max, part_sum, NP, NPs, (size_t)b * g1, g1, r_m, r_s);
    __syncthreads();

    if (wave == 0) {
        if (SPARSE && lane < gamma) qx = __uint_as_float(s_qx[lane]);
        bool keep = false;
        if (lane < gamma && valid) keep = ux * qx <= target_prob(lx, r_m[lane], r_s[lane]);
        const unsigned long long kept = __ballot(keep);
        const unsigned long long badm = __ballot(lane < gamma && !valid);
        if (lane == 0) {
            s_n = min(__builtin_ctzll(~kept), gamma);
            int f = badm != 0 ? SV_DEV_BAD_DRAFT : 0;
            if (SPARSE && s_badq) f |= SV_DEV_BAD_QID;
            s_flags = f;
        }
    }
    __syncthreads();
    *flags = s_flags;
    return s_n;
}

// Accept tests once per sequence (the split form, for many sequences):
// n, the row normalisers, the kept drafts, padding and status.
template <bool SPARSE>
__global__ __launch_bounds__(kDrawBlock) void accept_kernel(
    const float* __restrict__ logits, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, int NP, int NPs, const int32_t* __restrict__ draft,
    QArg q, const float* __restrict__ uniforms, int gamma, int V,
    float* __restrict__ row_max, float* __restrict__ row_sum, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ status) {
    __shared__ float r_m[SV_MAX_GAMMA + 1], r_s[SV_MAX_GAMMA + 1];
    const int b = blockIdx.x;
    const int g1 = gamma + 1;
    int flags;
    const int n = accept_tests<SPARSE>(logits, part_max, part_sum, NP, NPs, b, gamma, V, draft, q,
                                       uniforms, r_m, r_s, &flags);
    if (threadIdx.x < g1) {
        const int i = threadIdx.x;
        row_max[(size_t)b * g1 + i] = r_m[i];
        row_sum[(size_t)b * g1 + i] = r_s[i];
        if (i != n) out_tokens[(size_t)b * g1 + i] = i < n ? draft[(size_t)b * gamma + i] : -1;
    }
    if (threadIdx.x == 0) {
        n_accepted[b] = n;
        status[b] = flags;
    }
}

// Three forms.  kDrawFused: every chunk workgroup runs the accept tests
// itself and the sequence's last workgroup picks the token (few sequences:
// one launch).  kDrawInline: every chunk workgroup runs the accept tests and
// writes its chunk totals, chunk 0's workgroup writes the outputs that
// depend on n only, and pick_kernel follows (two launches, no device-scope
// arrival per workgroup).  kDrawSplit: accept_kernel ran first; the
// workgroup reads n and the draw row's normaliser it left and writes the
// chunk totals of its split_chunks_per_group chunks, and pick_kernel follows.  A kernel boundary orders the
// totals before the pick in both two-launch forms.
enum DrawForm { kDrawSplit = 0, kDrawFused = 1, kDrawInline = 2 };
// Chunks per workgroup in the split form (many sequences).  Dense q: four
// 4096-token chunks in turn, a quarter of the workgroups (stage 2 at B = 256,
// V = 128256: 63.2 -> 60.9 us; B = 64: 28.1 -> 27.1 us).  Sparse q: one,
// since each chunk rebuilds its dense q from all K entries of the row (four
// in turn measured 16.6 -> 23.4 us at B = 8).
constexpr int split_chunks_per_group(bool sparse) { return sparse ? 1 : 4; }

template <int FORM, bool SPARSE>
__global__ __launch_bounds__(kDrawBlock) void draw_kernel(
    const float* __restrict__ logits, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, int NP, int NPs, const int32_t* __restrict__ draft,
    QArg q, const float* __restrict__ uniforms, int gamma, int V, int NC, ChunkSums cs,
    int32_t* __restrict__ counters, float* __restrict__ row_max, float* __restrict__ row_sum,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ n_accepted,
    int32_t* __restrict__ status) {
    __shared__ float r_m[SV_MAX_GAMMA + 1], r_s[SV_MAX_GAMMA + 1];
    __shared__ __attribute__((aligned(16))) unsigned s_qc[SPARSE ? kDrawChunk : 4];
    // flat grid: workgroup x covers chunks CPW (x % NG) .. CPW (x % NG) + CPW - 1
    // of sequence x / NG, NG = ceil(NC / CPW) workgroups per sequence
    constexpr int CPW = FORM == kDrawSplit ? split_chunks_per_group(SPARSE) : 1;
    const int NG = (NC + CPW - 1) / CPW;
    const int cg = (int)(blockIdx.x % (unsigned)NG), b = (int)(blockIdx.x / (unsigned)NG);
    const int c = cg * CPW;                    // the first (with CPW = 1 the only) chunk
    const int g1 = gamma + 1;

    constexpr bool FUSED = FORM == kDrawFused;
    constexpr bool ACCEPT = FORM != kDrawSplit;
    int flags = 0;
    int n;
    float M, S;
    if (ACCEPT) {
        n = accept_tests<SPARSE>(logits, part_max, part_sum, NP, NPs, b, gamma, V, draft, q,
                                 uniforms, r_m, r_s, &flags);
        M = r_m[n];
        S = r_s[n];
    } else {
        n = n_accepted[b];
        M = row_max[(size_t)b * g1 + n];
        S = row_sum[(size_t)b * g1 + n];
    }
    const DrawRow d = draw_row<SPARSE>(logits, q, b, gamma, n, V, M, S);
    for (int i = 0; i < CPW && c + i < NC; ++i) {
        const int c0 = (c + i) * kDrawChunk;
        if (SPARSE && d.has_q()) stage_sparse_chunk(d, c0, s_qc);
        float w[kDrawPerThread], p[kDrawPerThread];
        draw_weights<SPARSE>(d, c0 + threadIdx.x * kDrawPerThread, s_qc, c0, w, p);
        double tw = 0.0, tp = 0.0;
#pragma unroll
        for (int e = 0; e < kDrawPerThread; ++e) { tw += (double)w[e]; tp += (double)p[e]; }
        store_chunk_totals(tw, tp, cs, (size_t)b * NC + c + i);
        // the next chunk reuses the totals' and the sparse chunk's LDS
        if (CPW > 1) __syncthreads();
    }
    if (FORM == kDrawInline && c == 0) {       // the outputs that depend on n only
        if (threadIdx.x < g1) {
            const int i = threadIdx.x;
            row_max[(size_t)b * g1 + i] = r_m[i];
            row_sum[(size_t)b * g1 + i] = r_s[i];
            if (i != n) out_tokens[(size_t)b * g1 + i] = i < n ? draft[(size_t)b * gamma + i] : -1;
        }
        if (threadIdx.x == 0) {
            n_accepted[b] = n;
            status[b] = flags;
        }
    }
    if (!FUSED) return;
    if (!arrive_last(&counters[(size_t)b * kCounterStride], NC)) return;
    if (threadIdx.x >= kWave) return;          // the rest is one wave's

    // The sequence's last workgroup: outputs that depend on n only ...
    if (FUSED && threadIdx.x < g1) {
        const int i = threadIdx.x;
        row_max[(size_t)b * g1 + i] = r_m[i];
        row_sum[(size_t)b * g1 + i] = r_s[i];
        if (i != n) out_tokens[(size_t)b * g1 + i] = i < n ? draft[(size_t)b * gamma + i] : -1;
    }
    // ... and the draw (the chunk pass is done with s_qc).
    int pflags;
    const int tok = pick<SPARSE>(d, b, NC, cs, uniforms[(size_t)b * g1 + gamma], s_qc, &pflags);
    if (threadIdx.x == 0) {
        out_tokens[(size_t)b * g1 + n] = tok;
        n_accepted[b] = n;
        status[b] = flags | pflags;
        counters[(size_t)b * kCounterStride] = 0;   // ready for a repeated stage-2 call
    }
}

// The draw for one sequence from the chunk totals draw_kernel<false> wrote:
// one wave per sequence.
template <bool SPARSE>
__global__ __launch_bounds__(kWave) void pick_kernel(
    const float* __restrict__ logits, QArg q,
    const float* __restrict__ uniforms, int gamma, int V, int NC, ChunkSums cs,
    const float* __restrict__ row_max, const float* __restrict__ row_sum,
    int32_t* __restrict__ out_tokens, const int32_t* __restrict__ n_accepted,
    int32_t* __restrict__ status) {
    __shared__ __attribute__((aligned(16))) unsigned s_qc[SPARSE ? kWave * kDrawPerThread : 4];
    const int b = blockIdx.x;
    const int g1 = gamma + 1;
    const int n = n_accepted[b];
    const size_t k = (size_t)b * g1 + n;
    const DrawRow d = draw_row<SPARSE>(logits, q, b, gamma, n, V, row_max[k], row_sum[k]);
    int flags;
    const int tok = pick<SPARSE>(d, b, NC, cs, uniforms[(size_t)b * g1 + gamma], s_qc, &flags);
    if (threadIdx.x == 0) {
        out_tokens[k] = tok;
        if (flags) status[b] |= flags;
    }
}

}  // namespace

// Fused form up to 64 draw workgroups: stage 2 measured 7.6 us fused vs
// 7.7 us inline at B = 1 over 64 chunks, 8.4 vs 8.0 us at B = 4 over 32
// chunks (and 10.8 us split), and 15.6 vs 9.6 us at 512 workgroups, where the
// workgroups' device-scope releases cost more than the pick's extra launch.
constexpr int kFuseMaxGroups = 64;
// Sparse q has no inline form (below), so it stays fused up to 256.
constexpr int kFuseMaxGroupsSparse = 256;
// Inline form from 65 to 1024 draw workgroups: 11.2 -> 9.6 us at 512
// (B = 8 over 64 chunks, B = 16 over 32); at 2048 it measured 24.2 us against
// 20.8 us split, where every workgroup repeating the accept tests costs more
// than the accept launch.
constexpr int kInlineMaxGroups = 1024;

namespace {

template <bool SPARSE>
hipError_t launch_accept_draw_t(const float* logits, const float* part_max, const float* part_sum,
                                int NP, int NPs, int B, int gamma, int V, const int32_t* draft,
                                QArg q, const float* uniforms, int NC, const ChunkSums& cs,
                                int32_t* counters, float* row_max, float* row_sum,
                                int32_t* out_tokens, int32_t* n_accepted, int32_t* status,
                                hipStream_t stream) {
    const unsigned groups = (unsigned)NC * (unsigned)B;
    // Few draw workgroups: fuse the accept tests into each and let the last
    // one pick (one launch).  More: the accept tests in each workgroup, then
    // the pick (two launches; no device-scope arrival per workgroup).  Many:
    // accept once per sequence, chunk totals, then the pick -- three
    // launches, no workgroup repeats the accept tests.
    if (groups <= (SPARSE ? kFuseMaxGroupsSparse : kFuseMaxGroups)) {
        draw_kernel<kDrawFused, SPARSE><<<dim3(groups), dim3(kDrawBlock), 0, stream>>>(
            logits, part_max, part_sum, NP, NPs, draft, q, uniforms, gamma, V, NC, cs, counters,
            row_max, row_sum, out_tokens, n_accepted, status);
        return hipGetLastError();
    }
    hipError_t e;
    // (Sparse q stays split: repeating its id lookups in every workgroup
    // measured slower, 172.3 -> 175.7 us per step at B = 8.)
    if (!SPARSE && groups <= kInlineMaxGroups) {
        draw_kernel<kDrawInline, SPARSE><<<dim3(groups), dim3(kDrawBlock), 0, stream>>>(
            logits, part_max, part_sum, NP, NPs, draft, q, uniforms, gamma, V, NC, cs, counters,
            row_max, row_sum, out_tokens, n_accepted, status);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        accept_kernel<SPARSE><<<dim3(B), dim3(kDrawBlock), 0, stream>>>(
            logits, part_max, part_sum, NP, NPs, draft, q, uniforms, gamma, V, row_max, row_sum,
            out_tokens, n_accepted, status);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        constexpr int cpw = split_chunks_per_group(SPARSE);
        const unsigned split_groups = (unsigned)((NC + cpw - 1) / cpw) * (unsigned)B;
        draw_kernel<kDrawSplit, SPARSE><<<dim3(split_groups), dim3(kDrawBlock), 0, stream>>>(
            logits, part_max, part_sum, NP, NPs, draft, q, uniforms, gamma, V, NC, cs, counters,
            row_max, row_sum, out_tokens, n_accepted, status);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    pick_kernel<SPARSE><<<dim3(B), dim3(kWave), 0, stream>>>(logits, q, uniforms, gamma, V, NC, cs,
                                                            row_max, row_sum, out_tokens,
                                                            n_accepted, status);
    return hipGetLastError();
}

}  // namespace

// q_idx == nullptr: dense q [B][gamma][V]; otherwise sparse q, K entries per row.
hipError_t launch_accept_draw(const float* logits, const float* part_max, const float* part_sum,
                              int NP, int NPs, int B, int gamma, int V, const int32_t* draft,
                              const float* q, const int32_t* q_idx, int K, const float* uniforms,
                              int NC, const ChunkSums& cs, int32_t* counters,
                              float* row_max, float* row_sum, int32_t* out_tokens,
                              int32_t* n_accepted, int32_t* status, hipStream_t stream) {
    const QArg qa{q, q_idx, K};
    if (q_idx)
        return launch_accept_draw_t<true>(logits, part_max, part_sum, NP, NPs, B, gamma, V, draft,
                                          qa, uniforms, NC, cs, counters, row_max, row_sum,
                                          out_tokens, n_accepted, status, stream);
    return launch_accept_draw_t<false>(logits, part_max, part_sum, NP, NPs, B, gamma, V, draft, qa,
                                       uniforms, NC, cs, counters, row_max, row_sum,
                                       out_tokens, n_accepted, status, stream);
}

}  // namespace sv
