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
// Kernels (all 256 threads, enqueued in this order on one stream):
//   accept_kernel     one workgroup per sequence: merge the LM-head tile
//                     partials into each row's softmax normaliser, run the
//                     gamma accept tests (r * q <= p) and find the first
//                     rejection with a wave ballot.
//   draw_sums_kernel  one workgroup per (sequence, 4096-token chunk): fp64
//                     totals of the draw weights (residual or p) and of p.
//   draw_pick_kernel  one workgroup per sequence: scan the chunk totals, find
//                     the chunk where the running sum reaches u * S, rescan
//                     that chunk and pick the first token that reaches it.
// The weights are recomputed from the logits in both draw kernels with the
// same code, and the chunk scan is the same routine, so the chunk totals the
// second kernel walks are bitwise those the first one wrote.

#include "sv_common.h"

namespace sv {

namespace {

__device__ __forceinline__ float target_prob(float logit, float row_max, float row_sum) {
    return expf(logit - row_max) / row_sum;
}

// Inclusive prefix sum of one double per thread over the workgroup, in a
// fixed order (Hillis-Steele within each wave, then the wave totals added in
// wave order).  Returns this thread's inclusive value; *total gets the sum.
__device__ double block_inclusive_scan(double v, double* total) {
    __shared__ double s_wave[kBlock / kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const double o = __shfl_up(v, off);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) s_wave[wave] = v;
    __syncthreads();
    double before = 0.0, all = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) {
        if (w < wave) before += s_wave[w];
        all += s_wave[w];
    }
    __syncthreads();
    // all = ((w0 + w1) + w2) + w3, the same association as the last thread's value.
    *total = all;
    return wave == 0 ? v : before + v;
}

__device__ __forceinline__ int block_min_int(int v) {
    __shared__ int s[kBlock / kWave];
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off));
    if ((threadIdx.x & (kWave - 1)) == 0) s[threadIdx.x / kWave] = v;
    __syncthreads();
    int r = s[0];
#pragma unroll
    for (int w = 1; w < kBlock / kWave; ++w) r = min(r, s[w]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ int block_max_int(int v) { return -block_min_int(-v); }

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kBlock) void accept_kernel(
    const float* __restrict__ logits, const float* __restrict__ part_max,
    const float* __restrict__ part_sum, int NP, int gamma, int V,
    const int32_t* __restrict__ draft, const float* __restrict__ q,
    const float* __restrict__ uniforms, float* __restrict__ row_max, float* __restrict__ row_sum,
    int32_t* __restrict__ out_tokens, int32_t* __restrict__ n_accepted,
    int32_t* __restrict__ status) {
    __shared__ float s_m[kBlock / kWave], s_s[kBlock / kWave];
    __shared__ float r_m[SV_MAX_GAMMA + 1], r_s[SV_MAX_GAMMA + 1];
    const int b = blockIdx.x;
    const int g1 = gamma + 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // Softmax normaliser of each of this sequence's gamma+1 rows.
    for (int i = 0; i < g1; ++i) {
        const size_t r = (size_t)b * g1 + i;
        float m = -INFINITY, s = 0.f;
        for (int j = threadIdx.x; j < NP; j += kBlock) lse_merge(m, s, part_max[r * NP + j], part_sum[r * NP + j]);
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
            lse_merge(m, s, m2, s2);
        }
        if (lane == 0) { s_m[wave] = m; s_s[wave] = s; }
        __syncthreads();
        if (threadIdx.x == 0) {
            float M = -INFINITY, S = 0.f;
            for (int w = 0; w < kBlock / kWave; ++w) lse_merge(M, S, s_m[w], s_s[w]);
            r_m[i] = M; r_s[i] = S;
            row_max[r] = M; row_sum[r] = S;
        }
        __syncthreads();
    }

    if (wave == 0) {
        bool keep = false;
        int flags = 0;
        if (lane < gamma) {
            const int x = draft[(size_t)b * gamma + lane];
            if (x >= 0 && x < V) {
                const size_t r = (size_t)b * g1 + lane;
                const float p = target_prob(logits[r * V + x], r_m[lane], r_s[lane]);
                const float qx = q[((size_t)b * gamma + lane) * V + x];
                keep = uniforms[(size_t)b * g1 + lane] * qx <= p;
            } else {
                flags = SV_DEV_BAD_DRAFT;
            }
        }
        const unsigned long long kept = __ballot(keep);
        const int n = min(__builtin_ctzll(~kept), gamma);
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) flags |= __shfl_xor(flags, off);
        if (lane == 0) { n_accepted[b] = n; status[b] = flags; }
        if (lane < g1 && lane != n)
            out_tokens[(size_t)b * g1 + lane] = lane < n ? draft[(size_t)b * gamma + lane] : -1;
    }
}

// ---------------------------------------------------------------------------
// The row a sequence draws from: its logits, the q of the rejected draft
// (nullptr for the bonus draw), and its softmax normaliser.
struct DrawRow {
    const float* lrow;   // logits of the draw row
    const float* qrow;   // q of the rejected draft, or nullptr for the bonus
    float M, S;          // softmax normaliser of the draw row
    int V;
};

__device__ __forceinline__ void load16(const float* row, int j0, int V, float (&x)[kDrawPerThread]) {
    if (((V & 3) == 0) && j0 + kDrawPerThread <= V) {
#pragma unroll
        for (int e = 0; e < kDrawPerThread; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + j0 + e);
            x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kDrawPerThread; ++e) x[e] = j0 + e < V ? row[j0 + e] : 0.f;
    }
}

// Draw weights w and target probabilities p of 16 consecutive tokens from j0
// (zero past the end of the vocabulary).
__device__ __forceinline__ void draw_weights16(const DrawRow& d, int j0, float (&w)[kDrawPerThread],
                                               float (&p)[kDrawPerThread]) {
    float l[kDrawPerThread], qv[kDrawPerThread];
    load16(d.lrow, j0, d.V, l);
    if (d.qrow) load16(d.qrow, j0, d.V, qv);
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) {
        const bool in = j0 + e < d.V;
        p[e] = in ? target_prob(l[e], d.M, d.S) : 0.f;
        w[e] = in ? (d.qrow ? fmaxf(0.f, p[e] - qv[e]) : p[e]) : 0.f;
    }
}

__device__ __forceinline__ DrawRow draw_row(const float* logits, const float* q, const float* row_max,
                                            const float* row_sum, const int32_t* n_accepted,
                                            int b, int gamma, int V) {
    const int n = n_accepted[b];
    const size_t k = (size_t)b * (gamma + 1) + n;
    DrawRow d;
    d.lrow = logits + k * V;
    d.qrow = n < gamma ? q + ((size_t)b * gamma + n) * V : nullptr;
    d.M = row_max[k];
    d.S = row_sum[k];
    d.V = V;
    return d;
}

__global__ __launch_bounds__(kBlock) void draw_sums_kernel(
    const float* __restrict__ logits, const float* __restrict__ q, const float* __restrict__ row_max,
    const float* __restrict__ row_sum, const int32_t* __restrict__ n_accepted, int gamma, int V,
    int NC, double* __restrict__ csum, double* __restrict__ psum) {
    // flat grid: workgroup x covers chunk x % NC of sequence x / NC
    const int c = (int)(blockIdx.x % (unsigned)NC), b = (int)(blockIdx.x / (unsigned)NC);
    const DrawRow d = draw_row(logits, q, row_max, row_sum, n_accepted, b, gamma, V);
    float w[kDrawPerThread], p[kDrawPerThread];
    draw_weights16(d, c * kDrawChunk + threadIdx.x * kDrawPerThread, w, p);
    double tw = 0.0, tp = 0.0;
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) { tw += (double)w[e]; tp += (double)p[e]; }
    double tot_w, tot_p;
    block_inclusive_scan(tw, &tot_w);
    block_inclusive_scan(tp, &tot_p);
    if (threadIdx.x == 0) {
        csum[(size_t)b * NC + c] = tot_w;
        psum[(size_t)b * NC + c] = tot_p;
    }
}

// Exclusive prefix of one double per thread: the inclusive value of the
// previous thread, so that excl(t) + own(t) is never needed.
__device__ double block_exclusive_scan(double v, double* total) {
    __shared__ double s_last[kBlock / kWave];
    const double incl = block_inclusive_scan(v, total);
    const int lane = threadIdx.x & (kWave - 1);
    const double up = __shfl_up(incl, 1);
    if (lane == kWave - 1) s_last[threadIdx.x / kWave] = incl;
    __syncthreads();
    const double r = lane > 0 ? up : (threadIdx.x == 0 ? 0.0 : s_last[threadIdx.x / kWave - 1]);
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kBlock) void draw_pick_kernel(
    const float* __restrict__ logits, const float* __restrict__ q, const float* __restrict__ row_max,
    const float* __restrict__ row_sum, const int32_t* __restrict__ n_accepted,
    const float* __restrict__ uniforms, int gamma, int V, int NC, const double* __restrict__ csum,
    const double* __restrict__ psum, int32_t* __restrict__ out_tokens, int32_t* __restrict__ status) {
    __shared__ double s_before;
    const int b = blockIdx.x;
    DrawRow d = draw_row(logits, q, row_max, row_sum, n_accepted, b, gamma, V);
    const int n = n_accepted[b];
    const size_t out_at = (size_t)b * (gamma + 1) + n;
    // Thread t owns chunks [t*per, (t+1)*per) of the chunk totals.
    const int per = (NC + kBlock - 1) / kBlock;
    const int c0 = threadIdx.x * per, c1 = min(NC, c0 + per);

    // Total draw weight S; fall back to p when the residual carries none.
    const double* sums = csum + (size_t)b * NC;
    double own = 0.0, S;
    for (int c = c0; c < c1; ++c) own += sums[c];
    double excl = block_exclusive_scan(own, &S);
    int flags = 0;
    if (!(S > 0.0)) {
        flags = SV_DEV_FALLBACK;
        d.qrow = nullptr;
        sums = psum + (size_t)b * NC;
        own = 0.0;
        for (int c = c0; c < c1; ++c) own += sums[c];
        excl = block_exclusive_scan(own, &S);
    }
    if (!(S > 0.0) || !(S < INFINITY)) {
        if (threadIdx.x == 0) {
            out_tokens[out_at] = 0;
            status[b] |= flags | SV_DEV_NONFINITE;
        }
        return;
    }
    const double t = (double)uniforms[(size_t)b * (gamma + 1) + gamma] * S;

    // The first chunk whose running sum reaches t and that carries weight;
    // failing that (only through rounding), the last chunk with weight.
    int first = INT_MAX, last_pos = -1;
    double run = excl;
    for (int c = c0; c < c1; ++c) {
        run += sums[c];
        if (sums[c] > 0.0) {
            last_pos = c;
            if (first == INT_MAX && run >= t) first = c;
        }
    }
    int chunk = block_min_int(first);
    if (chunk == INT_MAX) chunk = block_max_int(last_pos);
    // Running sum before that chunk, from its owner, in the same order.
    if (c0 <= chunk && chunk < c1) {
        double r = excl;
        for (int c = c0; c < chunk; ++c) r += sums[c];
        s_before = r;
    }
    __syncthreads();
    const double before = s_before;

    // Rescan the chunk in token order: exclusive prefix of this thread's
    // 16 tokens, then their sequential sums.
    const int j0 = chunk * kDrawChunk + threadIdx.x * kDrawPerThread;
    float w[kDrawPerThread], p[kDrawPerThread];
    draw_weights16(d, j0, w, p);
    double mine = 0.0, chunk_total;
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) mine += (double)w[e];
    const double base = before + block_exclusive_scan(mine, &chunk_total);
    int y = INT_MAX, ylast = -1;
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) {
        part += (double)w[e];
        if (w[e] > 0.f) {
            ylast = j0 + e;
            if (y == INT_MAX && base + part >= t) y = j0 + e;
        }
    }
    int pick = block_min_int(y);
    if (pick == INT_MAX) pick = block_max_int(ylast);
    if (threadIdx.x == 0) {
        out_tokens[out_at] = pick;
        if (flags) status[b] |= flags;
    }
}

}  // namespace

hipError_t launch_accept(const float* logits, const float* part_max, const float* part_sum, int NP,
                         int B, int gamma, int V, const int32_t* draft, const float* q,
                         const float* uniforms, float* row_max, float* row_sum, int32_t* out_tokens,
                         int32_t* n_accepted, int32_t* status, hipStream_t stream) {
    accept_kernel<<<dim3(B), dim3(kBlock), 0, stream>>>(logits, part_max, part_sum, NP, gamma, V, draft, q,
                                                       uniforms, row_max, row_sum, out_tokens,
                                                       n_accepted, status);
    return hipGetLastError();
}

hipError_t launch_draw(const float* logits, const float* q, const float* row_max, const float* row_sum,
                       const int32_t* n_accepted, const float* uniforms, int B, int gamma, int V,
                       int NC, double* csum, double* psum, int32_t* out_tokens, int32_t* status,
                       hipStream_t stream) {
    draw_sums_kernel<<<dim3((unsigned)NC * (unsigned)B), dim3(kBlock), 0, stream>>>(logits, q, row_max, row_sum, n_accepted,
                                                             gamma, V, NC, csum, psum);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    draw_pick_kernel<<<dim3(B), dim3(kBlock), 0, stream>>>(logits, q, row_max, row_sum, n_accepted,
                                                          uniforms, gamma, V, NC, csum, psum,
                                                          out_tokens, status);
    return hipGetLastError();
}

}  // namespace sv
