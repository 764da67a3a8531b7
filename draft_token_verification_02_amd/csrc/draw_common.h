// Device helpers shared by the draw kernels of chain and tree verification:
// the target probability, the sparse-q lookups, workgroup scans, the merge
// of the LM-head's softmax partials, the draw weights and the inverse-CDF
// pick.  Included by each kernel file (internal linkage, one copy per file).
//
// Source: "推测解码" (world.lapla.si/zh/specdec), section 通过的规则 -- keep
// a drafted token when r <= p/q, otherwise replace it with a draw from
// max(0, p - q) renormalised; the draw here is an inverse CDF over
// ascending token id.
#pragma once

#include "sv_common.h"

namespace sv {

namespace {

__device__ __forceinline__ float target_prob(float logit, float row_max, float row_sum) {
    return expf(logit - row_max) / row_sum;
}

// The drafter's q at the gamma drafted positions of every sequence.
//   dense:  val [B][gamma][V], idx == nullptr;
//   sparse: idx / val [B][gamma][K]: ids in [0, V) listed once each, ids < 0
//           are padding; a token not listed has q = 0.  Sparse values that
//           are negative or NaN count as 0, and an id listed more than once
//           takes the largest of its values (the same rule in the accept
//           test and in the draw, so the result stays deterministic).
struct QArg {
    const float* val;
    const int32_t* idx;
    int K;
};

// A sparse value as it is used: negative, -0 and NaN become +0, so the bit
// pattern orders like the value (the LDS chunk merges entries by unsigned max).
__device__ __forceinline__ float sparse_value(float v) { return v > 0.f ? v : 0.f; }

// Inclusive prefix sum of one double per thread over the workgroup, in a
// fixed order (Hillis-Steele within each wave, then the wave totals added in
// wave order).  Returns this thread's inclusive value; *total gets the sum,
// with the same association as the last thread's value.
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
    *total = all;
    return wave == 0 ? v : before + v;
}

// Exclusive prefix: the previous thread's inclusive value (never incl - own).
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

// Softmax normalisers (max, sum exp) of rows row0 .. row0+nrows-1 from the
// LM-head's per-workgroup partials, into r_m[i], r_s[i].  TPR threads of one
// wave share a row (TPR = 32, 16 or 8, the most that still fits every row in
// one pass when it can), each loading its 16-byte groups of maxima and sums
// kBatch at a time before merging them, so a row costs one memory round trip
// per kBatch * TPR * 4 partials.  Every thread of the workgroup takes part;
// the caller synchronises before reading the results.
template <int TPR>
__device__ void merge_row_partials_t(const float* __restrict__ part_max,
                                     const float* __restrict__ part_sum, int NP, int NPs,
                                     size_t row0, int nrows, float* r_m, float* r_s) {
    constexpr int kRows = kBlock / TPR;          // rows per pass
    constexpr int kBatch = 8;                    // float4 loads per thread and array in flight
    const int sub = threadIdx.x % TPR;
    const int grp = threadIdx.x / TPR;
    const int n4 = (NP + 3) / 4;
    for (int i0 = 0; i0 < nrows; i0 += kRows) {
        const int i = i0 + grp;
        float m = -INFINITY, s = 0.f;
        if (i < nrows) {
            const size_t r = row0 + i;
            const float4* pm = reinterpret_cast<const float4*>(part_max + r * NPs);
            const float4* ps = reinterpret_cast<const float4*>(part_sum + r * NPs);
            for (int j0 = 0; j0 < n4; j0 += kBatch * TPR) {
                float4 a[kBatch], c[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int jj = j0 + sub + u * TPR;
                    a[u] = jj < n4 ? pm[jj] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                    c[u] = jj < n4 ? ps[jj] : make_float4(0.f, 0.f, 0.f, 0.f);
                }
                // this batch's max, then its rescaled sum, merged into (m, s)
                float bm = -INFINITY, bs = 0.f;
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int j = 4 * (j0 + sub + u * TPR);      // entries past NP are padding
                    if (j + 0 < NP) bm = fmaxf(bm, a[u].x);
                    if (j + 1 < NP) bm = fmaxf(bm, a[u].y);
                    if (j + 2 < NP) bm = fmaxf(bm, a[u].z);
                    if (j + 3 < NP) bm = fmaxf(bm, a[u].w);
                }
                if (bm != -INFINITY) {
#pragma unroll
                    for (int u = 0; u < kBatch; ++u) {
                        const int j = 4 * (j0 + sub + u * TPR);
                        if (j + 0 < NP && a[u].x != -INFINITY) bs += c[u].x * expf(a[u].x - bm);
                        if (j + 1 < NP && a[u].y != -INFINITY) bs += c[u].y * expf(a[u].y - bm);
                        if (j + 2 < NP && a[u].z != -INFINITY) bs += c[u].z * expf(a[u].z - bm);
                        if (j + 3 < NP && a[u].w != -INFINITY) bs += c[u].w * expf(a[u].w - bm);
                    }
                }
                lse_merge(m, s, bm, bs);
            }
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) {
            const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
            lse_merge(m, s, m2, s2);
        }
        if (sub == 0 && i < nrows) { r_m[i] = m; r_s[i] = s; }
    }
}

__device__ void merge_row_partials(const float* __restrict__ part_max,
                                   const float* __restrict__ part_sum, int NP, int NPs, size_t row0,
                                   int nrows, float* r_m, float* r_s) {
    if (nrows <= kBlock / 32)
        merge_row_partials_t<32>(part_max, part_sum, NP, NPs, row0, nrows, r_m, r_s);
    else if (nrows <= kBlock / 16)
        merge_row_partials_t<16>(part_max, part_sum, NP, NPs, row0, nrows, r_m, r_s);
    else
        merge_row_partials_t<8>(part_max, part_sum, NP, NPs, row0, nrows, r_m, r_s);
}

// ---------------------------------------------------------------------------
// The row a sequence draws from: its logits, the q of the rejected draft
// (none for the bonus draw), and its softmax normaliser.  The draw weights
// are max(0, p - c q): c = 1 for the residual after one rejection; tree
// verification's residual after several rejected siblings has a larger c.
struct DrawRow {
    const float* lrow;
    const float* qrow;        // dense q row, or nullptr
    const int32_t* qids;      // sparse q row, or nullptr
    const float* qvals;
    int K;
    float M, S;
    float c;
    int V;
    __device__ bool has_q() const { return qrow != nullptr || qids != nullptr; }
    __device__ void drop_q() { qrow = nullptr; qids = nullptr; }
};

template <bool SPARSE>
__device__ __forceinline__ DrawRow draw_row(const float* logits, QArg q, int b, int gamma, int n,
                                            int V, float M, float S) {
    DrawRow d;
    const size_t k = (size_t)b * (gamma + 1) + n;
    d.lrow = logits + k * V;
    d.qrow = nullptr;
    d.qids = nullptr;
    d.qvals = nullptr;
    d.K = q.K;
    if (n < gamma) {
        const size_t r = (size_t)b * gamma + n;
        if (SPARSE) { d.qids = q.idx + r * q.K; d.qvals = q.val + r * q.K; }
        else        { d.qrow = q.val + r * V; }
    }
    d.M = M;
    d.S = S;
    d.c = 1.f;
    d.V = V;
    return d;
}

// The dense q of chunk [c0, c0 + kDrawChunk) of a sparse row, built in LDS:
// zeroed, then every entry whose id falls in the chunk merged in by unsigned
// max on the value's bits (values were made non-negative, where the bit
// order is the value order).  Every thread of the workgroup takes part.
__device__ void stage_sparse_chunk(const DrawRow& d, int c0, unsigned* s_qc) {
    for (int j = threadIdx.x; j < kDrawChunk; j += kBlock) s_qc[j] = 0u;
    __syncthreads();
    auto put = [&](int id, float v) {
        const unsigned rel = (unsigned)(id - c0);
        if (id >= 0 && id < d.V && rel < (unsigned)kDrawChunk)
            atomicMax(&s_qc[rel], __float_as_uint(sparse_value(v)));
    };
    if ((d.K & 3) == 0) {
        const int4* id4 = reinterpret_cast<const int4*>(d.qids);
        const float4* v4 = reinterpret_cast<const float4*>(d.qvals);
        const int K4 = d.K >> 2;
#pragma unroll 4
        for (int j = threadIdx.x; j < K4; j += kBlock) {
            const int4 i = id4[j];
            const float4 v = v4[j];
            put(i.x, v.x); put(i.y, v.y); put(i.z, v.z); put(i.w, v.w);
        }
    } else {
        for (int j = threadIdx.x; j < d.K; j += kBlock) put(d.qids[j], d.qvals[j]);
    }
    __syncthreads();
}

__device__ __forceinline__ void load16(const float* row, int j0, int V, float (&x)[kDrawPerThread]) {
    if (((V & 3) == 0) && j0 + kDrawPerThread <= V) {
#pragma unroll
        for (int e = 0; e < kDrawPerThread; e += 4) {
            const float4 v = *reinterpret_cast<const float4*>(row + j0 + e);
            x[e] = v.x; x[e + 1] = v.y; x[e + 2] = v.z; x[e + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < kDrawPerThread; ++e) x[e] = 0.f;
#pragma unroll
        for (int e = 0; e < kDrawPerThread; ++e)
            if (j0 + e < V) x[e] = row[j0 + e];
    }
}

// Draw weights w and target probabilities p of 16 consecutive tokens from j0
// (zero past the end of the vocabulary).  With sparse q, s_qc holds the
// chunk starting at c0 (stage_sparse_chunk).
template <bool SPARSE>
__device__ __forceinline__ void draw_weights16(const DrawRow& d, int j0, const unsigned* s_qc, int c0,
                                               float (&w)[kDrawPerThread], float (&p)[kDrawPerThread]) {
    float l[kDrawPerThread], qv[kDrawPerThread];
    load16(d.lrow, j0, d.V, l);
    const bool has_q = d.has_q();
    if (SPARSE) {
        if (has_q) {
            const uint4* src = reinterpret_cast<const uint4*>(s_qc + (j0 - c0));
#pragma unroll
            for (int e = 0; e < kDrawPerThread; e += 4) {
                const uint4 v = src[e / 4];
                qv[e] = __uint_as_float(v.x); qv[e + 1] = __uint_as_float(v.y);
                qv[e + 2] = __uint_as_float(v.z); qv[e + 3] = __uint_as_float(v.w);
            }
        }
    } else if (has_q) {
        load16(d.qrow, j0, d.V, qv);
    }
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) {
        const bool in = j0 + e < d.V;
        p[e] = in ? target_prob(l[e], d.M, d.S) : 0.f;
        w[e] = in ? (has_q ? fmaxf(0.f, p[e] - d.c * qv[e]) : p[e]) : 0.f;
    }
}

// The inverse-CDF draw for sequence b from its chunk totals.  Returns the
// token; *flags gets SV_DEV_FALLBACK / SV_DEV_NONFINITE.
template <bool SPARSE>
__device__ int pick(DrawRow d, int b, int NC, const double* csum, const double* psum, float u,
                    unsigned* s_qc, int* flags) {
    __shared__ double s_before;
    // Thread t owns chunks [t*per, (t+1)*per) of the chunk totals.
    const int per = (NC + kBlock - 1) / kBlock;
    const int c0 = threadIdx.x * per, c1 = min(NC, c0 + per);

    // Total draw weight S; fall back to p when the residual carries none.
    const double* sums = csum + (size_t)b * NC;
    double own = 0.0, S;
    for (int c = c0; c < c1; ++c) own += sums[c];
    double excl = block_exclusive_scan(own, &S);
    *flags = 0;
    if (!(S > 0.0)) {
        *flags = SV_DEV_FALLBACK;
        d.drop_q();
        sums = psum + (size_t)b * NC;
        own = 0.0;
        for (int c = c0; c < c1; ++c) own += sums[c];
        excl = block_exclusive_scan(own, &S);
    }
    if (!(S > 0.0) || !(S < INFINITY)) {
        *flags |= SV_DEV_NONFINITE;
        return 0;
    }
    const double t = (double)u * S;

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
    if (c0 <= chunk && chunk < c1) {          // its owner: running sum before it, same order
        double r = excl;
        for (int c = c0; c < chunk; ++c) r += sums[c];
        s_before = r;
    }
    __syncthreads();
    const double before = s_before;

    // Rescan that chunk in token order.
    const int cs = chunk * kDrawChunk;
    if (SPARSE && d.has_q()) stage_sparse_chunk(d, cs, s_qc);
    const int j0 = cs + threadIdx.x * kDrawPerThread;
    float w[kDrawPerThread], p[kDrawPerThread];
    draw_weights16<SPARSE>(d, j0, s_qc, cs, w, p);
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
    int tok = block_min_int(y);
    if (tok == INT_MAX) tok = block_max_int(ylast);
    return tok;
}

}  // namespace

}  // namespace sv
