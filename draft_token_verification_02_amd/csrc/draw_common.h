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

// exp(x) for x <= 0 as 2^(x log2 e) on the hardware exponential.  Its
// relative error is about |x| * 2^-23 from rounding x log2 e, plus the
// instruction's own ulp: below 2e-6 for every x down to -16, and further
// down the result is itself below 1.2e-7, so its absolute error is
// negligible next to the terms it is summed with.
__device__ __forceinline__ float exp_nonpos(float x) {
    return __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
}

// The target's probability of a token, exp(l - M) / S with the row's max M
// and normaliser S: exp_nonpos times the hardware reciprocal of S (one ulp),
// so its relative error stays near 2e-6 at worst, far inside the 1e-5 the
// results are held to.
__device__ __forceinline__ float target_prob(float logit, float row_max, float row_sum) {
    return exp_nonpos(logit - row_max) * __builtin_amdgcn_rcpf(row_sum);
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

// ---------------------------------------------------------------------------
// Wave-wide scans on DPP lane moves, which stay in the VALU (a shuffle goes
// through the LDS crossbar and waits on it): four row_shr steps scan each
// 16-lane row (Hillis-Steele), then the last lane of rows 0 and 2 is
// broadcast into rows 1 and 3 (row_bcast:15), then lane 31 into rows 2 and 3
// (row_bcast:31).  A lane or row with no source reads the identity.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppWaveShr1 = 0x138, kDppRowBcast15 = 0x142,
              kDppRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t identity) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double v) {      // identity +0
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = dpp_u32<CTRL, ROW_MASK>((uint32_t)b, 0u);
    const uint32_t hi = dpp_u32<CTRL, ROW_MASK>((uint32_t)(b >> 32), 0u);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float v, float identity) {
    return __uint_as_float(dpp_u32<CTRL, ROW_MASK>(__float_as_uint(v), __float_as_uint(identity)));
}

// Inclusive prefix sum within one wave (every scan of this file uses it).
__device__ __forceinline__ double wave_inclusive_scan(double v) {
    v += dpp_f64<kDppRowShr1, 0xf>(v);
    v += dpp_f64<kDppRowShr2, 0xf>(v);
    v += dpp_f64<kDppRowShr4, 0xf>(v);
    v += dpp_f64<kDppRowShr8, 0xf>(v);
    v += dpp_f64<kDppRowBcast15, 0xa>(v);
    v += dpp_f64<kDppRowBcast31, 0xc>(v);
    return v;
}

// The wave's maximum and sum, valid in lane 63.
__device__ __forceinline__ float wave_max_last(float v) {
    v = fmaxf(v, dpp_f32<kDppRowShr1, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowShr2, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowShr4, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowShr8, 0xf>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowBcast15, 0xa>(v, -INFINITY));
    v = fmaxf(v, dpp_f32<kDppRowBcast31, 0xc>(v, -INFINITY));
    return v;
}

__device__ __forceinline__ float wave_sum_last(float v) {
    v += dpp_f32<kDppRowShr1, 0xf>(v, 0.f);
    v += dpp_f32<kDppRowShr2, 0xf>(v, 0.f);
    v += dpp_f32<kDppRowShr4, 0xf>(v, 0.f);
    v += dpp_f32<kDppRowShr8, 0xf>(v, 0.f);
    v += dpp_f32<kDppRowBcast15, 0xa>(v, 0.f);
    v += dpp_f32<kDppRowBcast31, 0xc>(v, 0.f);
    return v;
}

// The previous lane's value (lane 0: +0), for an exclusive scan.
__device__ __forceinline__ double wave_shift_up(double v) { return dpp_f64<kDppWaveShr1, 0xf>(v); }

// Lane L's double (L uniform), in every lane (two readlanes).
__device__ __forceinline__ double wave_read(double v, int L) {
    const unsigned long long b = (unsigned long long)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, L);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), L);
    return __longlong_as_double((long long)(((unsigned long long)hi << 32) | lo));
}

// Lane 63's double, in every lane (two readlanes).
__device__ __forceinline__ double wave_last(double v) { return wave_read(v, kWave - 1); }

// The chunk pass's fp64 totals of the draw weights (tw) and of p (tp) of one
// chunk: per wave of the workgroup (the wave scan's last lane) and over the
// workgroup (a wave scan of the wave totals), stored into the chunk's entries
// of cs.  Wave 0 stores every one, so that a release by thread 0 orders all
// of them.  One barrier; the LDS it uses is its own.
__device__ __forceinline__ void store_chunk_totals(double tw, double tp, const ChunkSums& cs,
                                                   size_t chunk) {
    __shared__ double s_a[kDrawWaves], s_b[kDrawWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    tw = wave_inclusive_scan(tw);
    tp = wave_inclusive_scan(tp);
    if (lane == kWave - 1) { s_a[wave] = tw; s_b[wave] = tp; }
    __syncthreads();
    if (wave == 0) {
        double x = 0.0, y = 0.0;
        if (lane < kDrawWaves) {
            x = s_a[lane];
            y = s_b[lane];
            cs.cwave[chunk * kDrawWaves + lane] = x;
            cs.pwave[chunk * kDrawWaves + lane] = y;
        }
        x = wave_inclusive_scan(x);
        y = wave_inclusive_scan(y);
        if (lane == kWave - 1) {
            cs.csum[chunk] = x;
            cs.psum[chunk] = y;
        }
    }
}


// Softmax normalisers (max, sum exp) of rows row0 .. row0+nrows-1 from the
// LM-head's per-workgroup partials (m_j, s_j), into r_m[i] = M = max_j m_j and
// r_s[i] = sum_j s_j exp(m_j - M).  One wave per row, rows dealt to the waves
// in turn: lane l owns the 16-byte groups l, l + 64, l + 128 and l + 192 of
// the row (NP <= 1024), so a row needs neither LDS nor a barrier: the lane's
// maximum, the wave's on DPP moves, read from lane 63; then the lane's sum of
// s_j exp(m_j - M) in group order and the wave's sum.  One memory round trip
// and one exponential per partial; lane 63 writes the results.  The caller
// synchronises before reading them.  Always inlined: an out-of-line call
// starts by waiting for every memory operation in flight, which would put the
// caller's draft gathers in front of the partial loads.
constexpr int kMergeGroups = kLmMaxPartials / (4 * kWave);
static_assert(kMergeGroups * 4 * kWave == kLmMaxPartials, "whole float4 groups per lane");

__device__ __forceinline__ void merge_row_partials(const float* __restrict__ part_max,
                                                   const float* __restrict__ part_sum, int NP,
                                                   int NPs, size_t row0, int nrows, float* r_m,
                                                   float* r_s) {
    constexpr int NW = kDrawBlock / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int n4 = (NP + 3) / 4;
    // Row i goes to wave (i + 1) % NW: wave 0 gets no row while there are
    // fewer than NW, as it is the one that waits on the draft gathers.
    for (int i = (wave + NW - 1) % NW; i < nrows; i += NW) {
        const size_t r = row0 + i;
        const float4* pm = reinterpret_cast<const float4*>(part_max + r * NPs);
        const float4* ps = reinterpret_cast<const float4*>(part_sum + r * NPs);
        float4 a[kMergeGroups], c[kMergeGroups];
#pragma unroll
        for (int u = 0; u < kMergeGroups; ++u) {
            const int jj = min(lane + u * kWave, n4 - 1);    // past the end: loaded, masked
            a[u] = pm[jj];
            c[u] = ps[jj];
        }
        float m = -INFINITY;
#pragma unroll
        for (int u = 0; u < kMergeGroups; ++u) {
            const int e = 4 * (lane + u * kWave);
            a[u].x = e + 0 < NP ? a[u].x : -INFINITY;
            a[u].y = e + 1 < NP ? a[u].y : -INFINITY;
            a[u].z = e + 2 < NP ? a[u].z : -INFINITY;
            a[u].w = e + 3 < NP ? a[u].w : -INFINITY;
            m = fmaxf(m, fmaxf(fmaxf(a[u].x, a[u].y), fmaxf(a[u].z, a[u].w)));
        }
        const float M =
            __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_max_last(m)), kWave - 1));
        // entries at -inf are skipped outright, so that M = -inf (an empty
        // row) gives 0, not NaN
        auto term = [&](float x, float sj) {
            return x != -INFINITY ? sj * exp_nonpos(x - M) : 0.f;
        };
        float t = 0.f;
#pragma unroll
        for (int u = 0; u < kMergeGroups; ++u) {
            t += term(a[u].x, c[u].x);
            t += term(a[u].y, c[u].y);
            t += term(a[u].z, c[u].z);
            t += term(a[u].w, c[u].w);
        }
        t = wave_sum_last(t);
        if (lane == kWave - 1) { r_m[i] = M; r_s[i] = t; }
    }
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
    for (int j = threadIdx.x; j < kDrawChunk; j += kDrawBlock) s_qc[j] = 0u;
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
        for (int j = threadIdx.x; j < K4; j += kDrawBlock) {
            const int4 i = id4[j];
            const float4 v = v4[j];
            put(i.x, v.x); put(i.y, v.y); put(i.z, v.z); put(i.w, v.w);
        }
    } else {
        for (int j = threadIdx.x; j < d.K; j += kDrawBlock) put(d.qids[j], d.qvals[j]);
    }
    __syncthreads();
}

__device__ __forceinline__ void load_run(const float* row, int j0, int V, float (&x)[kDrawPerThread]) {
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

// Draw weights w and target probabilities p of the kDrawPerThread tokens from j0
// (zero past the end of the vocabulary).  With sparse q, s_qc holds the
// chunk starting at c0 (stage_sparse_chunk).
template <bool SPARSE>
__device__ __forceinline__ void draw_weights(const DrawRow& d, int j0, const unsigned* s_qc, int c0,
                                               float (&w)[kDrawPerThread], float (&p)[kDrawPerThread]) {
    float l[kDrawPerThread], qv[kDrawPerThread];
    load_run(d.lrow, j0, d.V, l);
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
        load_run(d.qrow, j0, d.V, qv);
    }
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) {
        const bool in = j0 + e < d.V;
        p[e] = in ? target_prob(l[e], d.M, d.S) : 0.f;
        w[e] = in ? (has_q ? fmaxf(0.f, p[e] - d.c * qv[e]) : p[e]) : 0.f;
    }
}

// The last-workgroup pattern of the fused draw and tree rounds: thread 0
// publishes its chunk totals with a release increment of the sequence's
// counter, and the workgroup that brings it to NC takes an acquire fence
// (agent scope) before anyone reads the other chunks' totals.  Only thread
// 0 fences; the workgroup barrier after it orders every thread's later
// reads.  Returns, in every thread, whether this is the last workgroup.
__device__ __forceinline__ bool arrive_last(int32_t* counter, int NC) {
    __shared__ int s_last;
    if (threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        s_last = done == NC - 1;
        if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
    return s_last;
}

// ---------------------------------------------------------------------------
// The pick, on one wave (wave 0 of the sequence's last workgroup): the sum S
// of the chunk totals, the chunk where the running sum reaches t = u S, then
// the wave of that chunk's workgroup from the wave totals the chunk pass
// left, then a rescan of that wave's 64 * kDrawPerThread tokens.  Each level
// takes the first entry with weight whose running sum reaches t, failing
// that (only through rounding) the last entry with weight.

// S, the sum of one sequence's chunk totals tot[0, NC): lanes own chunks, 64
// at a time, each window a wave scan, the windows added in order.  Every
// lane of the calling wave gets S.
__device__ __forceinline__ double chunk_total_sum(const double* tot, int NC) {
    const int lane = threadIdx.x & (kWave - 1);
    double S = 0.0;
    for (int w0 = 0; w0 < NC; w0 += kWave) {
        double own = 0.0;
        if (w0 + lane < NC) own += tot[w0 + lane];
        S += wave_last(wave_inclusive_scan(own));
    }
    return S;
}

// Where the running sum over n entries val (lane-owned, zero past the end)
// first reaches t from the offset carry: the lane and the running sum before
// it, or lane -1 when no entry with weight reaches it (*last_lane, *last_base
// then name the last entry with weight, if any).
struct Crossing {
    int lane;
    double base;
};

__device__ __forceinline__ Crossing crossing(double val, double carry, double t, int* last_lane,
                                             double* last_base, double* total) {
    const double incl = wave_inclusive_scan(val);
    const double base = carry + wave_shift_up(incl);
    *total = wave_last(incl);
    const unsigned long long reach = __ballot(val > 0.0 && base + val >= t);
    const unsigned long long any = __ballot(val > 0.0);
    if (any) {
        *last_lane = 63 - __builtin_clzll(any);
        *last_base = wave_read(base, *last_lane);
    }
    if (!reach) return {-1, 0.0};
    const int l = __builtin_ctzll(reach);
    return {l, wave_read(base, l)};
}

// The dense q of tokens [c0, c0 + kWave * kDrawPerThread) of a sparse row,
// built in s_qc by one wave: zeroed, then every entry whose id falls in the
// range merged in by unsigned max on the value's bits (values were made
// non-negative, where the bit order is the value order).  The ids go first,
// kSparseBatch 16-byte groups per lane at a time; a value is loaded only for
// an id in the range (a few per row).  One wave's LDS operations take effect
// in order, so the zeros land before the merges.
constexpr int kSparseBatch = 8;

__device__ void stage_sparse_wave(const DrawRow& d, int c0, unsigned* s_qc) {
    constexpr int n = kWave * kDrawPerThread;
    const int lane = threadIdx.x & (kWave - 1);
    for (int j = lane; j < n; j += kWave) s_qc[j] = 0u;
    auto in_range = [&](int id) {
        return id >= 0 && id < d.V && (unsigned)(id - c0) < (unsigned)n;
    };
    auto put = [&](int id, float v) { atomicMax(&s_qc[id - c0], __float_as_uint(sparse_value(v))); };
    if ((d.K & 3) == 0) {
        const int4* id4 = reinterpret_cast<const int4*>(d.qids);
        const int K4 = d.K >> 2;
        for (int j0 = 0; j0 < K4; j0 += kSparseBatch * kWave) {
            int4 ids[kSparseBatch];
#pragma unroll
            for (int u = 0; u < kSparseBatch; ++u) {
                const int j = j0 + lane + u * kWave;
                ids[u] = j < K4 ? id4[j] : make_int4(-1, -1, -1, -1);
            }
#pragma unroll
            for (int u = 0; u < kSparseBatch; ++u) {
                const int e = 4 * (j0 + lane + u * kWave);
                if (in_range(ids[u].x)) put(ids[u].x, d.qvals[e + 0]);
                if (in_range(ids[u].y)) put(ids[u].y, d.qvals[e + 1]);
                if (in_range(ids[u].z)) put(ids[u].z, d.qvals[e + 2]);
                if (in_range(ids[u].w)) put(ids[u].w, d.qvals[e + 3]);
            }
        }
    } else {
        for (int j = lane; j < d.K; j += kWave)
            if (in_range(d.qids[j])) put(d.qids[j], d.qvals[j]);
    }
}

// The inverse-CDF draw for sequence b from the chunk and wave totals.  Called
// by one whole wave; every lane returns the token.  *flags gets
// SV_DEV_FALLBACK (the residual carried no weight: drawn from p) and
// SV_DEV_NONFINITE (no finite positive total at all: token 0).  s_qc holds,
// for sparse q, kWave * kDrawPerThread words of LDS.
template <bool SPARSE>
__device__ int pick(DrawRow d, int b, int NC, const ChunkSums& cs, float u, unsigned* s_qc,
                    int* flags) {
    __shared__ double s_wv[kDrawWaves];
    const int lane = threadIdx.x & (kWave - 1);
    *flags = 0;
    const double* tot = cs.csum + (size_t)b * NC;
    const double* wtot = cs.cwave + (size_t)b * NC * kDrawWaves;
    auto fall_back = [&]() {                   // no residual mass: draw from p
        *flags = SV_DEV_FALLBACK;
        d.drop_q();
        tot = cs.psum + (size_t)b * NC;
        wtot = cs.pwave + (size_t)b * NC * kDrawWaves;
    };
    double t, before, wt = 0.0;
    int chunk;
    if (NC <= kWave) {
        // One window (V <= 262144): lane c loads chunk c's total and its wave
        // totals in the same round trip.
        double own, wv[kDrawWaves];
        auto load = [&]() {
            own = 0.0;
#pragma unroll
            for (int k = 0; k < kDrawWaves; ++k) wv[k] = 0.0;
            if (lane < NC) {
                own += tot[lane];
                const double2* src = reinterpret_cast<const double2*>(wtot + (size_t)lane * kDrawWaves);
#pragma unroll
                for (int k = 0; k < kDrawWaves; k += 2) {
                    const double2 v = src[k / 2];
                    wv[k] = v.x;
                    wv[k + 1] = v.y;
                }
            }
        };
        load();
        double incl = wave_inclusive_scan(own);
        double S = 0.0 + wave_last(incl);      // the association of chunk_total_sum
        if (!(S > 0.0)) {
            fall_back();
            load();
            incl = wave_inclusive_scan(own);
            S = 0.0 + wave_last(incl);
        }
        if (!(S > 0.0) || !(S < INFINITY)) {
            *flags |= SV_DEV_NONFINITE;
            return 0;
        }
        t = (double)u * S;
        const double base = 0.0 + wave_shift_up(incl);
        const unsigned long long reach = __ballot(own > 0.0 && base + own >= t);
        const unsigned long long any = __ballot(own > 0.0);
        chunk = reach ? __builtin_ctzll(reach) : any ? 63 - __builtin_clzll(any) : 0;
        before = wave_read(base, chunk);
        // lane k takes wave total k of the chunk, handed over through LDS
        // (one wave's LDS writes land before its later reads)
        if (lane == chunk) {
#pragma unroll
            for (int k = 0; k < kDrawWaves; ++k) s_wv[k] = wv[k];
        }
        __builtin_amdgcn_wave_barrier();
        if (lane < kDrawWaves) wt = s_wv[lane];
    } else {
        double S = chunk_total_sum(tot, NC);
        if (!(S > 0.0)) {
            fall_back();
            S = chunk_total_sum(tot, NC);
        }
        if (!(S > 0.0) || !(S < INFINITY)) {
            *flags |= SV_DEV_NONFINITE;
            return 0;
        }
        t = (double)u * S;
        int last = 0;
        double last_base = 0.0, carry = 0.0;
        chunk = -1;
        before = 0.0;
        for (int w0 = 0; w0 < NC && chunk < 0; w0 += kWave) {
            double own = 0.0, total;
            if (w0 + lane < NC) own += tot[w0 + lane];
            int ll = -1;
            double lb = 0.0;
            const Crossing x = crossing(own, carry, t, &ll, &lb, &total);
            if (ll >= 0) { last = w0 + ll; last_base = lb; }
            if (x.lane >= 0) { chunk = w0 + x.lane; before = x.base; }
            carry += total;
        }
        if (chunk < 0) { chunk = last; before = last_base; }
        if (lane < kDrawWaves) wt = wtot[(size_t)chunk * kDrawWaves + lane];
    }

    // The wave of the chunk's workgroup.
    int wl = 0;
    double wb = before, total;
    const Crossing x = crossing(wt, before, t, &wl, &wb, &total);
    const int sub = x.lane >= 0 ? x.lane : wl;
    const double base_w = x.lane >= 0 ? x.base : wb;

    // Its tokens, rescanned in order.
    const int c0 = chunk * kDrawChunk + sub * kWave * kDrawPerThread;
    if (SPARSE && d.has_q()) stage_sparse_wave(d, c0, s_qc);
    const int j0 = c0 + lane * kDrawPerThread;
    float w[kDrawPerThread], p[kDrawPerThread];
    draw_weights<SPARSE>(d, j0, s_qc, c0, w, p);
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < kDrawPerThread; ++e) mine += (double)w[e];
    const double base = base_w + wave_shift_up(wave_inclusive_scan(mine));
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
    // Lanes cover ascending tokens: the first candidate sits in the lowest
    // lane that has one, the last token with weight in the highest.
    const unsigned long long hit = __ballot(y != INT_MAX), pos = __ballot(ylast >= 0);
    if (hit) return __builtin_amdgcn_readlane(y, __builtin_ctzll(hit));
    return pos ? __builtin_amdgcn_readlane(ylast, 63 - __builtin_clzll(pos)) : c0;
}

}  // namespace

}  // namespace sv
