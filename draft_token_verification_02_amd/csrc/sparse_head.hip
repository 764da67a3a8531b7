// The drafter's clustered sparse LM head: q over the tokens of the k best
// clusters only, exactly 0 elsewhere.
//
// Source: "多詞元預測視覺化指南" (gemma.gh.miniasp.com), section 高效嵌入器:
// the tokens' embeddings are grouped into clusters, each with an embedding of
// its own; the hidden state times that small table gives one logit per
// cluster, the most likely clusters are chosen, and token logits are formed
// only for the tokens of the chosen clusters.  q is their softmax.
//
// Four launches, N hidden rows (one per drafted position):
//   scores_kernel  cluster logits h . centroid^T, [N][C] fp32.  The table is
//                  small (C x d bf16, 6 MB at C = 2048, d = 1536), so each
//                  workgroup takes 16 centroids and splits k over its eight
//                  waves (v_mfma_f32_16x16x32_bf16, centroids as A, hidden
//                  rows as B), each issuing its k steps' loads together, and
//                  sums them through LDS in wave order: C / 16 workgroups of
//                  one memory round trip each instead of a few long ones.
//   topk_kernel    per row, the k largest cluster logits (ties to the lower
//                  cluster id) by an exact 4-pass radix select on order-
//                  preserving keys held in registers (1024 threads, one LDS
//                  histogram, a DPP scan, two barriers per pass), then the
//                  chosen clusters in ascending id and their members in the
//                  members table's order: the row's K = k * M token ids.
//   gather_kernel  token logits h . W[id] for the K ids of each row: W rows
//                  gathered straight into the MFMA A operand (16 tokens per
//                  fragment, 16 contiguous bytes per lane), the hidden row as
//                  B; one softmax partial (max, sum exp) per workgroup.
//   qfinal_kernel  q = exp(l - max) / sum exp from the row's partials.
// Member ids outside [0, V) are dropped: their slots hold id -1 (the padding
// id of the sparse-q verify entry points) and q = 0.

#include "sv_common.h"

namespace sv {

namespace {

constexpr int kSplit = 8;            // waves splitting k in scores_kernel
constexpr int kGT = 2;               // 16-token fragments per wave in gather_kernel
constexpr int kGWaves = 4;           // waves per gather workgroup
constexpr int kGU = 8;               // k-steps loaded per batch in gather_kernel

// ---------------------------------------------------------------------------
// Cluster logits for 16 centroids x 16 * MT hidden rows per workgroup; kSplit
// waves take every kSplit-th 32-wide k step and issue up to kSB steps' loads
// at once (at d = 1536 all of them: one memory round trip per wave), then the
// waves' sums are added in wave order through LDS.
template <int MT>
__global__ __launch_bounds__(kSplit * kWave) void scores_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ cent, int N, int d, int C,
    float* __restrict__ scores) {
    constexpr int kSB = 8;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15, kg = lane >> 4;
    const int c0 = blockIdx.x * kLmTile;
    const int n0 = blockIdx.y * kLmTile * MT;

    const uint16_t* ap = cent + (size_t)min(c0 + r16, C - 1) * d + kg * 8;
    const uint16_t* bp[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) bp[m] = h + (size_t)min(n0 + m * kLmTile + r16, N - 1) * d + kg * 8;

    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nstep = (d + 31) / 32;
    const u32x4 zero{0u, 0u, 0u, 0u};
    for (int ks0 = wave; ks0 < nstep; ks0 += kSplit * kSB) {
        u32x4 a[kSB], bb[kSB][MT];
#pragma unroll
        for (int u = 0; u < kSB; ++u) {
            const int ks = ks0 + u * kSplit;
            const bool ok = ks < nstep && ks * 32 + kg * 8 < d;    // d is a multiple of 8
            a[u] = ok ? *reinterpret_cast<const u32x4*>(ap + ks * 32) : zero;
#pragma unroll
            for (int m = 0; m < MT; ++m)
                bb[u][m] = ok ? *reinterpret_cast<const u32x4*>(bp[m] + ks * 32) : zero;
        }
#pragma unroll
        for (int u = 0; u < kSB; ++u)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a[u]), __builtin_bit_cast(bf16x8, bb[u][m]), acc[m],
                    0, 0, 0);
    }

    __shared__ f32x4 red[kSplit][MT][kWave];
#pragma unroll
    for (int m = 0; m < MT; ++m) red[wave][m][lane] = acc[m];
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            f32x4 sum = red[0][m][lane];
#pragma unroll
            for (int w = 1; w < kSplit; ++w) sum += red[w][m][lane];
            // lane holds D[centroid 4*kg + i][hidden row r16] of fragment m
            const int n = n0 + m * kLmTile + r16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = c0 + 4 * kg + i;
                if (n < N && c < C) scores[(size_t)n * C + c] = sum[i];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Top-k of the cluster logits, one 1024-thread workgroup per row.  Thread t
// holds the keys of clusters t*P .. t*P+P-1 in registers (P = ceil(C/1024) <=
// 8), so the chosen clusters come out in ascending id by thread order.
constexpr int kTkBlock = 1024;
constexpr int kTkWaves = kTkBlock / kWave;
constexpr int kTkPer = (SV_HEAD_MAX_CLUSTERS + kTkBlock - 1) / kTkBlock;

// Wave-wide inclusive sum on DPP lane moves (row_shr 1, 2, 4, 8, then the
// row broadcasts 15 and 31); lanes without a source add 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_add_src(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}
__device__ __forceinline__ int wave_scan_int(int v) {
    v += dpp_add_src<0x111, 0xf>(v);
    v += dpp_add_src<0x112, 0xf>(v);
    v += dpp_add_src<0x114, 0xf>(v);
    v += dpp_add_src<0x118, 0xf>(v);
    v += dpp_add_src<0x142, 0xa>(v);
    v += dpp_add_src<0x143, 0xc>(v);
    return v;
}

// A key whose unsigned order is the float order (-0 and +0 equal, NaN lowest).
__device__ __forceinline__ unsigned order_key(float f) {
    if (f != f) return 0u;
    if (f == 0.f) f = 0.f;
    const unsigned u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kTkBlock) void topk_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ members, int C, int M, int k,
    int V, int32_t* __restrict__ q_ids, int32_t* __restrict__ clusters) {
    __shared__ int s_hist[256];
    __shared__ int s_sel[SV_HEAD_MAX_CLUSTERS];
    __shared__ int s_wsum[kTkWaves];
    __shared__ int s_digit, s_above;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n = blockIdx.x;
    const float* row = scores + (size_t)n * C;
    const int P = (C + kTkBlock - 1) / kTkBlock;
    const int cb = tid * P;
    unsigned key[kTkPer];
    bool valid[kTkPer];
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
        valid[j] = j < P && cb + j < C;
        key[j] = valid[j] ? order_key(row[cb + j]) : 0u;
    }
    if (tid < 256) s_hist[tid] = 0;
    __syncthreads();

    // The k-th largest key, 8 bits at a time from the top: count the keys
    // that match the digits found so far by their next digit (one LDS
    // histogram); wave 0 scans the 256 counts from the highest digit (four
    // per lane, a DPP scan), takes the digit where the count at or above it
    // reaches the number still needed, and clears the histogram.  Two
    // barriers per pass.
    unsigned prefix = 0u, pmask = 0u;
    int need = k;
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
#pragma unroll
        for (int j = 0; j < kTkPer; ++j)
            if (valid[j] && (key[j] & pmask) == prefix) atomicAdd(&s_hist[(key[j] >> shift) & 255u], 1);
        __syncthreads();
        if (wave == 0) {
            int cnt[4], tot = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) { cnt[i] = s_hist[255 - 4 * lane - i]; tot += cnt[i]; }
            const int incl = wave_scan_int(tot);
            const int before = incl - tot;                 // keys with a higher digit
            if (before < need && incl >= need) {
                int run = before;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (run + cnt[i] >= need) { s_digit = 255 - 4 * lane - i; s_above = run; break; }
                    run += cnt[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) s_hist[255 - 4 * lane - i] = 0;
        }
        __syncthreads();
        prefix |= (unsigned)s_digit << shift;
        pmask |= 255u << shift;
        need -= s_above;
    }

    // Chosen: every key above the threshold, and the first `need` keys equal
    // to it in cluster order.  One exclusive scan of (count above, count
    // equal), packed in 16-bit halves, places them in ascending id.
    int ngt = 0, neq = 0;
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
        ngt += valid[j] && key[j] > prefix;
        neq += valid[j] && key[j] == prefix;
    }
    const int mine = (ngt << 16) | neq;
    const int incl = wave_scan_int(mine);
    if (lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    int before = 0;
#pragma unroll
    for (int w = 0; w < kTkWaves; ++w)
        if (w < wave) before += s_wsum[w];
    const int packed = before + incl - mine;
    const int gt_before = packed >> 16, eq_before = packed & 0xffff;
    int pos = gt_before + min(eq_before, need), eqs = eq_before;
#pragma unroll
    for (int j = 0; j < kTkPer; ++j) {
        const bool chosen = valid[j] && (key[j] > prefix || (key[j] == prefix && eqs++ < need));
        if (chosen) s_sel[pos++] = cb + j;
    }
    __syncthreads();

    if (clusters)
        for (int j = tid; j < k; j += kTkBlock) clusters[(size_t)n * k + j] = s_sel[j];
    const int K = k * M;
    int32_t* out = q_ids + (size_t)n * K;
    // The members of the chosen clusters, 8 per thread in flight at a time.
    for (int e0 = 0; e0 < K; e0 += 8 * kTkBlock) {
        int id[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + tid + u * kTkBlock;
            id[u] = -1;
            if (e < K) {
                const int jj = e / M, m = e - jj * M;
                id[u] = members[(size_t)s_sel[jj] * M + m];
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int e = e0 + tid + u * kTkBlock;
            if (e < K) out[e] = id[u] >= 0 && id[u] < V ? id[u] : -1;
        }
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kGWaves * kWave) void gather_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ W,
    const int32_t* __restrict__ q_ids, int K, int d, float* __restrict__ tl,
    float* __restrict__ pmax, float* __restrict__ psum, int G) {
    constexpr int kTok = kGT * kLmTile;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15, kg = lane >> 4;
    const int n = blockIdx.y;
    const int tok0 = (blockIdx.x * kGWaves + wave) * kTok;
    const int32_t* ids = q_ids + (size_t)n * K;

    // A rows: the gathered W rows of this lane's fragment row (padding and
    // dropped ids read row 0; their results are discarded).
    const uint16_t* ap[kGT];
#pragma unroll
    for (int t = 0; t < kGT; ++t) {
        const int j = tok0 + t * kLmTile + r16;
        const int id = j < K ? ids[j] : -1;
        ap[t] = W + (size_t)(id >= 0 ? id : 0) * d + kg * 8;
    }
    // B: the hidden row in every column.
    const uint16_t* bp = h + (size_t)n * d + kg * 8;

    f32x4 acc[kGT];
#pragma unroll
    for (int t = 0; t < kGT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nstep = (d + 31) / 32;
    const u32x4 zero{0u, 0u, 0u, 0u};
    for (int ks0 = 0; ks0 < nstep; ks0 += kGU) {
        u32x4 a[kGU][kGT], b[kGU];
#pragma unroll
        for (int u = 0; u < kGU; ++u) {
            const int ks = ks0 + u;
            const bool ok = ks < nstep && ks * 32 + kg * 8 < d;
#pragma unroll
            for (int t = 0; t < kGT; ++t)
                a[u][t] = ok ? *reinterpret_cast<const u32x4*>(ap[t] + ks * 32) : zero;
            b[u] = ok ? *reinterpret_cast<const u32x4*>(bp + ks * 32) : zero;
        }
#pragma unroll
        for (int u = 0; u < kGU; ++u)
#pragma unroll
            for (int t = 0; t < kGT; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a[u][t]), __builtin_bit_cast(bf16x8, b[u]), acc[t],
                    0, 0, 0);
    }

    // Lane (r16, kg) holds D[token 4*kg + i][column r16]; the columns are
    // equal, so column 0's lanes write.  Their running (max, sum exp).
    float m = -INFINITY, s = 0.f;
    if (r16 == 0) {
        float v[kGT][4];
#pragma unroll
        for (int t = 0; t < kGT; ++t) {
            const int j0 = tok0 + t * kLmTile + 4 * kg;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = j0 + i;
                const bool live = j < K && ids[j] >= 0;
                v[t][i] = live ? acc[t][i] : -INFINITY;
                if (j < K) tl[(size_t)n * K + j] = v[t][i];
                m = fmaxf(m, v[t][i]);
            }
        }
        if (m != -INFINITY) {
#pragma unroll
            for (int t = 0; t < kGT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (v[t][i] != -INFINITY) s += expf(v[t][i] - m);
        }
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
        lse_merge(m, s, m2, s2);
    }
    __shared__ float s_m[kGWaves], s_s[kGWaves];
    if (lane == 0) { s_m[wave] = m; s_s[wave] = s; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float mm = -INFINITY, ss = 0.f;
#pragma unroll
        for (int w = 0; w < kGWaves; ++w) lse_merge(mm, ss, s_m[w], s_s[w]);
        pmax[(size_t)n * G + blockIdx.x] = mm;
        psum[(size_t)n * G + blockIdx.x] = ss;
    }
}

// ---------------------------------------------------------------------------
constexpr int kQPer = 4;                       // values per thread in qfinal_kernel

__global__ __launch_bounds__(kBlock) void qfinal_kernel(
    const float* __restrict__ tl, const float* __restrict__ pmax, const float* __restrict__ psum,
    int G, int K, float* __restrict__ q_vals) {
    __shared__ float s_m, s_s;
    const int n = blockIdx.y;
    if (threadIdx.x < kWave) {
        float m = -INFINITY, s = 0.f;
        for (int g = threadIdx.x; g < G; g += kWave)
            lse_merge(m, s, pmax[(size_t)n * G + g], psum[(size_t)n * G + g]);
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
            lse_merge(m, s, m2, s2);
        }
        if (threadIdx.x == 0) { s_m = m; s_s = s; }
    }
    __syncthreads();
    const float m = s_m, s = s_s;
    const int jb = blockIdx.x * kBlock * kQPer + threadIdx.x;
    float l[kQPer];
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
        const int j = jb + u * kBlock;
        l[u] = j < K ? tl[(size_t)n * K + j] : -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
        const int j = jb + u * kBlock;
        if (j < K) q_vals[(size_t)n * K + j] = s > 0.f && l[u] != -INFINITY ? expf(l[u] - m) / s : 0.f;
    }
}

}  // namespace

// Workspace of the sparse head: cluster scores [N][C], token logits [N][K],
// gather partials (max, sum exp) [N][G] each.
HeadLayout make_head_layout(int N, int C, int K) {
    HeadLayout L;
    L.G = (K + kGT * kLmTile * kGWaves - 1) / (kGT * kLmTile * kGWaves);
    size_t off = 0;
    L.scores = off; off = align_up(off + (size_t)N * C * sizeof(float), 256);
    L.tl = off;     off = align_up(off + (size_t)N * K * sizeof(float), 256);
    L.pmax = off;   off = align_up(off + (size_t)N * L.G * sizeof(float), 256);
    L.psum = off;   off = align_up(off + (size_t)N * L.G * sizeof(float), 256);
    L.total = off;
    return L;
}

hipError_t launch_sparse_head(const uint16_t* h, const uint16_t* W, const uint16_t* cent,
                              const int32_t* members, int N, int d, int V, int C, int M, int k,
                              int32_t* q_ids, float* q_vals, int32_t* clusters, void* ws,
                              hipStream_t stream) {
    const int K = k * M;
    const HeadLayout L = make_head_layout(N, C, K);
    char* base = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(base + L.scores);
    float* tl = reinterpret_cast<float*>(base + L.tl);
    float* pmax = reinterpret_cast<float*>(base + L.pmax);
    float* psum = reinterpret_cast<float*>(base + L.psum);

    const int ctiles = (C + kLmTile - 1) / kLmTile;
    const int mt = N <= 16 ? 1 : N <= 32 ? 2 : N <= 48 ? 3 : 4;
    const dim3 sg(ctiles, (N + kLmTile * mt - 1) / (kLmTile * mt)), sb(kSplit * kWave);
    switch (mt) {
        case 1: scores_kernel<1><<<sg, sb, 0, stream>>>(h, cent, N, d, C, scores); break;
        case 2: scores_kernel<2><<<sg, sb, 0, stream>>>(h, cent, N, d, C, scores); break;
        case 3: scores_kernel<3><<<sg, sb, 0, stream>>>(h, cent, N, d, C, scores); break;
        default: scores_kernel<4><<<sg, sb, 0, stream>>>(h, cent, N, d, C, scores); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    topk_kernel<<<dim3(N), dim3(kTkBlock), 0, stream>>>(scores, members, C, M, k, V, q_ids, clusters);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    gather_kernel<<<dim3(L.G, N), dim3(kGWaves * kWave), 0, stream>>>(h, W, q_ids, K, d, tl, pmax,
                                                                    psum, L.G);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    qfinal_kernel<<<dim3((K + kBlock * kQPer - 1) / (kBlock * kQPer), N), dim3(kBlock), 0, stream>>>(
        tl, pmax, psum, L.G, K, q_vals);
    return hipGetLastError();
}

}  // namespace sv
