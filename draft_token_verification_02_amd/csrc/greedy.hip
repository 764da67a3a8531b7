// Greedy (match) verification after the LM head.
//
// Sources: the maxstudionews.com article 1664 on multi-token prediction for
// the on-device Gemini Nano model, the paragraph on the draft / verify split
// (the large model checks every drafted token in one pass, keeps those equal
// to its own prediction and resumes from the first disagreement) and the one
// on bit-identical output; "推测解码" (world.lapla.si/zh/specdec), sections
// 先让小模型猜 (guess-then-check in its greedy form) and 留下对的，换掉错的
// (stop at the first failed draft, emit the target's own token there, or the
// bonus token when all pass).
//
// The target's prediction at a row is its greedy token: the largest logit,
// lowest id on ties.  The LM head already left one (largest logit, lowest id)
// candidate per row and workgroup, so one 256-thread workgroup per sequence
// merges those (32 threads per row), compares the gamma drafts in one wave
// ballot and writes the emitted tokens -- the logits themselves are not read.

#include "sv_common.h"

namespace sv {

namespace {

constexpr int kRowThreads = 32;
constexpr int kRowsPerPass = kBlock / kRowThreads;
constexpr int kBatch = 2;                 // 16-byte loads per thread per batch and array

__global__ __launch_bounds__(kBlock) void greedy_kernel(
    const float* __restrict__ part_max, const int32_t* __restrict__ part_arg, int NP, int NPs,
    const int32_t* __restrict__ draft, int gamma, int V, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ n_accepted, int32_t* __restrict__ target_tokens,
    int32_t* __restrict__ status) {
    __shared__ int s_tok[SV_MAX_GAMMA + 1];
    const int b = blockIdx.x;
    const int g1 = gamma + 1;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    // The draft ids, loaded before the partial merge they do not depend on.
    int x = -1;
    if (wave == 0 && lane < gamma) x = draft[(size_t)b * gamma + lane];

    const int sub = threadIdx.x % kRowThreads;
    const int grp = threadIdx.x / kRowThreads;
    for (int i0 = 0; i0 < g1; i0 += kRowsPerPass) {
        const int i = i0 + grp;
        float v = -INFINITY;
        int a = -1;
        if (i < g1) {
            // 16-byte loads (rows of NPs, a multiple of 4), a batch of
            // kBatch per thread issued before any is merged: one memory
            // round trip for up to 32 * 4 * kBatch partials.
            const size_t r = (size_t)b * g1 + i;
            const float4* pm = reinterpret_cast<const float4*>(part_max + r * NPs);
            const int4* pa = reinterpret_cast<const int4*>(part_arg + r * NPs);
            const int n4 = (NP + 3) / 4;
            for (int j0 = 0; j0 < n4; j0 += kBatch * kRowThreads) {
                float4 mv[kBatch];
                int4 av[kBatch];
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int jj = j0 + sub + u * kRowThreads;
                    mv[u] = jj < n4 ? pm[jj] : make_float4(0.f, 0.f, 0.f, 0.f);
                    av[u] = jj < n4 ? pa[jj] : make_int4(-1, -1, -1, -1);
                }
#pragma unroll
                for (int u = 0; u < kBatch; ++u) {
                    const int j = 4 * (j0 + sub + u * kRowThreads);   // entries past NP are padding
                    if (j + 0 < NP) arg_merge(v, a, mv[u].x, av[u].x);
                    if (j + 1 < NP) arg_merge(v, a, mv[u].y, av[u].y);
                    if (j + 2 < NP) arg_merge(v, a, mv[u].z, av[u].z);
                    if (j + 3 < NP) arg_merge(v, a, mv[u].w, av[u].w);
                }
            }
        }
#pragma unroll
        for (int off = 1; off < kRowThreads; off <<= 1) {
            const float v2 = __shfl_xor(v, off);
            const int a2 = __shfl_xor(a, off);
            arg_merge(v, a, v2, a2);
        }
        if (sub == 0 && i < g1) s_tok[i] = a;
    }
    __syncthreads();

    if (wave == 0) {
        const int t = lane < g1 ? s_tok[lane] : -1;
        const bool valid = lane < gamma && x >= 0 && x < V;
        const bool keep = valid && x == t;
        const unsigned long long kept = __ballot(keep);
        const unsigned long long badm = __ballot(lane < gamma && !valid);
        const int n = min(__builtin_ctzll(~kept), gamma);
        const int yn = s_tok[n];
        if (lane < g1) {
            out_tokens[(size_t)b * g1 + lane] = lane < n ? x : (lane == n ? (yn >= 0 ? yn : 0) : -1);
            if (target_tokens) target_tokens[(size_t)b * g1 + lane] = t;
        }
        if (lane == 0) {
            n_accepted[b] = n;
            status[b] = (badm ? SV_DEV_BAD_DRAFT : 0) | (yn < 0 ? SV_DEV_NONFINITE : 0);
        }
    }
}

}  // namespace

hipError_t launch_greedy(const float* part_max, const int32_t* part_arg, int NP, int NPs, int B,
                         int gamma, int V, const int32_t* draft, int32_t* out_tokens,
                         int32_t* n_accepted, int32_t* target_tokens, int32_t* status,
                         hipStream_t stream) {
    greedy_kernel<<<dim3(B), dim3(kBlock), 0, stream>>>(part_max, part_arg, NP, NPs, draft, gamma, V,
                                                        out_tokens, n_accepted, target_tokens, status);
    return hipGetLastError();
}

}  // namespace sv
