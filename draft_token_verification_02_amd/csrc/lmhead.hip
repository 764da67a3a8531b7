// LM-head GEMM of the verification step: logits = hidden . W^T for all
// B*(gamma+1) rows in one pass over W, plus per-tile softmax partials.
//
// Source: "推测解码" (world.lapla.si/zh/specdec), section 先让小模型猜 -- the
// target scores every drafted position plus one in a single read of its
// weights; "多詞元預測視覺化指南", section 高效嵌入器 -- the LM head multiplies
// hidden states by the tied embedding matrix W [V][d].
//
// Shape of the work.  With R <= 64 rows the GEMM moves ~2 bytes of W per
// 2*R flops, far below the MI355X ridge (~312 flop/byte), so it is bound by
// streaming W from HBM.  Each W byte is loaded exactly once, straight into
// the A operand of v_mfma_f32_16x16x32_bf16 (16 vocab rows x 32 k per
// fragment, 16 contiguous bytes per lane); the hidden rows are the B operand
// (16 rows x 32 k), re-read from L2 once per fragment step and shared by the
// wave's four vocab fragments.  K is a pure reduction, so both operands use
// the same (lane group, element) -> k mapping and no reordering is needed.
//
// Each wave owns 64 vocab rows for the full K range, so there is no barrier
// in the main loop.  Loads run one stage (2 k-steps x 4 fragments = 8 KB per
// wave) ahead of the MFMAs.  The epilogue stores the fp32 logits and reduces
// each row's 256-entry workgroup slice to a (max, sum exp) partial for the
// softmax, so no later pass needs to re-read the logits to normalise them.

#include "sv_common.h"

namespace sv {

namespace {

constexpr int T = kLmTilesPerWave;
constexpr int U = 2;                 // k-steps (of 32) per pipeline stage

template <int MT>
struct Frags {
    uint4 w[U][T];
    uint4 h[U][MT];
};

template <int MT>
__device__ __forceinline__ void load_stage(Frags<MT>& f, const uint4* const (&wp)[T],
                                           const uint4* const (&hp)[MT], int step) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int off = (step + u) * 4;   // 32 bf16 = 4 uint4 per k-step
#pragma unroll
        for (int t = 0; t < T; ++t) f.w[u][t] = wp[t][off];
#pragma unroll
        for (int m = 0; m < MT; ++m) f.h[u][m] = hp[m][off];
    }
}

template <int MT>
__device__ __forceinline__ void mma_stage(const Frags<MT>& f, f32x4 (&acc)[T][MT]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, f.w[u][t]), __builtin_bit_cast(bf16x8, f.h[u][m]),
                    acc[t][m], 0, 0, 0);
}

// One k-step of 32 with the k range cut at d (d is a multiple of 8, so each
// lane's 8-element group is either wholly inside or wholly outside).
template <int MT>
__device__ __forceinline__ void masked_step(const uint4* const (&wp)[T], const uint4* const (&hp)[MT],
                                            int step, int kg, int d, f32x4 (&acc)[T][MT]) {
    const bool in = step * 32 + kg * 8 < d;
    const uint4 zero = make_uint4(0, 0, 0, 0);
    uint4 w[T], h[MT];
#pragma unroll
    for (int t = 0; t < T; ++t) w[t] = in ? wp[t][step * 4] : zero;
#pragma unroll
    for (int m = 0; m < MT; ++m) h[m] = in ? hp[m][step * 4] : zero;
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m)
            acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, w[t]), __builtin_bit_cast(bf16x8, h[m]), acc[t][m], 0, 0, 0);
}

template <int MT>
__global__ __launch_bounds__(kBlock) void lmhead_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, int row0, int rows,
    int d, int V, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int NP) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int r16 = lane & 15;      // fragment row this lane loads (A: vocab, B: hidden)
    const int kg = lane >> 4;       // 8-element k group of this lane
    const int v_wave = blockIdx.x * kLmVocabPerBlock + wave * (T * kLmTile);

    // Per-lane fragment row pointers; rows past the end are clamped to a valid
    // row and their results are never stored.
    const uint4* wp[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int v = min(v_wave + t * kLmTile + r16, V - 1);
        wp[t] = reinterpret_cast<const uint4*>(W + (size_t)v * d) + kg;
    }
    const uint4* hp[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int r = row0 + min(m * kLmTile + r16, rows - 1);
        hp[m] = reinterpret_cast<const uint4*>(hidden + (size_t)r * d) + kg;
    }

    f32x4 acc[T][MT];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Full stages of U k-steps, ping-pong between two register buffers.
    const int nstage = d / (32 * U);
    if (nstage > 0) {
        Frags<MT> fa, fb;
        load_stage<MT>(fa, wp, hp, 0);
        for (int s = 0; s < nstage; s += 2) {
            if (s + 1 < nstage) load_stage<MT>(fb, wp, hp, (s + 1) * U);
            mma_stage<MT>(fa, acc);
            if (s + 2 < nstage) load_stage<MT>(fa, wp, hp, (s + 2) * U);
            if (s + 1 < nstage) mma_stage<MT>(fb, acc);
        }
    }
    // Remaining k-steps (d not a multiple of 64), each cut at d.
    const int nstep = (d + 31) / 32;
    for (int step = nstage * U; step < nstep; ++step) masked_step<MT>(wp, hp, step, kg, d, acc);

    // Epilogue.  Lane holds D[vocab 4*kg + i][hidden row r16] of each fragment.
    __shared__ float s_max[kBlock / kWave][MT * kLmTile];
    __shared__ float s_sum[kBlock / kWave][MT * kLmTile];
    const bool vec_store = (V & 3) == 0;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int rr = m * kLmTile + r16;                // row within this pass
        const bool row_ok = rr < rows;
        float* lrow = logits + (size_t)(row0 + (row_ok ? rr : 0)) * V;
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int v = v_wave + t * kLmTile + kg * 4;
            if (row_ok) {
                if (vec_store) {
                    if (v < V) *reinterpret_cast<float4*>(lrow + v) =
                        make_float4(acc[t][m][0], acc[t][m][1], acc[t][m][2], acc[t][m][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (v + i < V) lrow[v + i] = acc[t][m][i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (v + i < V) mx = fmaxf(mx, acc[t][m][i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        float sm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int v = v_wave + t * kLmTile + kg * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (v + i < V) sm += expf(acc[t][m][i] - mx);
            }
        }
        sm += __shfl_xor(sm, 16);
        sm += __shfl_xor(sm, 32);
        if (kg == 0) {
            s_max[wave][rr] = mx;
            s_sum[wave][rr] = sm;
        }
    }
    __syncthreads();
    if (threadIdx.x < MT * kLmTile && (int)threadIdx.x < rows) {
        const int rr = threadIdx.x;
        float m = -INFINITY, s = 0.f;
#pragma unroll
        for (int w = 0; w < kBlock / kWave; ++w) lse_merge(m, s, s_max[w][rr], s_sum[w][rr]);
        part_max[(size_t)(row0 + rr) * NP + blockIdx.x] = m;
        part_sum[(size_t)(row0 + rr) * NP + blockIdx.x] = s;
    }
}

}  // namespace

// Enqueue the LM-head stage: one launch per group of up to 64 hidden rows.
hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, int R, int d, int V,
                         float* logits, float* part_max, float* part_sum, int NP,
                         hipStream_t stream) {
    for (int row0 = 0; row0 < R; row0 += kLmRowsPerPass) {
        const int rows = min(kLmRowsPerPass, R - row0);
        const int mt = (rows + kLmTile - 1) / kLmTile;
        dim3 grid(NP), block(kBlock);
        switch (mt) {
            case 1: lmhead_kernel<1><<<grid, block, 0, stream>>>(hidden, W, row0, rows, d, V, logits, part_max, part_sum, NP); break;
            case 2: lmhead_kernel<2><<<grid, block, 0, stream>>>(hidden, W, row0, rows, d, V, logits, part_max, part_sum, NP); break;
            case 3: lmhead_kernel<3><<<grid, block, 0, stream>>>(hidden, W, row0, rows, d, V, logits, part_max, part_sum, NP); break;
            default: lmhead_kernel<4><<<grid, block, 0, stream>>>(hidden, W, row0, rows, d, V, logits, part_max, part_sum, NP); break;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sv
