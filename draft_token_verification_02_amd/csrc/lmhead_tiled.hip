// LM-head GEMM for many rows: logits = hidden . W^T with R > 64, plus one
// softmax partial and one greedy candidate (largest logit, lowest id) per
// (row, 256-entry vocab block).
//
// Source: "推测解码" (world.lapla.si/zh/specdec), sections 先让小模型猜 and
// 几段话一起写 -- one read of the target's weights serves every drafted
// position of every sequence in the batch; "多詞元預測視覺化指南", section
// 高效嵌入器 -- the LM head multiplies hidden states by the tied embedding
// matrix W [V][d].
//
// Shape of the work.  At R in the hundreds the GEMM does 2*R flops per two
// bytes of W, at or above the MI355X ridge (~312 flop/byte), so it is bound by
// the MFMA pipes rather than HBM.  Each workgroup computes a 256 (vocab) x
// 256 (hidden row) block with v_mfma_f32_16x16x32_bf16: 8 waves in a 2 x 4
// arrangement, 128 x 64 per wave (8 x 4 fragments, accumulators in 128
// registers).  K is walked in tiles of 64: both operand tiles are loaded from
// global memory into registers one tile ahead, written to LDS (rows padded
// to 144 bytes so the 16-byte fragment reads of 8 lanes hit distinct banks),
// and read back as MFMA fragments; one barrier per tile.  W is the A operand
// (vocab = M) and the hidden rows the B operand, so each lane ends with four
// consecutive vocab entries of one hidden row -- a 16-byte logits store.
//
// Block order.  Workgroups are dispatched round-robin over the 8 XCDs; the
// block index is remapped so that each XCD receives a contiguous run of the
// (vocab block, row block) sequence with row blocks fastest.  The row blocks
// that share a W tile then run together on one XCD and the tile comes from
// HBM once, from that XCD's L2 after.

#include "sv_common.h"

namespace sv {

namespace {

constexpr int kTV = kLmTiledVocab;   // vocab rows per workgroup
constexpr int kTR = 256;             // hidden rows per workgroup
constexpr int kTK = 64;              // k per LDS tile
constexpr int kTWaves = 8;
constexpr int kTThreads = kTWaves * kWave;
constexpr int kWaveV = 128, kWaveR = 64;           // per-wave block
constexpr int kFV = kWaveV / kLmTile, kFR = kWaveR / kLmTile;   // 8 x 4 fragments
constexpr int kRowBytes = kTK * 2 + 16;            // padded LDS row: 144 bytes
constexpr int kXcds = 8;

static_assert((kTV / kWaveV) * (kTR / kWaveR) == kTWaves, "wave grid");

// One K tile of both operands: 256 rows x 64 bf16 each = 2048 chunks of 16
// bytes per operand, 4 per thread.
struct Stage {
    u32x4 w[4], h[4];
};

__device__ __forceinline__ void load_stage(Stage& s, const uint16_t* __restrict__ W,
                                           const uint16_t* __restrict__ H, int v0, int r0, int k0,
                                           int V, int R, int d) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = threadIdx.x + j * kTThreads;      // chunk 0..2047
        const int row = c >> 3, col = (c & 7) * 8;      // 8 chunks per 64-element row
        const int k = k0 + col;
        const int v = min(v0 + row, V - 1);             // past the end: a valid row, never stored
        const int r = min(r0 + row, R - 1);
        if (k < d) {
            s.w[j] = *reinterpret_cast<const u32x4*>(W + (size_t)v * d + k);
            s.h[j] = *reinterpret_cast<const u32x4*>(H + (size_t)r * d + k);
        } else {
            s.w[j] = u32x4{0u, 0u, 0u, 0u};
            s.h[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
}

__device__ __forceinline__ void store_stage(const Stage& s, char* lw, char* lh) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = threadIdx.x + j * kTThreads;
        const int row = c >> 3, col = c & 7;
        *reinterpret_cast<u32x4*>(lw + row * kRowBytes + col * 16) = s.w[j];
        *reinterpret_cast<u32x4*>(lh + row * kRowBytes + col * 16) = s.h[j];
    }
}

__global__ __launch_bounds__(kTThreads) void lmhead_tiled_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, int R, int d, int V,
    int nvb, int nrb, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int32_t* __restrict__ part_arg, int NPs,
    int32_t* __restrict__ counters, int n_counters) {
    // LDS: two stages of (W tile, hidden tile), each 256 rows x 144 bytes.
    __shared__ __attribute__((aligned(16))) char lds[2][2][kTV * kRowBytes];
    __shared__ float s_max[kTV / kWaveV][kTR];
    __shared__ float s_sum[kTV / kWaveV][kTR];
    __shared__ float s_av[kTV / kWaveV][kTR];
    __shared__ int s_ai[kTV / kWaveV][kTR];

    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counters; i += gridDim.x * blockDim.x)
        counters[i] = 0;

    // XCD-aware block order: hardware block b runs on XCD b % 8; give each XCD
    // a contiguous run of logical blocks, row blocks fastest.
    const int nblocks = nvb * nrb;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nblocks) return;          // padding blocks of the rounded-up grid
    const int vb = logical / nrb, rb = logical % nrb;
    const int v0 = vb * kTV, r0 = rb * kTR;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wv = wave & 1, wr = wave >> 1;            // 2 (vocab) x 4 (rows) waves
    const int r16 = lane & 15, kg = lane >> 4;

    f32x4 acc[kFV][kFR];
#pragma unroll
    for (int a = 0; a < kFV; ++a)
#pragma unroll
        for (int b = 0; b < kFR; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (d + kTK - 1) / kTK;
    Stage st;
    load_stage(st, W, hidden, v0, r0, 0, V, R, d);
    store_stage(st, lds[0][0], lds[0][1]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_stage(st, W, hidden, v0, r0, (kt + 1) * kTK, V, R, d);
        const char* lw = lds[cur][0] + (wv * kWaveV + r16) * kRowBytes + kg * 16;
        const char* lh = lds[cur][1] + (wr * kWaveR + r16) * kRowBytes + kg * 16;
#pragma unroll
        for (int ks = 0; ks < kTK / 32; ++ks) {
            u32x4 fa[kFV], fb[kFR];
#pragma unroll
            for (int a = 0; a < kFV; ++a)
                fa[a] = *reinterpret_cast<const u32x4*>(lw + a * kLmTile * kRowBytes + ks * 64);
#pragma unroll
            for (int b = 0; b < kFR; ++b)
                fb[b] = *reinterpret_cast<const u32x4*>(lh + b * kLmTile * kRowBytes + ks * 64);
#pragma unroll
            for (int a = 0; a < kFV; ++a)
#pragma unroll
                for (int b = 0; b < kFR; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, fa[a]), __builtin_bit_cast(bf16x8, fb[b]),
                        acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) store_stage(st, lds[cur ^ 1][0], lds[cur ^ 1][1]);
        __syncthreads();
    }

    // Epilogue: lane holds D[vocab 4*kg + i][row r16] of each fragment; its
    // ids rise with a and i, so a strict '>' keeps the first maximum.  No
    // logits buffer: only the partials are written.
    const bool vec_store = (V & 3) == 0;
#pragma unroll
    for (int b = 0; b < kFR; ++b) {
        const int rl = wr * kWaveR + b * kLmTile + r16;     // row within the block
        const int r = r0 + rl;
        const bool row_ok = r < R;
        float* lrow = logits ? logits + (size_t)(row_ok ? r : 0) * V : nullptr;
        float mx = -INFINITY, av = -INFINITY;
        int ai = -1;
#pragma unroll
        for (int a = 0; a < kFV; ++a) {
            const int v = v0 + wv * kWaveV + a * kLmTile + kg * 4;
            if (row_ok && lrow) {
                if (vec_store) {
                    if (v < V) *reinterpret_cast<float4*>(lrow + v) =
                        make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (v + i < V) lrow[v + i] = acc[a][b][i];
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (v + i < V) {
                    mx = fmaxf(mx, acc[a][b][i]);
                    if (acc[a][b][i] > av) { av = acc[a][b][i]; ai = v + i; }
                }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
#pragma unroll
        for (int off = 16; off < kWave; off <<= 1) {
            const float av2 = __shfl_xor(av, off);
            const int ai2 = __shfl_xor(ai, off);
            arg_merge(av, ai, av2, ai2);
        }
        float sm = 0.f;
        if (mx != -INFINITY) {
#pragma unroll
            for (int a = 0; a < kFV; ++a) {
                const int v = v0 + wv * kWaveV + a * kLmTile + kg * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (v + i < V) sm += expf(acc[a][b][i] - mx);
            }
        }
        sm += __shfl_xor(sm, 16);
        sm += __shfl_xor(sm, 32);
        if (kg == 0) { s_max[wv][rl] = mx; s_sum[wv][rl] = sm; s_av[wv][rl] = av; s_ai[wv][rl] = ai; }
    }
    __syncthreads();
    if (threadIdx.x < kTR && r0 + (int)threadIdx.x < R) {
        const int rl = threadIdx.x;
        float m = -INFINITY, s = 0.f, av = -INFINITY;
        int ai = -1;
#pragma unroll
        for (int w = 0; w < kTV / kWaveV; ++w) {
            lse_merge(m, s, s_max[w][rl], s_sum[w][rl]);
            arg_merge(av, ai, s_av[w][rl], s_ai[w][rl]);
        }
        part_max[(size_t)(r0 + rl) * NPs + vb] = m;
        part_sum[(size_t)(r0 + rl) * NPs + vb] = s;
        part_arg[(size_t)(r0 + rl) * NPs + vb] = ai;
    }
}

}  // namespace

hipError_t launch_lmhead_tiled(const uint16_t* hidden, const uint16_t* W, int R, int d, int V,
                               float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                               int NPs, int32_t* counters, int n_counters, hipStream_t stream) {
    const int nvb = lmhead_tiled_partials(V);
    const int nrb = (R + kTR - 1) / kTR;
    const int nblocks = nvb * nrb;
    const int grid = (nblocks + kXcds - 1) / kXcds * kXcds;
    lmhead_tiled_kernel<<<dim3(grid), dim3(kTThreads), 0, stream>>>(
        hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    return hipGetLastError();
}

}  // namespace sv
