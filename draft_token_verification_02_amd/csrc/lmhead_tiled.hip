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
// Shape of the work.  The GEMM does 2*R flops per two bytes of W: below the
// MI355X ridge (~312 flop/byte) for R up to a few hundred, above it at
// R = 1280.  Both kernels use v_mfma_f32_16x16x32_bf16 with W as the A
// operand (vocab = M) and the hidden rows as B, so each lane ends with four
// consecutive vocab entries of one hidden row -- a 16-byte logits store.
//
// 64 < R <= 128 (lmhead_mid_kernel): W-bandwidth bound.  A workgroup of four
// waves computes a 256 (vocab) x 128 (row) block, each wave 64 vocab rows x
// all 128 rows (4 x 8 fragments); up to R = 96 the block is 96 rows (4 x 6
// fragments), since the hidden tile copied every K tile takes its share of
// the same load path as W.  The operands travel differently:
//   * W goes from memory straight into the MFMA A registers -- each lane
//     loads 16 contiguous bytes of one vocab row per 32-wide k step, the
//     fragment layout itself -- kept 8 k-steps ahead in a register ring
//     whose slots are compile-time constants (a straight-line loop body), so
//     each step waits only for its own loads;
//   * the hidden rows, shared by every wave, are copied from memory straight
//     into a four-stage LDS ring (global_load_lds_dwordx4), three 64-wide K
//     tiles ahead, with one explicit wait and one barrier per tile.
// Staging only the small operand in LDS keeps LDS traffic low, and W never
// waits behind the hidden tile's loads in the in-order vmcnt queue.
//
// R > 128 (lmhead_big_kernel): MFMA bound at R = 1280.  Blocks of 256 vocab
// entries x TR rows, TR = 128, 192 or 256 -- whichever leaves the fewest
// padded rows (R = 320 runs two 192-row blocks instead of two 256-row ones,
// 4.8 rather than 7.2 padded MFMA columns per computed one) -- 8 waves each;
// both operands staged through registers into LDS per 64-wide K tile
// (XOR-swizzled 128-byte rows, so fragment reads and stage writes hit
// distinct banks), one tile ahead.  At R = 1280 the 256-row block halves the L2
// traffic per flop of a 128-row block, which is what bounds that case.

// Block order.  Workgroups are dispatched round-robin over the 8 XCDs; the
// block index is remapped so that each XCD receives a contiguous run of the
// (vocab block, row block) sequence with row blocks fastest.  The row blocks
// that share a W tile then run together on one XCD and the tile comes from
// HBM once, from that XCD's L2 after.

#include "sv_common.h"

namespace sv {

namespace {

constexpr int kTV = kLmTiledVocab;   // vocab rows per workgroup (256)
constexpr int kTK = 64;              // k per LDS tile
constexpr int kTThreads = 4 * kWave;
constexpr int kRowBytes = kTK * 2 + 16;            // padded LDS row: 144 bytes
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// R > 128: 256 x TR blocks (TR = 128, 192 or 256 rows, whichever pads R
// least), 8 waves of (16 FV) x (16 FR), both operands staged in LDS.
constexpr int kBigWaves = 8;
constexpr int kBigThreads = kBigWaves * kWave;

// One K tile of both operands: 256 W rows and TR hidden rows x 64 bf16 =
// 8 chunks of 16 bytes per row, 4 (W) and TR / 64 (hidden) per thread.
template <int TR>
struct BigStage {
    u32x4 w[4], h[TR / 64];
};

template <int TR>
__device__ __forceinline__ void big_load_stage(BigStage<TR>& s, const uint16_t* __restrict__ W,
                                               const uint16_t* __restrict__ H, int v0, int r0,
                                               int k0, int V, int R, int d) {
    auto load = [&](const uint16_t* __restrict__ M, int base, int lim, int c) {
        const int row = c >> 3, col = (c & 7) * 8;      // 8 chunks per 64-element row
        const int k = k0 + col;
        const int x = min(base + row, lim - 1);         // past the end: a valid row, never stored
        return k < d ? *reinterpret_cast<const u32x4*>(M + (size_t)x * d + k) : u32x4{0u, 0u, 0u, 0u};
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) s.w[j] = load(W, v0, V, threadIdx.x + j * kBigThreads);
#pragma unroll
    for (int j = 0; j < TR / 64; ++j) s.h[j] = load(H, r0, R, threadIdx.x + j * kBigThreads);
}

// LDS rows of 128 bytes with chunk g of row r in slot g ^ (r & 7): the
// 16-byte fragment reads of 8 consecutive rows at one chunk, and the stage
// writes of a row's 8 chunks, then hit distinct banks.  (Rows padded to 144
// bytes instead left 37% of the LDS-active cycles as bank-conflict cycles in
// rocprofv3's SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE at R = 1280.)
constexpr int kBigRowBytes = kTK * 2;

template <int TR>
__device__ __forceinline__ void big_store_stage(const BigStage<TR>& s, char* lw, char* lh) {
    auto store = [&](char* l, int c, const u32x4& v) {
        const int row = c >> 3;
        *reinterpret_cast<u32x4*>(l + row * kBigRowBytes + ((c & 7) ^ (row & 7)) * 16) = v;
    };
#pragma unroll
    for (int j = 0; j < 4; ++j) store(lw, threadIdx.x + j * kBigThreads, s.w[j]);
#pragma unroll
    for (int j = 0; j < TR / 64; ++j) store(lh, threadIdx.x + j * kBigThreads, s.h[j]);
}

template <int TR, int WV, int FV, int FR>
__global__ __launch_bounds__(kBigThreads) void lmhead_big_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, int R, int d, int V,
    int nvb, int nrb, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int32_t* __restrict__ part_arg, int NPs,
    int32_t* __restrict__ counters, int n_counters) {
    constexpr int kWaveV = FV * kLmTile, kWaveR = FR * kLmTile;
    constexpr int WR = kBigWaves / WV;
    static_assert(WV * kWaveV == kTV && WR * kWaveR == TR && TR % 64 == 0, "wave grid");
    constexpr int kFV = FV, kFR = FR;
    // LDS: two stages of the W tile (256 rows) and the hidden tile (TR rows),
    // 144-byte rows.
    __shared__ __attribute__((aligned(16))) char ldsw[2][kTV * kBigRowBytes];
    __shared__ __attribute__((aligned(16))) char ldsh[2][TR * kBigRowBytes];
    __shared__ float s_max[WV][TR];
    __shared__ float s_sum[WV][TR];
    __shared__ float s_av[WV][TR];
    __shared__ int s_ai[WV][TR];

    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counters; i += gridDim.x * blockDim.x)
        counters[i] = 0;

    // XCD-aware block order: hardware block b runs on XCD b % 8; give each XCD
    // a contiguous run of logical blocks, row blocks fastest.
    const int nblocks = nvb * nrb;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nblocks) return;          // padding blocks of the rounded-up grid
    const int vb = logical / nrb, rb = logical % nrb;
    const int v0 = vb * kTV, r0 = rb * TR;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wv = wave % WV, wr = wave / WV;          // WV (vocab) x WR (rows) waves
    const int r16 = lane & 15, kg = lane >> 4;

    f32x4 acc[kFV][kFR];
#pragma unroll
    for (int a = 0; a < kFV; ++a)
#pragma unroll
        for (int b = 0; b < kFR; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (d + kTK - 1) / kTK;
    // K tiles from an offset of the block's own (see lmhead_mid_kernel).
    const int rot = (int)(((unsigned)vb * 2654435761u >> 16) % (unsigned)nk);
    auto ktile = [&](int kt) { const int t = kt + rot; return (t >= nk ? t - nk : t) * kTK; };
    BigStage<TR> st;
    big_load_stage<TR>(st, W, hidden, v0, r0, ktile(0), V, R, d);
    big_store_stage<TR>(st, ldsw[0], ldsh[0]);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) big_load_stage<TR>(st, W, hidden, v0, r0, ktile(kt + 1), V, R, d);
        // (fragment rows differ by multiples of 16, so every fragment of a
        // lane shares the row's swizzle r16 & 7)
        const char* lw = ldsw[cur] + (wv * kWaveV + r16) * kBigRowBytes;
        const char* lh = ldsh[cur] + (wr * kWaveR + r16) * kBigRowBytes;
#pragma unroll
        for (int ks = 0; ks < kTK / 32; ++ks) {
            const int off = ((ks * 4 + kg) ^ (r16 & 7)) * 16;
            u32x4 fa[kFV], fb[kFR];
#pragma unroll
            for (int a = 0; a < kFV; ++a)
                fa[a] = *reinterpret_cast<const u32x4*>(lw + a * kLmTile * kBigRowBytes + off);
#pragma unroll
            for (int b = 0; b < kFR; ++b)
                fb[b] = *reinterpret_cast<const u32x4*>(lh + b * kLmTile * kBigRowBytes + off);
            // Every fragment read is issued before the first MFMA: left to
            // itself the compiler reuses one register quad for the A
            // fragments and waits out each read in turn (about 8% slower).
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < kFV; ++a)
#pragma unroll
                for (int b = 0; b < kFR; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, fa[a]), __builtin_bit_cast(bf16x8, fb[b]),
                        acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) big_store_stage<TR>(st, ldsw[cur ^ 1], ldsh[cur ^ 1]);
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
    if (threadIdx.x < TR && r0 + (int)threadIdx.x < R) {
        const int rl = threadIdx.x;
        float m = -INFINITY, s = 0.f, av = -INFINITY;
        int ai = -1;
#pragma unroll
        for (int w = 0; w < WV; ++w) {
            lse_merge(m, s, s_max[w][rl], s_sum[w][rl]);
            arg_merge(av, ai, s_av[w][rl], s_ai[w][rl]);
        }
        part_max[(size_t)(r0 + rl) * NPs + vb] = m;
        part_sum[(size_t)(r0 + rl) * NPs + vb] = s;
        part_arg[(size_t)(r0 + rl) * NPs + vb] = ai;
    }
}


// ---------------------------------------------------------------------------
// 64 < R <= 128: 256 x 128 blocks, W straight into registers, hidden rows in LDS.
// s_waitcnt vmcnt(N), the other counters untouched (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The pipelined path keeps four hidden-tile stages in LDS.
constexpr int kStages = 4;

// vmcnt to wait for before reading tile kt's stage, counted in this wave's
// vector-memory operations issued after that tile's copies (issued S - 1
// tiles earlier): the copies and A refills of the S - 2 tiles in between,
// but not the refills of the copy's own tile.  h = -1: a tile of the main
// loop (every tile copies CHD chunks and refills 2 * FV registers); h >= 0:
// tile h of the last group, where only tile 0 still copies and only the
// k-steps 2h + s with 2h + s + U < 2S still refill.
template <int S, int U, int CHD, int FV>
constexpr int tail_wait(int h) {
    auto ops = [](int t) {                    // operations of last-group tile t
        int n = t == 0 ? CHD : 0;
        for (int s = 0; s < 2; ++s) n += (2 * t + s + U < 2 * S) ? FV : 0;
        return n;
    };
    const int main_ops = CHD + 2 * FV;
    if (h < 0) return (S - 2) * main_ops;
    int n = 0;
    if (h <= S - 2) {
        n = (S - 2 - h) * main_ops;
        for (int t = 0; t < h; ++t) n += ops(t);
    } else {
        for (int t = 1; t <= S - 2; ++t) n += ops(t);
    }
    return n;
}

template <int FV, int FR, int WV, int WR, int U, bool FAST>
__global__ __launch_bounds__(WV * WR * kWave) void lmhead_mid_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, int R, int d, int V,
    int nvb, int nrb, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int32_t* __restrict__ part_arg, int NPs,
    int32_t* __restrict__ counters, int n_counters) {
    constexpr int TR = kLmTile * FR * WR;             // rows per workgroup
    constexpr int kWaveV = kLmTile * FV;
    constexpr int kWaveR = kLmTile * FR;
    constexpr int NW = WV * WR;                       // waves
    constexpr int NT = NW * kWave;                    // threads
    constexpr int CH = TR * (kTK / 8) / NT;           // 16-byte hidden chunks per thread per tile
    static_assert(kWaveV * WV == kTV && CH >= 1, "wave grid");
    static_assert(!FAST || ((U == 2 || U == 4 || U == 8) && (FR % 8 == 0 || FR < 8)), "ring depth and fragment groups");

    // FAST: four stages of TR x 128 bytes (swizzled), each its own array so
    // that the compiler can tell a stage being read from the stages the
    // copies are filling; otherwise two buffers of TR x 144 bytes (padded).
    constexpr int kStageBytes = FAST ? TR * 128 : TR * kRowBytes;
    __shared__ __attribute__((aligned(16))) char lds0[kStageBytes];
    __shared__ __attribute__((aligned(16))) char lds1[kStageBytes];
    __shared__ __attribute__((aligned(16))) char lds2[FAST ? kStageBytes : 16];
    __shared__ __attribute__((aligned(16))) char lds3[FAST ? kStageBytes : 16];
    __shared__ float s_max[WV][TR];
    __shared__ float s_sum[WV][TR];
    __shared__ float s_av[WV][TR];
    __shared__ int s_ai[WV][TR];

    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counters; i += gridDim.x * blockDim.x)
        counters[i] = 0;

    // XCD-aware block order: hardware block b runs on XCD b % 8; give each XCD
    // a contiguous run of logical blocks, row blocks fastest.
    const int nblocks = nvb * nrb;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nblocks) return;          // padding blocks of the rounded-up grid
    const int vb = logical / nrb, rb = logical % nrb;
    const int v0 = vb * kTV, r0 = rb * TR;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wv = wave % WV, wr = wave / WV;
    const int r16 = lane & 15, kg = lane >> 4;

    // A: this lane's vocab row of each fragment (past V: a valid row, never stored)
    const uint16_t* ap[FV];
#pragma unroll
    for (int a = 0; a < FV; ++a) {
        const int v = min(v0 + wv * kWaveV + a * kLmTile + r16, V - 1);
        ap[a] = W + (size_t)v * d + kg * 8;
    }
    const int nsteps = (d + 31) / 32;
    const u32x4 zero{0u, 0u, 0u, 0u};
    u32x4 ar[U][FV];
    // The pipelined path walks k from a tile offset of its own (a hash of the
    // vocab block), wrapping: k is a pure reduction, so only the fp32
    // summation order changes, and the workgroups in flight no longer all
    // read the same offset within their rows at once (which made the time
    // depend on where the allocation of W sat in HBM).
    const int nk_all = (d + kTK - 1) / kTK;
    const int rot = FAST ? (int)(((unsigned)vb * 2654435761u >> 16) % (unsigned)nk_all) : 0;
    auto kstep = [&](int ks) {               // rotated 32-wide k step
        const int k = ks + 2 * rot;
        return k >= nsteps ? k - nsteps : k;
    };
    auto load_a = [&](int slot, int ks) {
#pragma unroll
        for (int a = 0; a < FV; ++a) {
            if (FAST) ar[slot][a] = *reinterpret_cast<const u32x4*>(ap[a] + kstep(ks) * 32);
            else ar[slot][a] = ks * 32 + kg * 8 < d ? *reinterpret_cast<const u32x4*>(ap[a] + ks * 32)
                                                    : zero;
        }
    };

    // B: the hidden tile, CH 16-byte chunks per thread (8 per 64-wide row)
    u32x4 hb[CH];
    auto load_b = [&](int k0) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = threadIdx.x + j * NT;
            const int row = c >> 3, col = (c & 7) * 8;
            const int r = min(r0 + row, R - 1);          // pad rows repeat the last row
            if (FAST || k0 + col < d) hb[j] = *reinterpret_cast<const u32x4*>(hidden + (size_t)r * d + k0 + col);
            else hb[j] = zero;
        }
    };
    auto store_b = [&](char* l) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int c = threadIdx.x + j * NT;
            const int row = c >> 3, col = c & 7;
            *reinterpret_cast<u32x4*>(l + row * kRowBytes + col * 16) = hb[j];
        }
    };

    f32x4 acc[FV][FR];
#pragma unroll
    for (int a = 0; a < FV; ++a)
#pragma unroll
        for (int b = 0; b < FR; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (d + kTK - 1) / kTK;
    auto mfma_step = [&](const char* lh, int s, int slot) {
        u32x4 fb[FR];
#pragma unroll
        for (int b = 0; b < FR; ++b)
            fb[b] = *reinterpret_cast<const u32x4*>(lh + b * kLmTile * kRowBytes + s * 64);
#pragma unroll
        for (int a = 0; a < FV; ++a)
#pragma unroll
            for (int b = 0; b < FR; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, ar[slot][a]), __builtin_bit_cast(bf16x8, fb[b]),
                    acc[a][b], 0, 0, 0);
    };
    const int lrow = (wr * kWaveR + r16) * kRowBytes + kg * 16;

    if constexpr (FAST) {
        // The hidden tile goes from memory straight into LDS
        // (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS,
        // 16 bytes per lane), into a ring of kStages tiles filled
        // kStages - 1 tiles ahead; no registers hold it on the way.  A
        // 64-wide row is 8 chunks of 16 bytes; chunk g of row r sits in slot
        // g ^ (r & 7), so the fragment reads of 8 consecutive rows at one
        // chunk hit distinct banks.  The compiler does not track these
        // copies, so each tile waits for its own explicitly: vmcnt counts
        // this wave's vector-memory operations in issue order, and the
        // straight-line loop fixes how many were issued after a tile's copy
        // (tail_wait; the A refills issued in the copy's own tile are not
        // counted, which only makes the wait stronger); a bare s_barrier then
        // makes every wave's part visible.  The loop body covers kStages
        // tiles, so stages and ring slots are compile-time constants.
        constexpr int S = kStages;
        constexpr int CHD = TR * 8 / NT;                   // copies per thread per tile
        auto stage = [&](int st) { return st == 0 ? lds0 : st == 1 ? lds1 : st == 2 ? lds2 : lds3; };
        auto copy_b = [&](int kt, int st) {
#pragma unroll
            for (int j = 0; j < CHD; ++j) {
                const int blk = j * NW + wave;               // 1 KB block of the stage
                const int c = blk * kWave + lane;
                const int row = c >> 3, g = (c & 7) ^ (row & 7);
                const int r = min(r0 + row, R - 1);          // pad rows repeat the last row
                __builtin_amdgcn_global_load_lds(
                    hidden + (size_t)r * d + (kt + rot < nk ? kt + rot : kt + rot - nk) * kTK + g * 8,
                    (__attribute__((address_space(3))) void*)(stage(st) + blk * 1024), 16, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        const int brow = (wr * kWaveR + r16) * 128;
        const int off0 = ((0 * 4 + kg) ^ (r16 & 7)) * 16, off1 = ((1 * 4 + kg) ^ (r16 & 7)) * 16;
        auto step_dma = [&](int st, int s, int slot) {
            const char* lh = stage(st) + brow + (s ? off1 : off0);
            // B fragments kFB at a time (register budget), each used by all FV
            constexpr int kFB = FR < 8 ? FR : 8;
#pragma unroll
            for (int b0 = 0; b0 < FR; b0 += kFB) {
                u32x4 fb[kFB];
#pragma unroll
                for (int b = 0; b < kFB; ++b)
                    fb[b] = *reinterpret_cast<const u32x4*>(lh + (b0 + b) * kLmTile * 128);
#pragma unroll
                for (int a = 0; a < FV; ++a)
#pragma unroll
                    for (int b = 0; b < kFB; ++b)
                        acc[a][b0 + b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, ar[slot][a]), __builtin_bit_cast(bf16x8, fb[b]),
                            acc[a][b0 + b], 0, 0, 0);
            }
        };

#pragma unroll
        for (int t = 0; t < S - 1; ++t) copy_b(t, t);
#pragma unroll
        for (int u = 0; u < U; ++u) load_a(u, u);
        int kt0 = 0;
        for (; kt0 < nk - S; kt0 += S) {
#pragma unroll
            for (int h = 0; h < S; ++h) {
                const int kt = kt0 + h;
                wait_vmcnt<tail_wait<S, U, CHD, FV>(-1)>();
                __builtin_amdgcn_s_barrier();
                copy_b(kt + S - 1, (h + S - 1) % S);
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    step_dma(h, s, (h * 2 + s) % U);
                    load_a((h * 2 + s) % U, kt * 2 + s + U);
                }
            }
        }
        // The last group: the copy for the last tile, refills only while
        // k-steps remain, then nothing.
#pragma unroll
        for (int h = 0; h < S; ++h) {
            const int kt = kt0 + h;
            if (h == 0) wait_vmcnt<tail_wait<S, U, CHD, FV>(0)>();
            else if (h == 1) wait_vmcnt<tail_wait<S, U, CHD, FV>(1)>();
            else if (h == 2) wait_vmcnt<tail_wait<S, U, CHD, FV>(2)>();
            else wait_vmcnt<tail_wait<S, U, CHD, FV>(3)>();
            __builtin_amdgcn_s_barrier();
            if (h == 0) copy_b(kt + S - 1, S - 1);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                step_dma(h, s, (h * 2 + s) % U);
                if (h * 2 + s + U < 2 * S) load_a((h * 2 + s) % U, kt * 2 + s + U);
            }
        }
    } else {
        // Any d (a multiple of 8): a two-deep ring, guarded loads.
        auto buf = [&](int i) { return i ? lds1 : lds0; };
        load_b(0);
        load_a(0, 0);
        if (1 < nsteps) load_a(1, 1);
        store_b(buf(0));
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_b((kt + 1) * kTK);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int ks = kt * 2 + s;
                if (ks < nsteps) {
                    mfma_step(buf(cur) + lrow, s, s);
                    if (ks + 2 < nsteps) load_a(s, ks + 2);
                }
            }
            if (kt + 1 < nk) store_b(buf(cur ^ 1));
            __syncthreads();
        }
    }

    // Epilogue: lane holds D[vocab 4*kg + i][row r16] of each fragment; its
    // ids rise with a and i, so a strict '>' keeps the first maximum.
    const bool vec_store = (V & 3) == 0;
#pragma unroll
    for (int b = 0; b < FR; ++b) {
        const int rl = wr * kWaveR + b * kLmTile + r16;     // row within the block
        const int r = r0 + rl;
        const bool row_ok = r < R;
        float* lrow = logits ? logits + (size_t)(row_ok ? r : 0) * V : nullptr;
        float mx = -INFINITY, av = -INFINITY;
        int ai = -1;
#pragma unroll
        for (int a = 0; a < FV; ++a) {
            const int v = v0 + wv * kWaveV + a * kLmTile + kg * 4;
            if (row_ok && lrow) {
                if (vec_store) {
                    if (v < V) __builtin_nontemporal_store(acc[a][b], reinterpret_cast<f32x4*>(lrow + v));
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
            for (int a = 0; a < FV; ++a) {
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
    for (int rl = threadIdx.x; rl < TR; rl += NT) {
        if (r0 + rl >= R) break;
        float m = -INFINITY, s = 0.f, av = -INFINITY;
        int ai = -1;
#pragma unroll
        for (int w = 0; w < WV; ++w) {
            lse_merge(m, s, s_max[w][rl], s_sum[w][rl]);
            arg_merge(av, ai, s_av[w][rl], s_ai[w][rl]);
        }
        part_max[(size_t)(r0 + rl) * NPs + vb] = m;
        part_sum[(size_t)(r0 + rl) * NPs + vb] = s;
        part_arg[(size_t)(r0 + rl) * NPs + vb] = ai;
    }
}


template <int FV, int FR, int WV, int WR, int U>
hipError_t launch_shape(const uint16_t* hidden, const uint16_t* W, int R, int d, int V,
                        float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                        int NPs, int32_t* counters, int n_counters, hipStream_t stream) {
    constexpr int TR = kLmTile * FR * WR;
    const int nvb = lmhead_tiled_partials(V);
    const int nrb = (R + TR - 1) / TR;
    const int nblocks = nvb * nrb;
    const int grid = (nblocks + kXcds - 1) / kXcds * kXcds;
    // pipelined: d a multiple of 4 tiles of 64, at least two groups of them
    if (d % (kTK * kStages) == 0 && d / (kTK * kStages) >= 2)
        lmhead_mid_kernel<FV, FR, WV, WR, U, true><<<dim3(grid), dim3(WV * WR * kWave), 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters,
            n_counters);
    else
        lmhead_mid_kernel<FV, FR, WV, WR, 2, false><<<dim3(grid), dim3(WV * WR * kWave), 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters,
            n_counters);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_lmhead_tiled(const uint16_t* hidden, const uint16_t* W, int R, int d, int V,
                               float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                               int NPs, int32_t* counters, int n_counters, hipStream_t stream) {
    // 64 < R <= 96: 96-row blocks -- the hidden tile every k step copies is
    // then 12 KB instead of 16 KB next to the same 32 KB of W.
    if (R <= 96)
        return launch_shape<4, 6, 4, 1, 8>(hidden, W, R, d, V, logits, part_max, part_sum, part_arg,
                                           NPs, counters, n_counters, stream);
    if (R <= 128)
        return launch_shape<4, 8, 4, 1, 8>(hidden, W, R, d, V, logits, part_max, part_sum, part_arg,
                                           NPs, counters, n_counters, stream);
    // The row-block height that pads R least (ties to the taller block, whose
    // W tile then serves more rows): R = 320 runs two blocks of 192 rows
    // rather than two of 256, R = 1280 five of 256.
    const int nvb = lmhead_tiled_partials(V);
    int TR = 256;
    for (int tr : {192, 128})
        if ((R + tr - 1) / tr * tr < (R + TR - 1) / TR * TR) TR = tr;
    const int nrb = (R + TR - 1) / TR;
    const int nblocks = nvb * nrb;
    const int grid = (nblocks + kXcds - 1) / kXcds * kXcds;
    const dim3 g(grid), b(kBigThreads);
    if (TR == 256)
        lmhead_big_kernel<256, 2, 8, 4><<<g, b, 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    else if (TR == 192)
        lmhead_big_kernel<192, 4, 4, 6><<<g, b, 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    else
        lmhead_big_kernel<128, 4, 4, 4><<<g, b, 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    return hipGetLastError();
}

}  // namespace sv
