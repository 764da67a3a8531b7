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
// R > 128: blocks of 256 vocab rows x TR = 64 FR hidden rows, eight waves in
// a 2 (vocab) x 4 (rows) grid, each 128 vocab rows x 16 FR hidden rows
// (8 x FR fragments).  Both operands go from memory straight into LDS
// (global_load_lds_dwordx4: 16 bytes per lane, no registers on the way)
// through a ring of S stages of one 32-wide k step each.
//
// Ping-pong.  Waves 0-3 (group A) and 4-7 (group B) share the SIMDs, one of
// each per SIMD, and take turns: while one group issues its MFMAs for a k
// step the other reads its next fragments from LDS, and two barriers per k
// step (X, Y) swap the roles, so a SIMD's matrix unit always has a wave with
// operands ready feeding it.  Each wave issues its share of the ring's
// copies between its own MFMAs (one after each of the first fragment rows):
// a copy that stalls in the memory pipeline then holds up only a wave whose
// MFMAs already keep the matrix unit busy.  Per k step t:
//   A: MFMAs(t) + copies of t+S-1 | wait own copies of t+1 | X | read frags(t+1) | Y
//   B: read frags(t) | wait own copies of t+1 | X | MFMAs(t) + copies of t+S-1 | Y
// Stage u % S holds step u.  Before X_t every wave has waited for its copies
// of step t+1, so after X_t the stage of t+1 is whole (A reads it in Q_t, B
// in P_{t+1}).  The copies of step t+S-1 go to stage (t-1) % S, which both
// groups finished reading before step t began (A in Q_{t-2}, waited before
// Y_{t-2}; B in P_{t-1}, waited before X_{t-1}).  Measured at R = 1280,
// d = 4096 (per k step, s_memtime in a probe build): 40 MFMAs take ~680
// cycles, a group's 13 fragment reads ~300-480.
//
// Stage layout: the 256 W rows, then the TR hidden rows, 64 bytes (32 bf16)
// each; chunk g of row r sits in slot g ^ ((r >> 1) & 3), which rocprofv3's
// SQ_LDS_BANK_CONFLICT counts as conflict-free for the fragment reads on
// gfx950 (g ^ ((r >> 2) & 3) counted conflicts on half the active cycles).
// A copy instruction writes 1 KB of the stage (lane i to byte 16 i), so each
// lane loads the global chunk that belongs at its slot.
constexpr int kBigK = 32;                          // k per stage: one MFMA k step
constexpr int kBigRowBytes = kBigK * 2;            // 64
constexpr int kBigWV = 2, kBigWR = 4, kBigFV = 8;  // wave grid and vocab fragments per wave
constexpr int kBigNW = kBigWV * kBigWR;            // 8 waves
constexpr int kBigNT = kBigNW * kWave;

template <int FR>
struct BigCfg {
    static constexpr int TV = kBigWV * kBigFV * kLmTile;        // 256 vocab rows per block
    static constexpr int TR = kBigWR * FR * kLmTile;            // hidden rows per block
    static constexpr int kStageBytes = (TV + TR) * kBigRowBytes;
    static constexpr int NI = (TV + TR) * (kBigRowBytes / 16) / kWave;   // 1 KB copies per stage
    static constexpr int NIW = (NI + kBigNW - 1) / kBigNW;               // per wave and stage
    static_assert((TV + TR) % 16 == 0, "whole 1 KB copies");
};

// vmcnt helper (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): wait until at most N vector-memory operations of this wave
// are outstanding, leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// lgkmcnt(0): every LDS read of this wave has returned.
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

template <int FR, int S, bool ARG>
__global__ __launch_bounds__(kBigNT) void lmhead_big_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, int R, int d, int V,
    int nvb, int nrb, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int32_t* __restrict__ part_arg, int NPs,
    int32_t* __restrict__ counters, int n_counters) {
    using C = BigCfg<FR>;
    constexpr int TV = C::TV, TR = C::TR, NI = C::NI, NIW = C::NIW;
    constexpr int WV = kBigWV, FV = kBigFV, NW = kBigNW;
    static_assert(TV == kTV, "256 vocab rows per block: one softmax partial column each");
    static_assert(S == 4, "ring depth");
    // One array per stage, so that the compiler can tell the stage a
    // fragment read uses from the stages copies are filling (with a single
    // array it waits for every copy in flight before each read).
    __shared__ __attribute__((aligned(1024))) char st0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st1[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st2[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st3[C::kStageBytes];
    __shared__ float s_max[WV][TR];
    __shared__ float s_sum[WV][TR];
    __shared__ float s_av[WV][TR];
    __shared__ int s_ai[WV][TR];

    // XCD-aware block order: hardware block b runs on XCD b % 8; give each XCD
    // a contiguous run of logical blocks, row blocks fastest, so the row
    // blocks sharing a W tile run together and take it from one L2.
    const int nblocks = nvb * nrb;
    const int per_xcd = (nblocks + kXcds - 1) / kXcds;
    const int logical = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;
    if (logical >= nblocks) return;          // padding blocks of the rounded-up grid
    const int vb = logical / nrb, rb = logical % nrb;
    const int v0 = vb * TV, r0 = rb * TR;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wv = wave % WV, wr = wave / WV;           // group A: wr 0-1, group B: wr 2-3
    const bool group_b = wave >= NW / 2;
    const int r16 = lane & 15, kg = lane >> 4;

    // This wave's copies: instruction j = wave + m * NW of the stage covers
    // chunks 64 j .. 64 j + 63, lane i chunk 64 j + i: row c / 4, slot c % 4,
    // holding k-chunk g = slot ^ ((row >> 1) & 3) of that row.  Rows past V
    // (or R) copy the last valid row; their results are never stored.  When
    // NI is not a multiple of NW a wave's last j may pass NI: it repeats its
    // previous copy (same bytes to the same place), so every wave issues NIW
    // copies per step and the vmcnt accounting is the same on every wave.
    const uint16_t* src[NIW];
    int dst[NIW];
    // row = 16 j + lane / 4 with 16 j a multiple of 8, so (row >> 1) & 3 = (lane >> 3) & 3
    const int goff = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
        const int j = wave + m * NW < NI ? wave + m * NW : wave + (m - 1) * NW;
        const int row = j * 16 + (lane >> 2);
        src[m] = (row < TV ? W + (size_t)min(v0 + row, V - 1) * d
                           : hidden + (size_t)min(r0 + row - TV, R - 1) * d) + goff;
        dst[m] = j * 1024;
    }

    const int nk = (d + kBigK - 1) / kBigK;
    const bool ragged = d % kBigK != 0;       // the last step has chunks past the end of a row
    auto stage = [&](int s) -> char* { return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3; };
    // Copies of step t (t >= nk: a repeat of the last step, into a stage no
    // step reads again, so that every step issues the same copies).  A chunk
    // past the end of a row copies the row's first chunk instead; the
    // fragment lanes holding it are zeroed after the read.
    auto copy_k = [&](int t) {
        t = t < nk ? t : nk - 1;
        const int k0 = t * kBigK;
        return (!ragged || k0 + goff < d) ? k0 : -goff;
    };
    auto copy_one = [&](int m, int kk, char* st) {
        __builtin_amdgcn_global_load_lds(
            (void*)(src[m] + kk), (__attribute__((address_space(3))) void*)(st + dst[m]), 16, 0, 0);
    };
    auto copy = [&](int t, char* st) {
        const int kk = copy_k(t);
#pragma unroll
        for (int m = 0; m < NIW; ++m) copy_one(m, kk, st);
    };

    f32x4 acc[FV][FR];
#pragma unroll
    for (int a = 0; a < FV; ++a)
#pragma unroll
        for (int b = 0; b < FR; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragment reads: lane (r16, kg) reads 16 bytes of row r16 of each
    // fragment at k-chunk kg; every fragment's rows start at a multiple of
    // 16, so the row's swizzle is (r16 >> 1) & 3 for all of them.
    const int sw = (kg ^ ((r16 >> 1) & 3)) * 16;
    const int aoff = (wv * FV * kLmTile + r16) * kBigRowBytes + sw;
    const int boff = (TV + wr * FR * kLmTile + r16) * kBigRowBytes + sw;
    u32x4 fa[FV], fb[FR];
    auto read_frags = [&](const char* st) {
#pragma unroll
        for (int a = 0; a < FV; ++a)
            fa[a] = *reinterpret_cast<const u32x4*>(st + aoff + a * kLmTile * kBigRowBytes);
#pragma unroll
        for (int b = 0; b < FR; ++b)
            fb[b] = *reinterpret_cast<const u32x4*>(st + boff + b * kLmTile * kBigRowBytes);
    };
    // The reads have returned; k-chunk kg of step t past the end of the rows
    // (last step, d not a multiple of 32) must contribute 0.
    auto finish_frags = [&](int t) {
        wait_lgkmcnt0();
        if (ragged && t == nk - 1 && t * kBigK + kg * 8 >= d) {
#pragma unroll
            for (int a = 0; a < FV; ++a) fa[a] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int b = 0; b < FR; ++b) fb[b] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // The step's MFMAs, fragment row by fragment row, with this wave's copies
    // of step t (into stage st) issued one after each of the first NIW rows:
    // a copy that has to wait for the memory pipeline then stalls this wave
    // while its MFMAs already issued keep the matrix unit busy.
    static_assert(NIW <= FV, "one copy per fragment row at most");
    auto mfmas_copy = [&](int t, char* st) {
        const int kk = copy_k(t);
#pragma unroll
        for (int a = 0; a < FV; ++a) {
#pragma unroll
            for (int b = 0; b < FR; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, fa[a]), __builtin_bit_cast(bf16x8, fb[b]),
                    acc[a][b], 0, 0, 0);
            if (a < NIW) copy_one(a, kk, st);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Each group issues its copies of step t+S-1 during its own MFMAs of
    // step t, into stage (t-1) % S, which both groups finished reading before
    // Y_{t-1} (A, in Q_{t-2}) and X_{t-1} (B, in P_{t-1}).  Before X_t each
    // wave needs its copies of step t+1 complete: group A issued them in
    // P_{t-2} and has those of t+2 and t+3 (P_{t-1}, P_t) after them; group B
    // in Q_{t-2}, with only those of t+2 (Q_{t-1}) after them.
    // Copies outstanding when a wave's copies of step t+1 are complete, at
    // X_t: those issued during step t-1, and for group A (whose MFMA phase
    // comes first) those of step t.
    constexpr int kWaitA = (S - 2) * NIW;
    constexpr int kWaitB = (S - 3) * NIW;
    if (!group_b) {
        // Group A.  Prologue: copies of steps 0 .. S-2; step 0 whole; its fragments.
#pragma unroll
        for (int t = 0; t < S - 1; ++t) copy(t, stage(t));
        wait_vmcnt<(S - 2) * NIW>();
        __builtin_amdgcn_s_barrier();
        read_frags(st0);
        finish_frags(0);
        for (int t0 = 0; t0 < nk; t0 += S) {
#pragma unroll
            for (int h = 0; h < S; ++h) {
                const int t = t0 + h;
                if (t >= nk) break;
                mfmas_copy(t + S - 1, stage((h + S - 1) % S));    // P_t
                wait_vmcnt<kWaitA>();
                __builtin_amdgcn_s_barrier();                      // X_t
                __builtin_amdgcn_sched_barrier(0);
                read_frags(stage((h + 1) % S));                    // Q_t
                finish_frags(t + 1);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();                      // Y_t
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // Group B.  Prologue: copies of steps 0 .. S-2; step 0 whole.
#pragma unroll
        for (int t = 0; t < S - 1; ++t) copy(t, stage(t));
        wait_vmcnt<(S - 2) * NIW>();
        __builtin_amdgcn_s_barrier();
        for (int t0 = 0; t0 < nk; t0 += S) {
#pragma unroll
            for (int h = 0; h < S; ++h) {
                const int t = t0 + h;
                if (t >= nk) break;
                read_frags(stage(h));                              // P_t
                finish_frags(t);
                wait_vmcnt<kWaitB>();
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();                      // X_t
                __builtin_amdgcn_sched_barrier(0);
                mfmas_copy(t + S - 1, stage((h + S - 1) % S));    // Q_t
                __builtin_amdgcn_s_barrier();                      // Y_t
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    wait_vmcnt<0>();                          // the trailing repeat copies

    // Epilogue: lane holds D[vocab 4*kg + i][row r16] of each fragment, ids
    // rising with (a, i).  Per fragment row b the lane stores its 32 logits
    // (16-byte stores, the two fragments of a 128-byte line back to back),
    // takes their maximum by a tree, the row's maximum over the four k-groups
    // (lanes 16 apart), the first id holding it (independent compares against
    // compile-time offsets; the lowest id of the row's four lanes), and the
    // sum of exp(x - max) by the hardware exp2 into four independent sums.
    // NaN never wins the maximum (fmaxf) nor the argmax (NaN == max is
    // false); a row block past V masks its missing ids to -inf and keeps them
    // out of the argmax.
    const bool vec_store = (V & 3) == 0;
    const bool inside = v0 + TV <= V;
    constexpr int kNoId = 0x7fffffff;
#pragma unroll
    for (int b = 0; b < FR; ++b) {
        const int rl = wr * FR * kLmTile + b * kLmTile + r16;     // row within the block
        const int r = r0 + rl;
        const bool row_ok = r < R;
        const int vl = v0 + wv * FV * kLmTile + kg * 4;             // id of this lane's (a = 0, i = 0)
        float* lrow = logits ? logits + (size_t)(row_ok ? r : 0) * V : nullptr;
        if (row_ok && lrow) {
#pragma unroll
            for (int a = 0; a < FV; ++a) {
                const int v = vl + a * kLmTile;
                if (vec_store) {
                    if (inside || v < V) *reinterpret_cast<f32x4*>(lrow + v) = acc[a][b];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (v + i < V) lrow[v + i] = acc[a][b][i];
                }
            }
        }
        float x[FV * 4];
#pragma unroll
        for (int a = 0; a < FV; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                x[a * 4 + i] = (inside || vl + a * kLmTile + i < V) ? acc[a][b][i] : -INFINITY;
        float mt[FV * 2];
#pragma unroll
        for (int e = 0; e < FV * 2; ++e) mt[e] = fmaxf(x[2 * e], x[2 * e + 1]);
#pragma unroll
        for (int w = FV; w >= 1; w >>= 1)
#pragma unroll
            for (int e = 0; e < w; ++e) mt[e] = fmaxf(mt[e], mt[e + w]);
        float mx = mt[0];
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // first id of the maximum, as an offset a * 16 + i from vl, scanned
        // from the back (greedy candidates; skipped when nobody reads them)
        int ai = kNoId;
        if constexpr (ARG) {
            int off = kNoId;
#pragma unroll
            for (int e = FV * 4 - 1; e >= 0; --e)
                off = (x[e] == mx && (inside || vl + (e >> 2) * kLmTile + (e & 3) < V))
                          ? (e >> 2) * kLmTile + (e & 3) : off;
            ai = (mx == -INFINITY || off == kNoId) ? kNoId : vl + off;
            ai = min(ai, __shfl_xor(ai, 16));
            ai = min(ai, __shfl_xor(ai, 32));
        }
        float sm4[4] = {0.f, 0.f, 0.f, 0.f};
        if (mx != -INFINITY) {
#pragma unroll
            for (int e = 0; e < FV * 4; ++e) sm4[e & 3] += exp2_scaled(x[e] - mx);
        }
        float sm = (sm4[0] + sm4[1]) + (sm4[2] + sm4[3]);
        sm += __shfl_xor(sm, 16);
        sm += __shfl_xor(sm, 32);
        if (kg == 0) {
            s_max[wv][rl] = mx;
            s_sum[wv][rl] = sm;
            s_av[wv][rl] = mx;
            s_ai[wv][rl] = ai == kNoId ? -1 : ai;
        }
    }
    __syncthreads();
    for (int rl = threadIdx.x; rl < TR; rl += kBigNT) {
        if (r0 + rl >= R) break;
        float m = -INFINITY, s = 0.f, av = -INFINITY;
        int ai = -1;
#pragma unroll
        for (int w = 0; w < WV; ++w) {
            lse_merge(m, s, s_max[w][rl], s_sum[w][rl]);
            if (ARG) arg_merge(av, ai, s_av[w][rl], s_ai[w][rl]);
        }
        part_max[(size_t)(r0 + rl) * NPs + vb] = m;
        part_sum[(size_t)(r0 + rl) * NPs + vb] = s;
        if (ARG) part_arg[(size_t)(r0 + rl) * NPs + vb] = ai;
    }
    // The per-sequence counters of the stage-2 kernels start at zero (after
    // the main loop, so these stores never sit in the copies' vmcnt queue).
    for (int i = logical * kBigNT + threadIdx.x; i < n_counters; i += nblocks * kBigNT)
        counters[i] = 0;
}


// ---------------------------------------------------------------------------
// 64 < R <= 128: 256 x 128 blocks, W straight into registers, hidden rows in LDS.

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
        if (part_arg) part_arg[(size_t)(r0 + rl) * NPs + vb] = ai;
    }
}


template <int FR>
hipError_t launch_big(const uint16_t* hidden, const uint16_t* W, int R, int d, int V,
                      float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                      int NPs, int32_t* counters, int n_counters, hipStream_t stream) {
    using C = BigCfg<FR>;
    const int nvb = (V + C::TV - 1) / C::TV;
    const int nrb = (R + C::TR - 1) / C::TR;
    const int nblocks = nvb * nrb;
    const int grid = (nblocks + kXcds - 1) / kXcds * kXcds;
    if (part_arg)
        lmhead_big_kernel<FR, 4, true><<<dim3(grid), dim3(kBigNT), 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters,
            n_counters);
    else
        lmhead_big_kernel<FR, 4, false><<<dim3(grid), dim3(kBigNT), 0, stream>>>(
            hidden, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters,
            n_counters);
    return hipGetLastError();
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
    // The row-block height (64 FR rows) that pads R least, ties to the taller
    // block, whose W tile then serves more rows: R = 320 runs one block of
    // 320 rows, R = 1280 four.
    int FR = 5;
    for (int fr : {4, 3, 2})
        if ((R + 64 * fr - 1) / (64 * fr) * (64 * fr) < (R + 64 * FR - 1) / (64 * FR) * (64 * FR)) FR = fr;
    switch (FR) {
        case 5: return launch_big<5>(hidden, W, R, d, V, logits, part_max, part_sum, part_arg, NPs,
                                     counters, n_counters, stream);
        case 4: return launch_big<4>(hidden, W, R, d, V, logits, part_max, part_sum, part_arg, NPs,
                                     counters, n_counters, stream);
        case 3: return launch_big<3>(hidden, W, R, d, V, logits, part_max, part_sum, part_arg, NPs,
                                     counters, n_counters, stream);
        default: return launch_big<2>(hidden, W, R, d, V, logits, part_max, part_sum, part_arg, NPs,
                                      counters, n_counters, stream);
    }
}

}  // namespace sv
