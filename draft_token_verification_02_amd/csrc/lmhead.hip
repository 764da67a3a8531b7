// LM-head GEMM of the verification step: logits = hidden . W^T for all
// B*(gamma+1) rows in one pass over W, plus per-workgroup softmax and argmax
// partials.
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
// (16 rows x 32 k), re-read from L2 and shared by the T vocab fragments a
// wave works on at once.  K is a pure reduction, so both operands use the
// same (lane group, element) -> k mapping and no reordering is needed.
//
// Launch shape.  The grid is persistent: one workgroup of kLmWaves waves per
// compute unit (the register budget lets only one fit), and the vocabulary's
// groups of T fragments are dealt round-robin to all waves, so the grid
// sweeps W front to back together.  Each wave streams its groups as one
// sequence of (group, k-step) loads kept U steps ahead of the MFMAs in a
// register ring; the ring runs across group boundaries, so a group's
// epilogue (staging its fp32 logits and a running (max, sum exp) per row)
// overlaps the next group's loads.
// The workgroup reduces its running maxima and sums to one softmax partial
// per row, so no later pass has to re-read the logits to normalise them, and
// its greedy candidates to one (largest logit, lowest id) pair per row, from
// which greedy verification takes each row's argmax without the logits.

#include <type_traits>

#include "sv_common.h"

namespace sv {

namespace {

// Fragments per wave and ring depth (k-steps in flight) by hidden-row
// fragments MT, from sweeps on MI355X at d = 1536 and 4096 with the
// round-robin group order: two fragments four steps deep for one hidden
// fragment (one fragment loses once the 16 hidden rows are distinct: its
// hidden loads match its W loads byte for byte); more fragments, to share
// each hidden-row load, and shallower rings as MT grows.
template <int MT> struct LmCfg;
template <> struct LmCfg<1> { static constexpr int T = 2, U = 4; };
template <> struct LmCfg<2> { static constexpr int T = 4, U = 2; };
template <> struct LmCfg<3> { static constexpr int T = 8, U = 2; };
template <> struct LmCfg<4> { static constexpr int T = 8, U = 2; };
constexpr int kGenericU = 4;         // ring depth of the path for ragged d

// Groups of T fragments a wave stages in LDS before writing them out: a
// 32 KB stage per wave, at least one group.
template <int MT, int T>
constexpr int kStageGroups = (32768 / (MT * kLmTile * T * kLmTile * 4)) > 0
                                 ? (32768 / (MT * kLmTile * T * kLmTile * 4)) : 1;

__device__ __forceinline__ bool vec_store_ok(int V) { return (V & 3) == 0; }

// DPP quad permutations: exchange with lane ^ 1 and with lane ^ 2.
constexpr int kQuadXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);
constexpr int kQuadXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);

template <int CTRL>
__device__ __forceinline__ float quad_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int quad_i32(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Merge this lane's softmax partial (m, s) and greedy candidate (av, ai)
// with those of its partner lane in the quad.
template <int CTRL>
__device__ __forceinline__ void quad_merge(float& m, float& s, float& av, int& ai) {
    const float m2 = quad_f32<CTRL>(m), s2 = quad_f32<CTRL>(s), av2 = quad_f32<CTRL>(av);
    const int ai2 = quad_i32<CTRL>(ai);
    const float nm = fmaxf(m, m2);
    s = nm == -INFINITY ? 0.f : s * exp2_scaled(m - nm) + s2 * exp2_scaled(m2 - nm);
    m = nm;
    arg_merge(av, ai, av2, ai2);
}

// WT: W in 1 KB tiles of 16 vocab rows x 32 hidden columns (tile (i, t) at
// element (i * nstep + t) * 512, rows within it 64 bytes apart), so a
// fragment's k step is one contiguous 1 KB; otherwise [V][d] row-major.
template <int MT, int T, int U, bool FAST, bool WT>
__global__ __launch_bounds__(kLmWaves * kWave) void lmhead_kernel(
    const uint16_t* __restrict__ hidden, const uint16_t* __restrict__ W, int row0, int rows,
    int d, int V, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int32_t* __restrict__ part_arg, int NPs,
    int32_t* __restrict__ counters, int n_counters) {
    const int lane = threadIdx.x & (kWave - 1);
    // The wave index is the same on every lane; saying so keeps the wave's
    // range, cursors and branches in scalar registers, which lets the
    // compiler keep the load ring in flight across loop iterations.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int r16 = lane & 15;      // fragment row this lane loads (A: vocab, B: hidden)
    const int kg = lane >> 4;       // 8-element k group of this lane

    // The draw stage counts finished workgroups per sequence; start it at zero.
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n_counters; i += gridDim.x * blockDim.x)
        counters[i] = 0;

    // This wave's groups of T fragments: wid, wid + nwaves, wid + 2 nwaves,
    // ...  Dealt round-robin, the groups in flight across the GPU at any
    // moment are neighbours, so the whole grid sweeps W from front to back
    // in one narrow window -- the access order of a plain streaming read --
    // rather than every wave walking a range of its own (measured: 138 ->
    // 131 us at d = 1536, V = 262144 with one hidden fragment; 177 -> 172
    // us at d = 4096).
    const int ntiles = (V + kLmTile - 1) / kLmTile;
    const int ngroups = (ntiles + T - 1) / T;
    const int nwaves = gridDim.x * kLmWaves;
    const int wid = blockIdx.x * kLmWaves + wave;
    const int gb = wid, ge = ngroups, gstep = nwaves;   // groups gb, gb + gstep, ... < ge
    const int nstep = (d + 31) / 32;

    const u32x4* hp[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int r = row0 + min(m * kLmTile + r16, rows - 1);   // pad rows repeat the last row
        hp[m] = reinterpret_cast<const u32x4*>(hidden + (size_t)r * d) + kg;
    }

    // Load cursor (group lg, k-step lk) with its fragment row pointers.
    // Rows past V are clamped to a valid row; their results are never kept.
    // A lane's W chunk of k step lk is lp[t][lk * kWStep].
    constexpr int kWStep = WT ? 64 : 4;      // 16-byte units between k steps of a row
    int lg = gb, lk = 0;
    const u32x4* lp[T];
    auto set_rows = [&](int g) {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int v = min((g * T + t) * kLmTile + r16, V - 1);
            const size_t row = WT ? (size_t)(v >> 4) * nstep * 512 + (v & 15) * 32 : (size_t)v * d;
            lp[t] = reinterpret_cast<const u32x4*>(W + row) + kg;
        }
    };
    set_rows(lg);
    u32x4 wr[U][T], hr[U][MT];
    auto load = [&](int slot) {
        if (FAST || lk * 32 + kg * 8 < d) {        // lanes past d load nothing
#pragma unroll
            for (int t = 0; t < T; ++t) wr[slot][t] = lp[t][lk * kWStep];
#pragma unroll
            for (int m = 0; m < MT; ++m) hr[slot][m] = hp[m][lk * 4];
        } else {
#pragma unroll
            for (int t = 0; t < T; ++t) wr[slot][t] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int m = 0; m < MT; ++m) hr[slot][m] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto advance = [&]() {
        if (++lk == nstep) { lk = 0; lg += gstep; if (lg < ge) set_rows(lg); }
    };

    f32x4 acc[T][MT];
    auto zero_acc = [&]() {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                acc[t][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, wr[slot][t]), __builtin_bit_cast(bf16x8, hr[slot][m]),
                    acc[t][m], 0, 0, 0);
    };

    // Running softmax partial of this lane's hidden rows over its vocab
    // entries, and the running greedy candidate (largest logit, first id).
    float run_m[MT], run_s[MT], run_av[MT];
    int run_ai[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) { run_m[m] = -INFINITY; run_s[m] = 0.f; run_av[m] = -INFINITY; run_ai[m] = -1; }
    // Without a logits buffer (greedy verification needs only the partials)
    // nothing is staged or stored.
    const bool keep_logits = logits != nullptr;

    // Logits are staged per wave in LDS (kStageGroups of the wave's groups,
    // rows padded by 16 bytes so the 16-byte writes of one fragment hit
    // distinct banks) and written out when the stage is full and at the end:
    // per row, one T*64-byte segment per staged group, instead of 64-byte
    // pieces of 16 rows after every fragment.  Group k of the stage is the
    // wave's group stage_first + k * gstep.
    constexpr int kSeg = kStageGroups<MT, T> * T * kLmTile;    // floats per staged row
    constexpr int kSegPad = kSeg + 4;
    __shared__ __attribute__((aligned(16))) float stage[kLmWaves][MT * kLmTile][kSegPad];
    float (*st)[kSegPad] = stage[wave];
    int stage_first = gb, staged = 0;
    // The stage is written as one flat run of 16-byte pieces over (row,
    // vocab), kWave pieces per store instruction: each lane reads
    // kFlushBatch pieces from LDS before storing any, so the LDS latency is
    // paid once per batch rather than once per row, and walks its (row,
    // piece) position by adding a fixed step -- no division per piece.
    constexpr int kFlushBatch = 8;
    auto flush = [&]() {
        const int vbase = stage_first * T * kLmTile;
        const int per_row = staged * T * (kLmTile / 4);        // 16-byte pieces per row, >= 16
        const int nrows = min(rows, MT * kLmTile);
        const int dq = kWave / per_row, dr = kWave % per_row;  // the step, in rows + pieces
        const bool whole = vec_store_ok(V) && (stage_first + (staged - 1) * gstep + 1) * T * kLmTile <= V;
        int rr = lane / per_row, jp = lane % per_row;
        while (rr < nrows) {
            f32x4 x[kFlushBatch];
            int ur[kFlushBatch], uj[kFlushBatch];
#pragma unroll
            for (int u = 0; u < kFlushBatch; ++u) {
                ur[u] = rr;
                uj[u] = (jp / (T * 4)) * gstep * T * kLmTile + (jp % (T * 4)) * 4;
                x[u] = *reinterpret_cast<const f32x4*>(&st[min(rr, nrows - 1)][jp * 4]);
                rr += dq;
                jp += dr;
                if (jp >= per_row) { jp -= per_row; ++rr; }
            }
            if (whole) {                                       // no piece crosses V
#pragma unroll
                for (int u = 0; u < kFlushBatch; ++u)
                    if (ur[u] < nrows)
                        __builtin_nontemporal_store(
                            x[u], reinterpret_cast<f32x4*>(logits + (size_t)(row0 + ur[u]) * V + vbase + uj[u]));
            } else {
#pragma unroll
                for (int u = 0; u < kFlushBatch; ++u) {
                    if (ur[u] >= nrows) continue;
                    float* lrow = logits + (size_t)(row0 + ur[u]) * V;
                    const int v = vbase + uj[u];
                    if (vec_store_ok(V) && v + 3 < V) {
                        __builtin_nontemporal_store(x[u], reinterpret_cast<f32x4*>(lrow + v));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (v + i < V) lrow[v + i] = x[u][i];
                    }
                }
            }
        }
        stage_first += staged * gstep;
        staged = 0;
    };
    // Lane holds D[vocab 4*kg + i][hidden row r16] of each fragment; its ids
    // rise with t and i, and with g, so a strict '>' keeps the first maximum.
    // The epilogue runs between two k-steps of the stream, with the ring's
    // loads in flight, on one wave per SIMD: short dependency chains matter.
    // A group that lies inside V (all but possibly the last) takes the
    // unchecked form: the group's max by a tree, the running sum's terms by
    // the hardware exp2 (arguments <= 0, relative error near 1e-7) into four
    // independent sums, and the first id of the group's max found by
    // independent compares.
    auto epilogue_row = [&](int m, int g, auto full_tag) {
        constexpr bool kFull = decltype(full_tag)::value;
        const int v0 = g * T * kLmTile + kg * 4;              // id of acc[0][m][0]
        float mx = -INFINITY;
        if (kFull) {
            float mt[T];
#pragma unroll
            for (int t = 0; t < T; ++t)
                mt[t] = fmaxf(fmaxf(acc[t][m][0], acc[t][m][1]), fmaxf(acc[t][m][2], acc[t][m][3]));
#pragma unroll
            for (int h = T / 2; h >= 1; h >>= 1)
#pragma unroll
                for (int t = 0; t < h; ++t) mt[t] = fmaxf(mt[t], mt[t + h]);
            mx = mt[0];
            if (mx > run_av[m]) {
                int id = 0;
#pragma unroll
                for (int t = T - 1; t >= 0; --t)
#pragma unroll
                    for (int e = 3; e >= 0; --e)
                        id = acc[t][m][e] == mx ? v0 + t * kLmTile + e : id;
                run_av[m] = mx;
                run_ai[m] = id;
            }
        } else {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (v0 + t * kLmTile + e < V) {
                        mx = fmaxf(mx, acc[t][m][e]);
                        if (acc[t][m][e] > run_av[m]) { run_av[m] = acc[t][m][e]; run_ai[m] = v0 + t * kLmTile + e; }
                    }
        }
        if (mx == -INFINITY) return;
        const float nm = fmaxf(run_m[m], mx);
        float sm[4] = {run_m[m] == -INFINITY ? 0.f : run_s[m] * exp2_scaled(run_m[m] - nm), 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (kFull || v0 + t * kLmTile + e < V) sm[e] += exp2_scaled(acc[t][m][e] - nm);
        run_m[m] = nm;
        run_s[m] = (sm[0] + sm[1]) + (sm[2] + sm[3]);
    };
    auto epilogue = [&](int g) {
        const bool full = (g + 1) * T * kLmTile <= V;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if (keep_logits) {
#pragma unroll
                for (int t = 0; t < T; ++t)
                    *reinterpret_cast<f32x4*>(&st[m * kLmTile + r16][(staged * T + t) * kLmTile + kg * 4]) =
                        acc[t][m];
            }
            if (full) epilogue_row(m, g, std::true_type{});
            else epilogue_row(m, g, std::false_type{});
        }
        if (++staged == kStageGroups<MT, T>) {
            if (keep_logits) flush();
            else { stage_first += staged * gstep; staged = 0; }
        }
    };

    // Fill the ring, then stream: MFMA on the oldest slot, refill it.
    zero_acc();
    int cg = gb, ck = 0;
    if (gb < ge) {
        if (FAST) {
            // nstep is a multiple of U, so groups start and end on ring
            // boundaries and the load cursor moves once per block.  The
            // block's loads are unconditional: past the wave's last group the
            // cursor keeps pointing at that group's rows (valid memory; the
            // loaded values are never used), which keeps the loop free of
            // branches around loads and the loads in flight across iterations.
            auto load_block = [&]() {
#pragma unroll
                for (int u = 0; u < U; ++u) {
#pragma unroll
                    for (int t = 0; t < T; ++t) wr[u][t] = lp[t][(lk + u) * kWStep];
#pragma unroll
                    for (int m = 0; m < MT; ++m) hr[u][m] = hp[m][(lk + u) * 4];
                }
            };
            // Each group walks its k-steps from a block of its own (a hash
            // of the group index) and wraps; k is a pure reduction, so only
            // the fp32 summation order changes.  Otherwise every wave reads
            // the same offset within its rows at the same moment, and with a
            // power-of-two row pitch (d = 4096: 8 KB) all requests in flight
            // share their low address bits; the achieved bandwidth then
            // depended on where the allocation of W happened to sit in HBM
            // (175-217 us for the same 1 GB on four allocations, 179-181 us
            // with the offsets spread).
            const int nblk = nstep / U;
            auto rot = [&](int g) {
                return (int)(((unsigned)g * 2654435761u >> 16) % (unsigned)nblk) * U;
            };
            int lcnt = 0;                 // k-steps loaded in the current load group
            lk = rot(lg);
            auto next_block = [&]() {
                lk += U;
                lcnt += U;
                if (lk == nstep) lk = 0;
                if (lcnt == nstep) {
                    lcnt = 0;
                    lg += gstep;
                    if (lg < ge) { set_rows(lg); lk = rot(lg); }
                }
            };
            load_block();
            next_block();
            while (cg < ge) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    mma(u);
#pragma unroll
                    for (int t = 0; t < T; ++t) wr[u][t] = lp[t][(lk + u) * kWStep];
#pragma unroll
                    for (int m = 0; m < MT; ++m) hr[u][m] = hp[m][(lk + u) * 4];
                }
                next_block();
                ck += U;
                if (ck == nstep) { epilogue(cg); zero_acc(); ck = 0; cg += gstep; }
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (lg < ge) load(u);
                advance();
            }
            while (cg < ge) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (cg < ge) {
                        mma(u);
                        if (lg < ge) load(u);
                        advance();
                        if (++ck == nstep) { epilogue(cg); zero_acc(); ck = 0; cg += gstep; }
                    }
                }
            }
        }
    }

    if (keep_logits && staged > 0) flush();

    // One partial per hidden row for the whole workgroup.  Every lane's
    // running partial (one per wave and k group: kSrc per row) goes to LDS as
    // it is; then four adjacent lanes per row merge four partials each and
    // combine across their quad with two DPP exchanges.  The end of the
    // stream runs on few waves, so what counts is the length of the
    // dependent instruction chain: the hardware exp2 (rescale factors are
    // <= 1, relative error near 1e-7) and no LDS shuffles.
    constexpr int kSrc = kLmWaves * 4;
    constexpr int kSrcPad = kSrc + 4;                     // rows stay 16-byte aligned
    static_assert(kSrc == 16, "four lanes per row, four partials per lane");
    static_assert(MT * kLmTile * 4 <= kLmWaves * kWave, "a quad of lanes per row");
    __shared__ __attribute__((aligned(16))) float s_max[MT * kLmTile][kSrcPad];
    __shared__ __attribute__((aligned(16))) float s_sum[MT * kLmTile][kSrcPad];
    __shared__ __attribute__((aligned(16))) float s_av[MT * kLmTile][kSrcPad];
    __shared__ __attribute__((aligned(16))) int s_ai[MT * kLmTile][kSrcPad];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int c = wave * 4 + kg;
        s_max[m * kLmTile + r16][c] = run_m[m];
        s_sum[m * kLmTile + r16][c] = run_s[m];
        s_av[m * kLmTile + r16][c] = run_av[m];
        s_ai[m * kLmTile + r16][c] = run_ai[m];
    }
    __syncthreads();
    const int prow = threadIdx.x >> 2, pq = (threadIdx.x & 3) * 4;
    if (prow < MT * kLmTile && prow < rows) {             // whole quads: a row's 4 lanes agree
        const f32x4 mv = *reinterpret_cast<const f32x4*>(&s_max[prow][pq]);
        const f32x4 sv = *reinterpret_cast<const f32x4*>(&s_sum[prow][pq]);
        const f32x4 a4 = *reinterpret_cast<const f32x4*>(&s_av[prow][pq]);
        const int4 i4 = *reinterpret_cast<const int4*>(&s_ai[prow][pq]);
        float m = fmaxf(fmaxf(mv[0], mv[1]), fmaxf(mv[2], mv[3]));
        float s = 0.f;
        if (m != -INFINITY)
            s = (sv[0] * exp2_scaled(mv[0] - m) + sv[1] * exp2_scaled(mv[1] - m)) +
                (sv[2] * exp2_scaled(mv[2] - m) + sv[3] * exp2_scaled(mv[3] - m));
        float av = a4[0], av1 = a4[2];
        int ai = i4.x, ai1 = i4.z;
        arg_merge(av, ai, a4[1], i4.y);
        arg_merge(av1, ai1, a4[3], i4.w);
        arg_merge(av, ai, av1, ai1);
        quad_merge<kQuadXor1>(m, s, av, ai);
        quad_merge<kQuadXor2>(m, s, av, ai);
        if ((threadIdx.x & 3) == 0) {
            part_max[(size_t)(row0 + prow) * NPs + blockIdx.x] = m;
            part_sum[(size_t)(row0 + prow) * NPs + blockIdx.x] = s;
            if (part_arg) part_arg[(size_t)(row0 + prow) * NPs + blockIdx.x] = ai;
        }
    }
}

int cu_count() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    int* slot = dev >= 0 && dev < 64 ? &cached[dev] : nullptr;
    int n = slot ? __atomic_load_n(slot, __ATOMIC_RELAXED) : 0;
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        if (slot) __atomic_store_n(slot, n, __ATOMIC_RELAXED);
    }
    return n;
}

template <int MT, bool WT>
void launch_mt(dim3 g, dim3 b, hipStream_t s, const uint16_t* hidden, const uint16_t* W, int row0,
               int rows, int d, int V, float* logits, float* pm, float* ps, int32_t* pa, int NPs,
               int32_t* counters, int nc) {
    constexpr int T = LmCfg<MT>::T, U = LmCfg<MT>::U;
    const int nstep = (d + 31) / 32;
    if (d % 32 == 0 && nstep % U == 0)
        lmhead_kernel<MT, T, U, true, WT><<<g, b, 0, s>>>(hidden, W, row0, rows, d, V, logits, pm, ps, pa, NPs, counters, nc);
    else
        lmhead_kernel<MT, T, kGenericU, false, WT><<<g, b, 0, s>>>(hidden, W, row0, rows, d, V, logits, pm, ps, pa, NPs, counters, nc);
}

template <bool WT>
void launch_rows(int mt, dim3 g, dim3 b, hipStream_t s, const uint16_t* hidden, const uint16_t* W,
                 int row0, int rows, int d, int V, float* logits, float* pm, float* ps, int32_t* pa,
                 int NPs, int32_t* counters, int nc) {
    switch (mt) {
        case 1: launch_mt<1, WT>(g, b, s, hidden, W, row0, rows, d, V, logits, pm, ps, pa, NPs, counters, nc); break;
        case 2: launch_mt<2, WT>(g, b, s, hidden, W, row0, rows, d, V, logits, pm, ps, pa, NPs, counters, nc); break;
        case 3: launch_mt<3, WT>(g, b, s, hidden, W, row0, rows, d, V, logits, pm, ps, pa, NPs, counters, nc); break;
        default: launch_mt<4, WT>(g, b, s, hidden, W, row0, rows, d, V, logits, pm, ps, pa, NPs, counters, nc); break;
    }
}

}  // namespace

// Workgroups of the LM-head launch (also the number of softmax partials per
// row): one per compute unit, capped so every wave has fragments to stream.
int lmhead_grid(int V) {
    const int ntiles = (V + kLmTile - 1) / kLmTile;
    // One workgroup per CU at most, and just enough of them that every wave
    // gets the same number of fragment groups (measured on the grouping of
    // the one-hidden-fragment configuration, which all row counts share).
    const int T1 = LmCfg<1>::T;
    const int ngroups = (ntiles + T1 - 1) / T1;
    const int waves = cu_count() * kLmWaves;
    const int per_wave = (ngroups + waves - 1) / waves;
    const int grid = (ngroups + per_wave * kLmWaves - 1) / (per_wave * kLmWaves);
    return max(1, min(grid, lmhead_useful_groups(V)));
}

// Enqueue the LM-head stage: one launch per group of up to 64 hidden rows.
// logits may be null: then only the partials are written.  w_tiled: W is in
// the 16 x 32 tile layout, else [V][d] row-major.
hipError_t launch_lmhead(const uint16_t* hidden, const uint16_t* W, bool w_tiled, int R, int d,
                         int V, float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                         int NPs, int grid, int32_t* counters, int n_counters, hipStream_t stream) {
    for (int row0 = 0; row0 < R; row0 += kLmRowsPerPass) {
        const int rows = min(kLmRowsPerPass, R - row0);
        const int mt = (rows + kLmTile - 1) / kLmTile;
        const int nc = row0 == 0 ? n_counters : 0;
        dim3 g(grid), b(kLmWaves * kWave);
        if (w_tiled)
            launch_rows<true>(mt, g, b, stream, hidden, W, row0, rows, d, V, logits, part_max, part_sum, part_arg, NPs, counters, nc);
        else
            launch_rows<false>(mt, g, b, stream, hidden, W, row0, rows, d, V, logits, part_max, part_sum, part_arg, NPs, counters, nc);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sv
