// LM-head GEMM for many rows: logits = hidden . W^T with R > 64, plus one
// softmax partial and (when asked) one greedy candidate (largest logit, lowest
// id) per (row, 256-entry vocab block).
//
// Source: "推测解码" (world.lapla.si/zh/specdec), sections 先让小模型猜 and
// 几段话一起写 -- one read of the target's weights serves every drafted
// position of every sequence in the batch; "多詞元預測視覺化指南", section
// 高效嵌入器 -- the LM head multiplies hidden states by the tied embedding
// matrix W [V][d].
//
// Shape of the work.  The GEMM does 2*R flops per two bytes of W: below the
// MI355X ridge (~312 flop/byte) for R up to a few hundred, above it at
// R = 1280.  One kernel serves all R > 64: v_mfma_f32_16x16x32_bf16 with W as
// the A operand (vocab = M) and the hidden rows as B, so each lane ends with
// four consecutive vocab entries of one hidden row -- a 16-byte logits store.
// A workgroup of eight waves computes 256 vocab entries x TR = 64 FR rows;
// both operands go from memory straight into LDS through a ring of k steps,
// and the waves take turns between MFMAs and fragment reads (ping-pong).
// The hidden rows arrive in 1 KB tiles of 16 rows x 32 columns (the caller
// tiles them into the workspace first), W in the same tiles or [V][d]
// row-major: a tiled operand's 16-row slice of a k step is one contiguous
// 1 KB, where a row-major one takes half of a 128-byte line from each of
// 16 rows and the next k step the other half.
//
//   R <= 128: FR = 2 with a three-stage ring -- 74 KB of LDS (76 KB with
//     argmax partials) and <= 128 registers, so two workgroups share a CU
//     and one's loads, epilogue and stores overlap the other's MFMAs.
//     HBM-bound: W is streamed once.
//   R > 128: FR in {5, 4, 3, 2}, whichever pads R least (ties to the taller
//     block), with a four-stage ring, one workgroup per CU.  At R = 1280 the
//     GEMM is MFMA-bound and four 320-row blocks share each W tile.
//
// Block order.  Workgroups are dispatched round-robin over the 8 XCDs; the
// block index is remapped so that each XCD receives a contiguous run of the
// (vocab block, row block) sequence with row blocks fastest.  The row blocks
// that share a W tile then run together on one XCD and the tile comes from
// HBM once, from that XCD's L2 after.

#include "sv_common.h"

namespace sv {

namespace {

constexpr int kTV = kLmTiledVocab;   // vocab rows per workgroup (256)
constexpr int kXcds = 8;

// ---------------------------------------------------------------------------
// Blocks of 256 vocab rows x TR = 64 FR hidden rows, eight waves in a
// 2 (vocab) x 4 (rows) grid, each 128 vocab rows x 16 FR hidden rows
// (8 x FR fragments).  Both operands go from memory straight into LDS
// (buffer_load_dwordx4 ... lds or global_load_lds_dwordx4: 16 bytes per
// lane, no registers on the way) through a ring of S stages of one 32-wide
// k step each.
//
// Ping-pong.  Waves 0-3 (group A) and 4-7 (group B) share the SIMDs, one of
// each per SIMD, and take turns: while one group issues its MFMAs for a k
// step the other reads its next fragments from LDS, and two barriers per k
// step (X, Y) swap the roles, so a SIMD's matrix unit always has a wave with
// operands ready feeding it.  Phase P_t runs from Y_{t-1} to X_t, Q_t from
// X_t to Y_t.  Each copy instruction holds its wave ~30 cycles, so with the
// four-stage ring (R > 128) a wave issues its share of the ring's copies in
// its read phase, once its fragments have landed, where it would otherwise
// wait at the next barrier; its MFMA phase is MFMAs only.  Per k step t:
//   A: MFMAs(t) | wait own copies of t+1 | X | read frags(t+1), copies of t+S-1 | Y
//   B: read frags(t), copies of t+S-1 | wait own copies of t+1 | X | MFMAs(t) | Y
// With the three-stage ring (R <= 128, HBM-bound) that would leave group A
// at most one phase to cover the memory latency, so there each wave issues
// its copies between its own MFMAs instead (one after each of the first
// fragment rows: the MFMAs already issued keep the matrix unit busy while
// the copy waits):
//   A: MFMAs(t) + copies of t+S-1 | wait own copies of t+1 | X | read frags(t+1) | Y
//   B: read frags(t) | wait own copies of t+1 | X | MFMAs(t) + copies of t+S-1 | Y
// Stage u % S holds step u.  Before X_t every wave has waited for its copies
// of step t+1, so after X_t the stage of t+1 is whole (A reads it in Q_t, B
// in P_{t+1}).  The copies of step t+S-1 go to stage (t-1) % S, which both
// groups finished reading before step t began (A in Q_{t-2}, waited before
// Y_{t-2}; B in P_{t-1}, waited before X_{t-1}), and which no wave reads
// during P_t or Q_t (A reads stage (t+1) % S, B stage t % S).  Measured at
// R = 1280, d = 4096 (per k step, s_memtime in a probe build): a group's 40
// MFMAs take ~650 cycles (~790 with copies between them), its 13 fragment
// reads ~300; each barrier costs ~90-140 cycles.
//
// Fragment reads are one inline-asm block per k step (all reads, then the
// lgkmcnt(0) wait, inside it).  Written as plain LDS loads, the compiler
// cannot prove at the loop head that they miss the stages the copies in
// flight are filling, and waits for every copy (vmcnt(0)) once per ring
// turn in each group; that wait exposed the full memory latency every S
// steps (R = 128: 268 -> 251 us; R = 320: 402 -> 387 us).
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

// One 1 KB copy from memory into LDS through a buffer resource: lane i's 16
// bytes from base + voff (a lane beyond the range's nbytes reads zeros) go to
// lds + 16 i.  Records in bytes; 0x00020000 is the 32-bit data format any
// raw buffer on gfx9 uses.
__device__ __forceinline__ void buffer_copy_lds(const char* base, uint32_t nbytes, uint32_t voff,
                                                __attribute__((address_space(3))) void* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)nbytes, 0x00020000), lds, 16,
        voff, 0, 0, 0);
}

// LDS address (byte offset in the workgroup's LDS) of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// One k step's fragment reads of a wave: FV = 8 A fragments 1 KB apart from
// address a, FR B fragments 1 KB apart from address b, then lgkmcnt(0) in
// the same block, so every output register is written when the block ends.
// Outputs are early-clobber: the two address registers stay live throughout.
// The memory clobber keeps the block after the copies and barriers that make
// the stage's bytes valid.
#define SV_DSR(o, base, off) "ds_read_b128 %" #o ", %" #base " offset:" #off "\n"
#define SV_DSR_A(base)                                                               \
    SV_DSR(0, base, 0) SV_DSR(1, base, 1024) SV_DSR(2, base, 2048) SV_DSR(3, base, 3072) \
    SV_DSR(4, base, 4096) SV_DSR(5, base, 5120) SV_DSR(6, base, 6144) SV_DSR(7, base, 7168)
#define SV_OUT_A                                                                       \
    "=&v"(fa[0]), "=&v"(fa[1]), "=&v"(fa[2]), "=&v"(fa[3]), "=&v"(fa[4]), "=&v"(fa[5]), \
    "=&v"(fa[6]), "=&v"(fa[7])
template <int FR>
__device__ __forceinline__ void read_frags_asm(u32x4 (&fa)[8], u32x4 (&fb)[FR], uint32_t a, uint32_t b) {
    static_assert(FR >= 2 && FR <= 5, "fragment rows");
    if constexpr (FR == 5) {
        asm volatile(SV_DSR_A(13) SV_DSR(8, 14, 0) SV_DSR(9, 14, 1024) SV_DSR(10, 14, 2048)
                     SV_DSR(11, 14, 3072) SV_DSR(12, 14, 4096) "s_waitcnt lgkmcnt(0)"
                     : SV_OUT_A, "=&v"(fb[0]), "=&v"(fb[1]), "=&v"(fb[2]), "=&v"(fb[3]), "=&v"(fb[4])
                     : "v"(a), "v"(b)
                     : "memory");
    } else if constexpr (FR == 4) {
        asm volatile(SV_DSR_A(12) SV_DSR(8, 13, 0) SV_DSR(9, 13, 1024) SV_DSR(10, 13, 2048)
                     SV_DSR(11, 13, 3072) "s_waitcnt lgkmcnt(0)"
                     : SV_OUT_A, "=&v"(fb[0]), "=&v"(fb[1]), "=&v"(fb[2]), "=&v"(fb[3])
                     : "v"(a), "v"(b)
                     : "memory");
    } else if constexpr (FR == 3) {
        asm volatile(SV_DSR_A(11) SV_DSR(8, 12, 0) SV_DSR(9, 12, 1024) SV_DSR(10, 12, 2048)
                     "s_waitcnt lgkmcnt(0)"
                     : SV_OUT_A, "=&v"(fb[0]), "=&v"(fb[1]), "=&v"(fb[2])
                     : "v"(a), "v"(b)
                     : "memory");
    } else {
        asm volatile(SV_DSR_A(10) SV_DSR(8, 11, 0) SV_DSR(9, 11, 1024) "s_waitcnt lgkmcnt(0)"
                     : SV_OUT_A, "=&v"(fb[0]), "=&v"(fb[1])
                     : "v"(a), "v"(b)
                     : "memory");
    }
}
#undef SV_OUT_A
#undef SV_DSR_A
#undef SV_DSR

// Two waves per SIMD (one workgroup per CU) with the four-stage ring; four
// (two workgroups per CU: <= 128 registers) with the three-stage one.
// htile: the R hidden rows in 1 KB tiles of 16 rows x 32 columns (tile
// (i, t) at element (i * nk + t) * 512, zero past R and d), so each 16-row
// slice of a stage is one contiguous 1 KB of memory.  W the same with WT,
// otherwise [V][d] row-major.
template <int FR, int S, bool ARG, bool BUF, bool WT>
__global__ __launch_bounds__(kBigNT) __attribute__((amdgpu_waves_per_eu(S == 3 ? 4 : 2))) void lmhead_big_kernel(
    const uint16_t* __restrict__ htile, const uint16_t* __restrict__ W, int R, int d, int V,
    int nvb, int nrb, float* __restrict__ logits, float* __restrict__ part_max,
    float* __restrict__ part_sum, int32_t* __restrict__ part_arg, int NPs,
    int32_t* __restrict__ counters, int n_counters) {
    using C = BigCfg<FR>;
    constexpr int TV = C::TV, TR = C::TR, NI = C::NI, NIW = C::NIW;
    constexpr int WV = kBigWV, FV = kBigFV, NW = kBigNW;
    static_assert(TV == kTV, "256 vocab rows per block: one softmax partial column each");
    static_assert(S == 3 || S == 4, "ring depth");
    static_assert(FV == 8 && kLmTile * kBigRowBytes == 1024, "fragment reads 1 KB apart");
    // One array per stage, each selected by a compile-time stage index in
    // the unrolled loop (the fragment reads take them as LDS offsets).
    __shared__ __attribute__((aligned(1024))) char st0[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st1[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st2[C::kStageBytes];
    __shared__ __attribute__((aligned(1024))) char st3[S == 4 ? C::kStageBytes : 1024];
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
    // (or R) copy the last valid row; their results are never stored.  One
    // instruction on a tiled operand reads one whole 1 KB tile.  When
    // NI is not a multiple of NW a wave's last j may pass NI: it repeats its
    // previous copy (same bytes to the same place), so every wave issues NIW
    // copies per step and the vmcnt accounting is the same on every wave.
    //
    // BUF (both operands under 4 GiB): each copy is a buffer load with the
    // lane's byte offset from the matrix start fixed for the whole walk and
    // the step's k in the resource base, so a copy costs scalar work, one
    // M0 write and the load itself -- no per-lane address arithmetic, which
    // as 64-bit pointer adds between the MFMAs held the MFMA phase back
    // (R = 1280: 1179 -> 1120-1146 us).  The resource's range ends with the
    // matrix, so a chunk past the end of the last row reads zeros.
    // Otherwise: 64-bit pointers per copy.
    const uint16_t* src[BUF ? 1 : NIW];
    uint32_t voff[BUF ? NIW : 1];
    bool from_w[NIW];
    int dst[NIW];
    // row = 16 j + lane / 4 with 16 j a multiple of 8, so (row >> 1) & 3 = (lane >> 3) & 3
    const int goff = ((lane & 3) ^ ((lane >> 3) & 3)) * 8;
    const int nk = (d + kBigK - 1) / kBigK;
    // Element offset of k step 0 of row v of a tiled operand, and of W.
    auto tile_row = [&](int v) -> size_t { return (size_t)(v >> 4) * nk * 512 + (v & 15) * kBigK; };
    auto w_row = [&](int v) -> size_t { return WT ? tile_row(v) : (size_t)v * d; };
#pragma unroll
    for (int m = 0; m < NIW; ++m) {
        const int j = wave + m * NW < NI ? wave + m * NW : wave + (m - 1) * NW;
        const int row = j * 16 + (lane >> 2);
        const size_t elem = (row < TV ? w_row(min(v0 + row, V - 1)) : tile_row(min(r0 + row - TV, R - 1))) + goff;
        from_w[m] = j < TV / 16;                 // the same for every lane of the instruction
        if constexpr (BUF) voff[m] = (uint32_t)(elem * 2);
        else src[m] = (row < TV ? W : htile) + elem;
        dst[m] = j * 1024;
    }

    const bool ragged = d % kBigK != 0;       // the last step has chunks past the end of a row
    auto stage = [&](int s) -> char* { return s == 0 ? st0 : s == 1 ? st1 : s == 2 ? st2 : st3; };
    // Copies of step t (t >= nk: a repeat of the last step, into a stage no
    // step reads again, so that every step issues the same copies), as
    // element offsets from each copy's step-0 address.  A tiled operand
    // moves one 1 KB tile per step, and its chunks past d read the tiles'
    // zeros.  In row-major W a chunk past the end of a row copies the row's
    // first chunk instead (pointer copies) or reads the next row's first
    // bytes (buffer copies; zeros past the matrix); the fragment lanes
    // holding it are zeroed after the read.
    auto tile_step = [&](int t) { return (t < nk ? t : nk - 1) * kBigK * 16; };
    auto w_step = [&](int t) {
        if (WT) return tile_step(t);
        const int k0 = (t < nk ? t : nk - 1) * kBigK;
        return (BUF || !ragged || k0 + goff < d) ? k0 : -goff;
    };
    // A buffer copy reads from the operand at the step's offset (base) up
    // to the operand's end (range): both uniform, so they live in scalar
    // registers.
    const uint32_t w_bytes = BUF ? (uint32_t)(WT ? tiled_bytes(V, d) : (size_t)V * d * 2) : 0u;
    const uint32_t h_bytes = BUF ? (uint32_t)tiled_bytes(R, d) : 0u;
    auto copy_one = [&](int m, int kh, int kw, char* st) {
        auto* l = (__attribute__((address_space(3))) void*)(st + dst[m]);
        if constexpr (BUF) {
            const uint32_t kb = (uint32_t)(from_w[m] ? kw : kh) * 2u;
            buffer_copy_lds(from_w[m] ? (const char*)W + kb : (const char*)htile + kb,
                            (from_w[m] ? w_bytes : h_bytes) - kb, voff[m], l);
        } else {
            __builtin_amdgcn_global_load_lds((void*)(src[m] + (from_w[m] ? kw : kh)), l, 16, 0, 0);
        }
    };
    auto copy = [&](int t, char* st) {
        const int kh = tile_step(t), kw = w_step(t);
#pragma unroll
        for (int m = 0; m < NIW; ++m) copy_one(m, kh, kw, st);
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
        read_frags_asm<FR>(fa, fb, lds_addr(st + aoff), lds_addr(st + boff));
    };
    // The reads have returned; k-chunk kg of step t past the end of the rows
    // (last step, d not a multiple of 32) must contribute 0.
    auto finish_frags = [&](int t) {
        if (ragged && t == nk - 1 && t * kBigK + kg * 8 >= d) {
#pragma unroll
            for (int a = 0; a < FV; ++a) fa[a] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int b = 0; b < FR; ++b) fb[b] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // The step's MFMAs, fragment row by fragment row; with the three-stage
    // ring this wave's copies of step t (into stage st) go one after each of
    // the first NIW rows, with the four-stage ring into the read phase.
    static_assert(NIW <= FV, "one copy per fragment row at most");
    constexpr bool kCopyInRead = S == 4;
    auto mfmas_copy = [&](int t, char* st) {
        const int kh = tile_step(t), kw = w_step(t);
#pragma unroll
        for (int a = 0; a < FV; ++a) {
#pragma unroll
            for (int b = 0; b < FR; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, fa[a]), __builtin_bit_cast(bf16x8, fb[b]),
                    acc[a][b], 0, 0, 0);
            if (!kCopyInRead && a < NIW) copy_one(a, kh, kw, st);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // Each group issues its copies of step t+S-1 during step t, into stage
    // (t-1) % S.  Before X_t each wave needs its copies of step t+1 complete
    // (vmcnt counts in issue order); after them it has issued those of the
    // later steps up to the last phase before X_t that carries copies.
    // Copies in the read phase: A issued step t+1's in Q_{t+2-S}, then
    // t+2 .. t+S-2 (S-3 sets); B in P_{t+2-S}, then t+2 .. t+S-1 (S-2
    // sets, P_t included).  Copies in the MFMA phase: A in P_{t+2-S}, then
    // t+2 .. t+S-1 (S-2 sets, P_t included); B in Q_{t+2-S}, then
    // t+2 .. t+S-2 (S-3 sets).
    constexpr int kWaitA = (kCopyInRead ? S - 3 : S - 2) * NIW;
    constexpr int kWaitB = (kCopyInRead ? S - 2 : S - 3) * NIW;
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
                if (kCopyInRead) copy(t + S - 1, stage((h + S - 1) % S));
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
                if (kCopyInRead) copy(t + S - 1, stage((h + S - 1) % S));
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


template <int FR, int S, bool WT>
hipError_t launch_big(const uint16_t* htile, const uint16_t* W, int R, int d, int V,
                      float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                      int NPs, int32_t* counters, int n_counters, hipStream_t stream) {
    using C = BigCfg<FR>;
    const int nvb = (V + C::TV - 1) / C::TV;
    const int nrb = (R + C::TR - 1) / C::TR;
    const int nblocks = nvb * nrb;
    const int grid = (nblocks + kXcds - 1) / kXcds * kXcds;
    // Buffer copies need both matrices' byte sizes to fit the 32-bit range.
    const size_t w_bytes = WT ? tiled_bytes(V, d) : (size_t)V * d * 2;
    const bool buf = w_bytes < (1ull << 32) && tiled_bytes(R, d) < (1ull << 32);
    const dim3 g(grid), blk(kBigNT);
    if (part_arg && buf)
        lmhead_big_kernel<FR, S, true, true, WT><<<g, blk, 0, stream>>>(
            htile, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    else if (part_arg)
        lmhead_big_kernel<FR, S, true, false, WT><<<g, blk, 0, stream>>>(
            htile, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    else if (buf)
        lmhead_big_kernel<FR, S, false, true, WT><<<g, blk, 0, stream>>>(
            htile, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    else
        lmhead_big_kernel<FR, S, false, false, WT><<<g, blk, 0, stream>>>(
            htile, W, R, d, V, nvb, nrb, logits, part_max, part_sum, part_arg, NPs, counters, n_counters);
    return hipGetLastError();
}

template <bool WT>
hipError_t launch_any(const uint16_t* htile, const uint16_t* W, int R, int d, int V,
                      float* logits, float* part_max, float* part_sum, int32_t* part_arg,
                      int NPs, int32_t* counters, int n_counters, hipStream_t stream) {
    // 64 < R <= 128: one 128-row block per W tile, two workgroups per CU.
    if (R <= 128)
        return launch_big<2, 3, WT>(htile, W, R, d, V, logits, part_max, part_sum, part_arg, NPs,
                                    counters, n_counters, stream);
    // The row-block height (64 FR rows) that pads R least, ties to the taller
    // block, whose W tile then serves more rows: R = 320 runs one block of
    // 320 rows, R = 1280 four.
    int FR = 5;
    for (int fr : {4, 3, 2})
        if ((R + 64 * fr - 1) / (64 * fr) * (64 * fr) < (R + 64 * FR - 1) / (64 * FR) * (64 * FR)) FR = fr;
    switch (FR) {
        case 5: return launch_big<5, 4, WT>(htile, W, R, d, V, logits, part_max, part_sum, part_arg,
                                            NPs, counters, n_counters, stream);
        case 4: return launch_big<4, 4, WT>(htile, W, R, d, V, logits, part_max, part_sum, part_arg,
                                            NPs, counters, n_counters, stream);
        case 3: return launch_big<3, 4, WT>(htile, W, R, d, V, logits, part_max, part_sum, part_arg,
                                            NPs, counters, n_counters, stream);
        default: return launch_big<2, 4, WT>(htile, W, R, d, V, logits, part_max, part_sum, part_arg,
                                             NPs, counters, n_counters, stream);
    }
}

}  // namespace

// htile: the hidden rows in the 16 x 32 tile layout; w_tiled: W in it too,
// else [V][d] row-major.
hipError_t launch_lmhead_tiled(const uint16_t* htile, const uint16_t* W, bool w_tiled, int R,
                               int d, int V, float* logits, float* part_max, float* part_sum,
                               int32_t* part_arg, int NPs, int32_t* counters, int n_counters,
                               hipStream_t stream) {
    return w_tiled ? launch_any<true>(htile, W, R, d, V, logits, part_max, part_sum, part_arg, NPs,
                                      counters, n_counters, stream)
                   : launch_any<false>(htile, W, R, d, V, logits, part_max, part_sum, part_arg,
                                       NPs, counters, n_counters, stream);
}

}  // namespace sv
