// The tiled layout of a [N][d] bf16 matrix (the LM-head matrix W, N = V, or
// the hidden rows, N = R): 1 KB tiles of 16 rows x 32 columns.  Tile (i, t)
// holds rows 16 i .. 16 i + 15, columns 32 t .. 32 t + 31, row-major, at
// element (i * nt + t) * 512 with nt = ceil(d / 32); entries past N or d are
// zero.  A k step of the LM-head GEMM (32 columns) then reads each 16-row
// slice of an operand as one contiguous 1 KB run instead of 64 bytes from
// each of 16 rows 2d bytes apart: half of a 128-byte L2 line per row, whose
// other half the next k step wants after the line may have been evicted.
// The GEMM reads the same values in the same order either way, so its
// results do not depend on the layout.

#include "sv_common.h"

namespace sv {
namespace {

// Workgroup (i, j): the four tiles (i, 4 j .. 4 j + 3), one per wave, for
// row tiles i = blockIdx.x, + gridDim.x, ...; lane l writes 16 bytes of its
// wave's tile: row l / 4, columns 8 (l % 4) .. 8 (l % 4) + 7.  Each wave
// writes one whole 1 KB tile, and the four waves read 256 contiguous bytes
// of each of the 16 rows.
__global__ __launch_bounds__(256) void tile_w_kernel(const uint16_t* __restrict__ W, int V, int d,
                                                     int nt, uint16_t* __restrict__ Wt) {
    const int t = blockIdx.y * 4 + (int)(threadIdx.x >> 6);
    if (t >= nt) return;
    const int lane = threadIdx.x & 63;
    const int r = lane >> 2, k = t * 32 + (lane & 3) * 8;
    const int ni = (V + 15) / 16;
    for (int i = blockIdx.x; i < ni; i += gridDim.x) {
        const int v = i * 16 + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        // d is a multiple of 8, so a chunk that starts before d ends by d
        if (v < V && k < d) x = *reinterpret_cast<const u32x4*>(W + (size_t)v * d + k);
        reinterpret_cast<u32x4*>(Wt)[((size_t)i * nt + t) * 64 + lane] = x;
    }
}

}  // namespace

size_t tiled_w_bytes(int V, int d) { return tiled_bytes(V, d); }

// Enqueue the tiling of the [V][d] matrix W (the LM-head matrix, or the R
// hidden rows) into Wt (tiled_bytes(V, d) bytes): up to 2^20 x ceil(nt / 4)
// workgroups of four waves.
hipError_t launch_tile_rows(const uint16_t* W, int V, int d, uint16_t* Wt, hipStream_t stream) {
    const int nt = (d + 31) / 32;
    const int ni = (V + 15) / 16;
    const dim3 grid((unsigned)(ni < (1 << 20) ? ni : (1 << 20)), (unsigned)((nt + 3) / 4));
    tile_w_kernel<<<grid, 256, 0, stream>>>(W, V, d, nt, Wt);
    return hipGetLastError();
}

}  // namespace sv
