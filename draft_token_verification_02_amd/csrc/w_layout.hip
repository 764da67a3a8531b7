// The tiled layout of the LM-head matrix W: 1 KB tiles of 16 vocab rows x 32
// hidden columns.  Tile (i, t) holds rows 16 i .. 16 i + 15, columns
// 32 t .. 32 t + 31, row-major, at element (i * nt + t) * 512 with
// nt = ceil(d / 32); entries past V or d are zero.  A k step of the LM-head
// GEMM (32 columns) then reads each 16-row slice of W as one contiguous
// 1 KB run instead of 64 bytes from each of 16 rows 2d bytes apart.  The
// GEMM reads the same values in the same order either way, so its results
// do not depend on the layout.

#include "sv_common.h"

namespace sv {
namespace {

// One 16-byte chunk of the output per thread and pass: chunk c is tile c / 64,
// row (c % 64) / 4, columns 8 (c % 4) .. 8 (c % 4) + 7.  The four waves of a
// workgroup write four consecutive tiles, so each row's source reads are
// 256-byte runs.
__global__ __launch_bounds__(256) void tile_w_kernel(const uint16_t* __restrict__ W, int V, int d,
                                                     int nt, size_t nchunks,
                                                     uint16_t* __restrict__ Wt) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x; c < nchunks; c += stride) {
        const size_t tile = c >> 6;
        const int r = (int)(c >> 2) & 15, g = (int)c & 3;
        const size_t i = tile / (size_t)nt;
        const int t = (int)(tile - i * nt);
        const size_t v = i * 16 + r;
        const int k = t * 32 + g * 8;
        u32x4 x = {0u, 0u, 0u, 0u};
        // d is a multiple of 8, so a chunk that starts before d ends by d
        if (v < (size_t)V && k < d) x = *reinterpret_cast<const u32x4*>(W + v * d + k);
        reinterpret_cast<u32x4*>(Wt)[c] = x;
    }
}

}  // namespace

size_t tiled_w_bytes(int V, int d) {
    return (size_t)(V + 15) / 16 * (size_t)((d + 31) / 32) * 1024;
}

hipError_t launch_tile_w(const uint16_t* W, int V, int d, uint16_t* Wt, hipStream_t stream) {
    const int nt = (d + 31) / 32;
    const size_t nchunks = tiled_w_bytes(V, d) / 16;
    const size_t blocks = (nchunks + 255) / 256;
    const unsigned grid = (unsigned)(blocks < 8192 ? blocks : 8192);
    tile_w_kernel<<<grid, 256, 0, stream>>>(W, V, d, nt, nchunks, Wt);
    return hipGetLastError();
}

}  // namespace sv
