// MXFP8 grouped GEMM kernels for few rows per expert and their launchers; the
// device code and its description are in dev_gemm_mx.h.
#include "dev_gemm_mx.h"

namespace moe {

namespace {

using namespace mx_gemm;

template <int NT, int WT, int NW>
__global__ __launch_bounds__(NW * 64) void gemm1_mx_kernel(GemmArgs g, int ntiles) {
    int blk, tile;
    if (!map_active_tile(g, ntiles, blk, tile)) return;
    gemm1_mx_tile<NT, WT, NW>(g, blk, tile);
}

template <int NT, int WT, int NW>
__global__ __launch_bounds__(NW * 64) void gemm2_mx_kernel(GemmArgs g, int ntiles) {
    int blk, tile;
    if (!map_active_tile(g, ntiles, blk, tile)) return;
    gemm2_mx_tile<NT, WT, NW>(g, blk, tile);
}

// GEMM2, NTILE column tiles of one block per workgroup (block-major over the
// blocks' tile groups)
template <int NT, int WT, int NW, int NTILE>
__global__ __launch_bounds__(NW * 64) void gemm2_mx_tiles_kernel(GemmArgs g, int ngroups) {
    int blk, grp;
    if (!map_active_tile<true>(g, ngroups, blk, grp)) return;
    gemm2_mx_tiles<NT, WT, NW, NTILE>(g, blk, grp * NTILE);
}

template <typename K>
hipError_t launch_tiles(K kernel, const GemmArgs& g, int ntiles, int threads, hipStream_t s) {
    const int64_t n = int64_t(g.num_blocks) * ntiles;
    const int64_t grid = (n + 7) / 8 * 8;
    hipLaunchKernelGGL(kernel, dim3(unsigned(grid)), dim3(threads), 0, s, g, ntiles);
    return hipGetLastError();
}

template <int NT>
hipError_t gemm1_mx(const GemmArgs& g, hipStream_t s) {
    // 4 waves x (32 gate + 32 up) rows = 128 columns, one MX group per wave;
    // 8 waves x (16 + 16) for 64-token blocks (registers)
    if constexpr (NT <= 2) return launch_tiles(gemm1_mx_kernel<NT, 2, 4>, g, g.I / 128, 256, s);
    else return launch_tiles(gemm1_mx_kernel<NT, 1, 8>, g, g.I / 128, 512, s);
}

// Two column tiles per workgroup up to 32-token blocks, four at 64 (the
// block-fp8 GEMM2's measured choice; the loops are the same).
template <int NT>
hipError_t gemm2_mx(const GemmArgs& g, hipStream_t s) {
    constexpr int kTiles = NT >= 4 ? 4 : 2;
    const bool multi = g.I / kStepK <= kTabSteps;
    if constexpr (NT <= 2) {
        if (g.H % 256 == 0) {
            if (multi && (g.H / 256) % kTiles == 0)
                return launch_tiles(gemm2_mx_tiles_kernel<NT, 4, 4, kTiles>, g, g.H / 256 / kTiles, 256, s);
            return launch_tiles(gemm2_mx_kernel<NT, 4, 4>, g, g.H / 256, 256, s);
        }
    }
    if (multi && (g.H / 128) % kTiles == 0)
        return launch_tiles(gemm2_mx_tiles_kernel<NT, 2, 4, kTiles>, g, g.H / 128 / kTiles, 256, s);
    return launch_tiles(gemm2_mx_kernel<NT, 2, 4>, g, g.H / 128, 256, s);
}

}  // namespace

hipError_t launch_gemm1_mx(const GemmArgs& g, hipStream_t s) {
    switch (g.block_m) {
        case 16: return gemm1_mx<1>(g, s);
        case 32: return gemm1_mx<2>(g, s);
        case 64: return gemm1_mx<4>(g, s);
        default: return hipErrorInvalidValue;
    }
}

namespace {

// Packed MXFP8 weight scales: output byte o is lane (o % 64) of K step
// (o / 64) % (kb / 4) of 16-row group o / (16 kb); that lane's row and
// 32-element block are (lane % 16, lane / 16) (kb = K / 32 bytes per row).
__global__ __launch_bounds__(256) void pack_mx_scales_kernel(const uint8_t* __restrict__ in, int64_t n, int kb,
                                                             uint8_t* __restrict__ out) {
    const int64_t o = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (o >= n) return;
    const int64_t grp = o / (16 * kb);
    const int rem = int(o - grp * 16 * kb);
    const int step = rem >> 6, lane = rem & 63;
    out[o] = in[(grp * 16 + (lane & 15)) * kb + 4 * step + (lane >> 4)];
}

}  // namespace

hipError_t launch_pack_mx_scales(const uint8_t* scales, int E, int rows, int K, uint8_t* packed, hipStream_t s) {
    const int kb = K / kMxBlock;
    const int64_t n = int64_t(E) * rows * kb;
    hipLaunchKernelGGL(pack_mx_scales_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, scales, n, kb,
                       packed);
    return hipGetLastError();
}

hipError_t launch_gemm2_mx(const GemmArgs& g, hipStream_t s) {
    switch (g.block_m) {
        case 16: return gemm2_mx<1>(g, s);
        case 32: return gemm2_mx<2>(g, s);
        case 64: return gemm2_mx<4>(g, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
