// Weight-streaming grouped GEMM kernels for few rows per expert (decode) and
// their launchers; the device code and its description are in
// dev_gemm_small.h.
#include "dev_gemm_small.h"

namespace moe {

namespace {

using namespace small_gemm;

// kRot: the fp8 GEMM1 with the rotated K walk (a separate kernel, so the
// plain one keeps its own code and registers; the host picks by g.krot)
template <bool FP8, int NT, int WT, int NW, int U, bool kRot = false>
__global__ __launch_bounds__(NW * 64) void gemm1_small_kernel(GemmArgs g, int ntiles) {
    int blk, tile;
    if (!map_active_tile(g, ntiles, blk, tile)) return;
    gemm1_small_tile<FP8, NT, WT, NW, U, kRot>(g, blk, tile);
}

// GEMM2 takes its items block-major: the column tiles of one expert block,
// adjacent, sweep that expert's W2 rows in order (down GEMM 483 -> 447 us on
// 16 tokens of the skewed layer, 201 -> 196 us on the decode layer; GEMM1
// gained nothing from the same order).
template <bool FP8, int NT, int WT, int NW, int U>
__global__ __launch_bounds__(NW * 64) void gemm2_small_kernel(GemmArgs g, int ntiles) {
    int blk, tile;
    if (!map_active_tile<true>(g, ntiles, blk, tile)) return;
    gemm2_small_tile<FP8, NT, WT, NW, U>(g, blk, tile);
}

// GEMM2, NTILE column tiles of one block per workgroup (block-major over the
// blocks' tile groups)
template <bool FP8, int NT, int WT, int NW, int U, int NTILE>
__global__ __launch_bounds__(NW * 64) void gemm2_tiles_kernel(GemmArgs g, int ngroups) {
    int blk, grp;
    if (!map_active_tile<true>(g, ngroups, blk, grp)) return;
    gemm2_tiles<FP8, NT, WT, NW, U, NTILE>(g, blk, grp * NTILE);
}

template <typename K>
hipError_t launch_tiles(K kernel, const GemmArgs& g, int ntiles, int threads, hipStream_t s) {
    const int64_t n = int64_t(g.num_blocks) * ntiles;
    const int64_t grid = (n + 7) / 8 * 8;
    hipLaunchKernelGGL(kernel, dim3(unsigned(grid)), dim3(threads), 0, s, g, ntiles);
    return hipGetLastError();
}

template <bool FP8, int NT>
hipError_t gemm1_dispatch(const GemmArgs& g, hipStream_t s) {
    if constexpr (FP8) {
        // one 128-column group per workgroup: 4 waves x (32 gate + 32 up)
        // rows, or 8 waves x (16 + 16) for 64-token blocks (registers)
        const int ntiles = g.I / 128;
        if constexpr (NT <= 2)
            return g.krot ? launch_tiles(gemm1_small_kernel<true, NT, 2, 4, 1, true>, g, ntiles, 256, s)
                          : launch_tiles(gemm1_small_kernel<true, NT, 2, 4, 1>, g, ntiles, 256, s);
        else
            return g.krot ? launch_tiles(gemm1_small_kernel<true, NT, 1, 8, 1, true>, g, ntiles, 512, s)
                          : launch_tiles(gemm1_small_kernel<true, NT, 1, 8, 1>, g, ntiles, 512, s);
    } else {
        // 4 waves x (16 gate + 16 up) = 64 columns.  16-row blocks take 8
        // K-steps per register stage (twice the bytes in flight per wave at
        // half the occupancy: 3 % faster on the decode layers); larger blocks
        // would spill at 8.
        const int ntiles = g.I / 64;
        if constexpr (NT == 1) {
            if ((g.H / 32) % 8 == 0) return launch_tiles(gemm1_small_kernel<false, NT, 1, 4, 8>, g, ntiles, 256, s);
        }
        // 64-token blocks: 2 K-steps per stage (4 would need every register
        // and run one wave per SIMD: 1.52 vs 1.36 ms at 64 rows per expert)
        if constexpr (NT < 4) {
            if ((g.H / 32) % 4 == 0) return launch_tiles(gemm1_small_kernel<false, NT, 1, 4, 4>, g, ntiles, 256, s);
        }
        return launch_tiles(gemm1_small_kernel<false, NT, 1, 4, 2>, g, ntiles, 256, s);
    }
}

template <int NT, int WT>
hipError_t gemm2_bf16(const GemmArgs& g, hipStream_t s) {
    constexpr int NW = 4;
    if constexpr (NT < 4) {   // 64-token blocks: 2 K-steps per stage (registers)
        if ((g.I / 32) % 4 == 0)
            return launch_tiles(gemm2_small_kernel<false, NT, WT, NW, 4>, g, g.H / (NW * WT * 16), NW * 64, s);
    }
    return launch_tiles(gemm2_small_kernel<false, NT, WT, NW, 2>, g, g.H / (NW * WT * 16), NW * 64, s);
}

// Column tiles per workgroup, measured on the fp8 layer (1024 tokens, 256
// experts, H 4096, I 256): GEMM2 113 (one tile) / 101.5 (2) / 109 (4) / 110
// (8) / 137 us (16) at 32-token blocks; 145 / 130 / 121 / 126 / 125 us at 64.
template <int NT, int WT>
hipError_t gemm2_fp8(const GemmArgs& g, hipStream_t s) {
    constexpr int NW = 4, kTiles = NT >= 4 ? 4 : 2;
    const int ntiles = g.H / (NW * WT * 16);
    if (ntiles % kTiles == 0 && g.I / 128 <= kTabSteps)
        return launch_tiles(gemm2_tiles_kernel<true, NT, WT, NW, 1, kTiles>, g, ntiles / kTiles, NW * 64, s);
    return launch_tiles(gemm2_small_kernel<true, NT, WT, NW, 1>, g, ntiles, NW * 64, s);
}

template <bool FP8, int NT>
hipError_t gemm2_dispatch(const GemmArgs& g, hipStream_t s) {
    if constexpr (FP8) {
        // K = I is short: 64 output rows per wave keep more bytes in flight
        // (32 for 64-token blocks, registers; 32 when H % 256 != 0)
        if constexpr (NT <= 2) {
            if (small_gemm2_cols(g.T, g.topk, g.E, g.H, true, NT) == 256) return gemm2_fp8<NT, 4>(g, s);
        }
        return gemm2_fp8<NT, 2>(g, s);
    } else {
        // 128 output columns per workgroup, or 64 when H is not a multiple of
        // 128 (narrower tiles for one or two decode tokens measured slower);
        // 256 when a single token's experts leave the grid short of waves
        const int cols = small_gemm2_cols(g.T, g.topk, g.E, g.H, false, NT);
        if (cols == 256) return gemm2_bf16<NT, 4>(g, s);
        if (cols == 128) return gemm2_bf16<NT, 2>(g, s);
        return gemm2_bf16<NT, 1>(g, s);
    }
}

}  // namespace

// GEMM2 output rows of H per workgroup on the weight-streaming path (the
// dispatch above follows the same rule)
int small_gemm2_cols(int T, int topk, int E, int H, bool fp8, int NT) {
    (void)E;
    if (fp8) return (NT <= 2 && H % 256 == 0) ? 256 : 128;
    // at most 8 routed rows (one decode token): 64 output rows per wave ran
    // 12 % faster than 32 (one token, 8 of 256 experts, H 7168, I 2048), and
    // slower from 4 tokens on
    if (NT == 1 && int64_t(T) * topk <= 8 && H % 256 == 0) return 256;
    return H % 128 == 0 ? 128 : 64;
}

hipError_t launch_gemm1_small(const GemmArgs& g, bool fp8, hipStream_t s) {
    switch (g.block_m) {
        case 16: return fp8 ? gemm1_dispatch<true, 1>(g, s) : gemm1_dispatch<false, 1>(g, s);
        case 32: return fp8 ? gemm1_dispatch<true, 2>(g, s) : gemm1_dispatch<false, 2>(g, s);
        case 64: return fp8 ? gemm1_dispatch<true, 4>(g, s) : gemm1_dispatch<false, 4>(g, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm2_small(const GemmArgs& g, bool fp8, hipStream_t s) {
    switch (g.block_m) {
        case 16: return fp8 ? gemm2_dispatch<true, 1>(g, s) : gemm2_dispatch<false, 1>(g, s);
        case 32: return fp8 ? gemm2_dispatch<true, 2>(g, s) : gemm2_dispatch<false, 2>(g, s);
        case 64: return fp8 ? gemm2_dispatch<true, 4>(g, s) : gemm2_dispatch<false, 4>(g, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
