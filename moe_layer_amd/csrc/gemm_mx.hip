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

// ----------------------------------------------------------------------------
// MXFP8 down GEMM of 16-row blocks through LDS (I <= 256), the form of the
// block-fp8 one in gemm_small.hip: 4 waves x 16 rows of a 64-row column tile,
// W2 moved global -> LDS by direct-to-LDS loads of 8 whole 128-byte row
// pieces into a 3-slot ring, a stage = one 128-K step of one tile, 8 adjacent
// tiles (512 output rows) walked as one stream of stages.  The block's token
// rows, their E8M0 bytes and the workgroup's weight-scale bytes (512 rows:
// one contiguous 4 KB run in the packed and in the row-major layout) are
// staged in LDS once.  Each lane passes the scaled instruction the 32 bytes
// it takes from memory in gemm2_mx_tiles (K [16 g, 16 g + 16) and
// [64 + 16 g, 64 + 16 g + 16) of the step, g = lane / 16: LDS chunks g and
// 4 + g) and the same scale bytes, in the same K order: y is bitwise the same.
// ----------------------------------------------------------------------------
constexpr int kMxLdsRows = 64;                         // output rows per column tile
constexpr int kMxLdsTiles = 8;                         // column tiles per workgroup
constexpr int kMxLdsMaxSteps = 2;                      // I <= 256
constexpr int kMxLdsRowBytes = 128;
constexpr int kMxLdsNB = 3;
constexpr int kMxLdsSlot = kMxLdsRows * kMxLdsRowBytes;
constexpr int kMxLdsTok = kMxLdsMaxSteps * 16 * kMxLdsRowBytes;                 // token rows
constexpr int kMxLdsWsc = kMxLdsTiles * kMxLdsRows * kMxLdsMaxSteps * 4;        // weight E8M0 bytes
constexpr int kMxLdsTsc = 16 * kMxLdsMaxSteps * 4;                              // token E8M0 bytes

template <int N>
__device__ __forceinline__ void mx_wait_vm_n() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int NLD, int MAXA>
__device__ __forceinline__ void mx_wait_stages(int ahead) {
    if constexpr (MAXA <= 0) {
        mx_wait_vm_n<0>();
    } else {
        if (ahead >= MAXA) mx_wait_vm_n<MAXA * NLD>();
        else mx_wait_stages<NLD, MAXA - 1>(ahead);
    }
}

__global__ __launch_bounds__(256) void gemm2_mx_lds_kernel(GemmArgs g, int ngroups) {
    typedef __attribute__((address_space(3))) uint8_t lds_t;
    typedef const __attribute__((address_space(3))) i32x4 lds_v4;
    // one LDS object: with several, the compiler waits for every
    // direct-to-LDS load before each LDS read
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kMxLdsNB * kMxLdsSlot + kMxLdsTok + kMxLdsWsc + kMxLdsTsc];
    uint8_t* tok = ring + kMxLdsNB * kMxLdsSlot;
    uint8_t* wsc = tok + kMxLdsTok;
    uint8_t* tsc = wsc + kMxLdsWsc;
    constexpr int D = kMxLdsNB - 1;
    int blk, grp;
    if (!map_active_tile<true>(g, ngroups, blk, grp)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int ns = I / kStepK;                      // 128-K steps per tile
    const int kbi = I / kMxBlock;                   // E8M0 bytes per row
    const int V = kMxLdsTiles * ns;
    const int h00 = grp * kMxLdsTiles * kMxLdsRows;
    const int lr = lane & 15, lk = lane >> 4;

    const int f = g.sorted_ids[blk * 16 + lr];
    const bool upper = (__ballot(f < R) & 0xff00ull) != 0;
    const float tw = f < R ? gemm2_row_weight(g, f) : 0.0f;

    // scale bytes: the workgroup's 512 weight rows (a contiguous run in either
    // layout) and the block's 16 token rows
    {
        const uint8_t* ws = static_cast<const uint8_t*>(g.w2_scale) + (size_t(e) * H + h00) * kbi;
        for (int i = threadIdx.x; i < kMxLdsTiles * kMxLdsRows * kbi / 4; i += 256)
            reinterpret_cast<uint32_t*>(wsc)[i] = reinterpret_cast<const uint32_t*>(ws)[i];
        const uint8_t* ts = reinterpret_cast<const uint8_t*>(g.inter_scale) + size_t(blk) * 16 * kbi;
        for (int i = threadIdx.x; i < 16 * kbi / 4; i += 256)
            reinterpret_cast<uint32_t*>(tsc)[i] = reinterpret_cast<const uint32_t*>(ts)[i];
    }
    const uint32_t ch0 = uint32_t((lane & 7) ^ ((lane >> 4) & 7)) << 4;
    const uint32_t ch1 = uint32_t((lane & 7) ^ (((lane >> 4) + 4) & 7)) << 4;
    // the token tile: step k, 8-row group q at LDS rows 16 k + 8 q + lane / 8
    const uint8_t* inter = static_cast<const uint8_t*>(g.inter) + (size_t(blk) * 16 + (lane >> 3)) * I;
    for (int i = wv; i < 2 * ns; i += 4) {
        const int k = i >> 1, q = i & 1;
        if (q == 1 && !upper) continue;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(inter + size_t(8 * q) * I + k * kStepK +
                                                                       (q ? ch1 : ch0)),
                                         (lds_t*)(tok) + (16 * k + 8 * q) * kMxLdsRowBytes, 16, 0, 0);
    }
    const uint8_t* wsrc = static_cast<const uint8_t*>(g.w2) + (size_t(e) * H + h00 + wv * 16 + (lane >> 3)) * I;
    auto issue = [&](int v) {
        const int t = v / ns, k = v - t * ns;
        lds_t* slot = (lds_t*)(ring) + (v % kMxLdsNB) * kMxLdsSlot + wv * 2048;
        const uint8_t* src = wsrc + size_t(t) * kMxLdsRows * I + k * kStepK;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + ch0), slot, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + size_t(8) * I + ch1), slot + 1024, 16,
                                         0, 0);
    };
    for (int v = 0; v < D && v < V; ++v) issue(v);
    mx_wait_vm_n<0>();
    __syncthreads();

    // fragment reads: chunks lk and 4 + lk of row r
    const int arow = wv * 16 + lr;
    const uint32_t a0 = uint32_t(arow * kMxLdsRowBytes + ((lk ^ ((arow >> 1) & 7)) << 4));
    const uint32_t a1 = uint32_t(arow * kMxLdsRowBytes + (((4 + lk) ^ ((arow >> 1) & 7)) << 4));
    // the lane's weight-scale byte: packed [row group][step][64], row-major [row][kbi]
    const int sa_lane = g.mx_packed ? lr + 16 * lk : lr * kbi + lk;
    f32x4 acc = {0, 0, 0, 0};
    for (int v = 0; v < V; ++v) {
        mx_wait_stages<2, D - 1>(min(v + D - 1, V - 1) - v);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (v + D < V) issue(v + D);
        const int t = v / ns, k = v - t * ns;
        const lds_t* slot = (const lds_t*)(ring) + (v % kMxLdsNB) * kMxLdsSlot;
        const int brow = 16 * k + lr;
        const lds_t* tb = (const lds_t*)(tok) + brow * kMxLdsRowBytes;
        const i32x4 x0 = *reinterpret_cast<lds_v4*>(slot + a0);
        const i32x4 x1 = *reinterpret_cast<lds_v4*>(slot + a1);
        const i32x4 y0 = *reinterpret_cast<lds_v4*>(tb + ((lk ^ ((brow >> 1) & 7)) << 4));
        const i32x4 y1 = *reinterpret_cast<lds_v4*>(tb + (((4 + lk) ^ ((brow >> 1) & 7)) << 4));
        const int rg = t * 4 + wv;   // the wave's 16-row group inside the workgroup's rows
        const uint32_t sa = g.mx_packed ? wsc[(rg * ns + k) * 64 + sa_lane]
                                        : wsc[(rg * 16) * kbi + sa_lane + 4 * k];
        const uint32_t sb = tsc[lr * kbi + 4 * k + lk];
        const i32x8 av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const i32x8 bv = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, int(sa), 0, int(sb));
        if (k == ns - 1) {
            if (f < R) {
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = __fmul_rn(acc[j], tw);
                store_y4<true>(g.y, int64_t(f) * H + h00 + t * kMxLdsRows + wv * 16 + 4 * lk, o);
            }
            acc = f32x4{0, 0, 0, 0};
        }
    }
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
    if constexpr (NT == 1) {
        if (g.H % (kMxLdsTiles * kMxLdsRows) == 0 && g.I / kStepK <= kMxLdsMaxSteps)
            return launch_tiles(gemm2_mx_lds_kernel, g, g.H / (kMxLdsTiles * kMxLdsRows), 256, s);
    }
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
