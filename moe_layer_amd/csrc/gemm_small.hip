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

// ----------------------------------------------------------------------------
// Down GEMM (a6) for 16-row blocks, its weights streamed through LDS.
//
// gemm2_small_kernel loads every lane's 16-byte operand pieces straight into
// registers, so each load instruction touches 32 bytes of 16 different W2
// rows.  Here the weights move global -> LDS with direct-to-LDS loads (lane
// i's 16 bytes land at the instruction's LDS base + 16 i), each instruction
// covering 8 whole 128-byte row pieces, through a kNB-slot ring kNB - 1 stages
// deep.  A workgroup of 4 waves owns 64 output rows (16 per wave) of one
// expert block; a stage is 64 K (two MFMA steps); the block's 16 token rows of
// the stage ride in the same slot (rows 64..79; the second 8-row group only
// when it holds a routed row).  Waves 0..3 each load 16 weight rows, waves 0
// and 1 one token group: each waits for its own loads, then one barrier per
// stage publishes the slot and frees the slot read in the previous stage.
// LDS rows are 128 bytes with chunk c of row r at position c ^ ((r >> 1) & 7),
// so a fragment read (16 rows at one chunk) hits distinct banks.
//
// Operands, MFMA (16x16x32 bf16), K order and epilogue are gemm2_small_tile's
// for one 16-token tile, so y is bitwise the same.
// ----------------------------------------------------------------------------
constexpr int kLdsRows = 64;                       // output rows per workgroup
constexpr int kLdsRowBytes = 128;                  // K bytes of a row per stage
constexpr int kLdsSlot = (kLdsRows + 16) * kLdsRowBytes;

template <int N>
__device__ __forceinline__ void wait_vm_n() {
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// wait until at most `ahead` stages of NLD loads each are still in flight
template <int NLD, int MAXA>
__device__ __forceinline__ void wait_stages(int ahead) {
    if constexpr (MAXA <= 0) {
        wait_vm_n<0>();
    } else {
        if (ahead >= MAXA) wait_vm_n<MAXA * NLD>();
        else wait_stages<NLD, MAXA - 1>(ahead);
    }
}

template <int kNB>
__global__ __launch_bounds__(256) void gemm2_lds_kernel(GemmArgs g, int ntiles) {
    typedef __attribute__((address_space(3))) uint8_t lds_t;
    typedef const __attribute__((address_space(3))) i32x4 lds_v4;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kNB * kLdsSlot];
    constexpr int D = kNB - 1;
    int blk, tile;
    if (!map_active_tile<true>(g, ntiles, blk, tile)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int nst = I / 64;
    const int h0 = tile * kLdsRows;
    const int lr = lane & 15, lk = lane >> 4;

    // this lane's token row of the block; rows 8..15 loaded only if one is routed
    const int f = g.sorted_ids[blk * 16 + lr];
    const bool upper = (__ballot(f < R) & 0xff00ull) != 0;
    const bool tok_loader = wv == 0 || (wv == 1 && upper);

    // load sources: load q of wave w fills LDS rows 16 w + 8 q + lane / 8 at
    // position lane % 8, the token group t rows 64 + 8 t + lane / 8; both with
    // chunk (lane % 8) ^ ((row >> 1) & 7) = (lane % 8) ^ ((lane / 16 + 4 q) % 8)
    const uint32_t ch0 = uint32_t((lane & 7) ^ ((lane >> 4) & 7)) << 4;
    const uint32_t ch1 = uint32_t((lane & 7) ^ (((lane >> 4) + 4) & 7)) << 4;
    const size_t rowb = size_t(I) * 2;
    const uint8_t* wsrc = static_cast<const uint8_t*>(g.w2) + (size_t(e) * H + h0 + wv * 16 + (lane >> 3)) * rowb;
    const uint8_t* tsrc = static_cast<const uint8_t*>(g.inter) + (size_t(blk) * 16 + wv * 8 + (lane >> 3)) * rowb +
                          ((wv & 1) ? ch1 : ch0);
    auto issue = [&](int st) {
        lds_t* slot = (lds_t*)(ring) + (st % kNB) * kLdsSlot;
        const size_t k0 = size_t(st) * kLdsRowBytes;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(wsrc + k0 + ch0), slot + wv * 2048, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(wsrc + 8 * rowb + k0 + ch1),
                                         slot + wv * 2048 + 1024, 16, 0, 0);
        if (tok_loader)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tsrc + k0),
                                             slot + kLdsRows * kLdsRowBytes + wv * 1024, 16, 0, 0);
    };
    // fragment reads: row r at chunk 4 j + lane / 16 (MFMA step j of the stage)
    const int arow = wv * 16 + lr, brow = kLdsRows + lr;
    uint32_t aoff[2], boff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        aoff[j] = uint32_t(arow * kLdsRowBytes + (((4 * j + lk) ^ ((arow >> 1) & 7)) << 4));
        boff[j] = uint32_t(brow * kLdsRowBytes + (((4 * j + lk) ^ ((brow >> 1) & 7)) << 4));
    }

    f32x4 acc = {0, 0, 0, 0};
    for (int st = 0; st < D && st < nst; ++st) issue(st);
    for (int s = 0; s < nst; ++s) {
        const int ahead = min(s + D - 1, nst - 1) - s;   // stages issued beyond s
        if (tok_loader) wait_stages<3, D - 1>(ahead);
        else wait_stages<2, D - 1>(ahead);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (s + D < nst) issue(s + D);
        const lds_t* slot = (const lds_t*)(ring) + (s % kNB) * kLdsSlot;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const i32x4 a = *reinterpret_cast<lds_v4*>(slot + aoff[j]);
            const i32x4 b = *reinterpret_cast<lds_v4*>(slot + boff[j]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                          acc, 0, 0, 0);
        }
    }
    if (f >= R) return;
    const float tw = gemm2_row_weight(g, f);
    f32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(acc[j], tw);
    store_y4<false>(g.y, int64_t(f) * H + h0 + wv * 16 + 4 * lk, v);
}

// ----------------------------------------------------------------------------
// fp8 (128x128 block scales) down GEMM of 16-row blocks through LDS.
//
// The weights stream as in gemm2_lds_kernel (4 waves x 16 rows of a 64-row
// column tile, two direct-to-LDS loads of 8 whole 128-byte row pieces per wave
// and stage, a kNB-slot ring); a stage is one 128-K weight-scale block of one
// tile.  K = I is short (up to 256 here: two stages), so a workgroup walks
// kLdsQTiles adjacent column tiles of its block as one stream of stages,
// storing each tile when its last block is in.  The block's 16
// token rows (all of I, with their group scales) and the weight-block scales
// of the workgroup's rows are staged in LDS once.  Per tile the arithmetic is
// gemm2_tiles' (one fp8 MFMA per 128-K block, its sums scaled by weight-block
// x token-group scale with one fma), so y is bitwise the same.  Measured on
// the fp8 layer (E 256, H 4096, I 256) at 64 / 256 / 512 tokens, down GEMM
// 56 / 70 / 83 us in registers, 53 / 65 / 71 us here (512 rows per workgroup,
// a 3-slot ring: the smallest LDS footprint, most workgroups per CU, measured
// best among 128-1024 rows and 3-6 slots).
// ----------------------------------------------------------------------------
constexpr int kLdsQTiles = 8;                     // column tiles per workgroup (512 output rows)
constexpr int kLdsQMaxKb = 2;                     // I <= 256 (LDS for more workgroups per CU)
constexpr int kLdsQSlot = kLdsRows * kLdsRowBytes;
constexpr int kLdsQTok = kLdsQMaxKb * 16 * kLdsRowBytes;                  // the block's token rows
constexpr int kLdsQWsc = kLdsQTiles * kLdsRows / kGroup * kLdsQMaxKb;     // weight-block scales (floats)
constexpr int kLdsQTsc = 16 * kLdsQMaxKb;                                 // token-group scales (floats)

template <int kNB>
__global__ __launch_bounds__(256) void gemm2_lds_fp8_kernel(GemmArgs g, int ngroups) {
    typedef __attribute__((address_space(3))) uint8_t lds_t;
    typedef const __attribute__((address_space(3))) i32x4 lds_v4;
    // one LDS object (ring, token rows, scale tables): with several, the
    // compiler waits for every direct-to-LDS load before each LDS read
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kNB * kLdsQSlot + kLdsQTok + 4 * (kLdsQWsc + kLdsQTsc)];
    uint8_t* tok = ring + kNB * kLdsQSlot;
    float* wsc = reinterpret_cast<float*>(tok + kLdsQTok);
    float* tsc = wsc + kLdsQWsc;
    constexpr int D = kNB - 1;
    int blk, grp;
    if (!map_active_tile<true>(g, ngroups, blk, grp)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int nkb = I / kGroup;
    const int V = kLdsQTiles * nkb;                 // stages: tile t = v / nkb, K block v % nkb
    const int h00 = grp * kLdsQTiles * kLdsRows;    // first output row of the workgroup
    const int lr = lane & 15, lk = lane >> 4;

    const int f = g.sorted_ids[blk * 16 + lr];
    const bool upper = (__ballot(f < R) & 0xff00ull) != 0;
    const float tw = f < R ? gemm2_row_weight(g, f) : 0.0f;

    // scale tables: weight blocks of the workgroup's 8 row blocks, the tokens' groups
    const float* w2s = static_cast<const float*>(g.w2_scale) + (size_t(e) * (H / kGroup) + h00 / kGroup) * nkb;
    for (int i = threadIdx.x; i < (kLdsQTiles * kLdsRows / kGroup) * nkb; i += 256) wsc[i] = w2s[i];
    for (int i = threadIdx.x; i < 16 * nkb; i += 256) tsc[i] = g.inter_scale[size_t(blk) * 16 * nkb + i];

    // load sources (as in gemm2_lds_kernel): chunk (lane % 8) ^ ((lane / 16 + 4 q) % 8)
    const uint32_t ch0 = uint32_t((lane & 7) ^ ((lane >> 4) & 7)) << 4;
    const uint32_t ch1 = uint32_t((lane & 7) ^ (((lane >> 4) + 4) & 7)) << 4;
    // the token tile: K block k, 8-row group q at LDS rows 16 k + 8 q + lane / 8
    const uint8_t* inter = static_cast<const uint8_t*>(g.inter) + (size_t(blk) * 16 + (lane >> 3)) * I;
    for (int i = wv; i < 2 * nkb; i += 4) {
        const int k = i >> 1, q = i & 1;
        if (q == 1 && !upper) continue;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(inter + size_t(8 * q) * I + k * kGroup +
                                                                       (q ? ch1 : ch0)),
                                         (lds_t*)(tok) + (16 * k + 8 * q) * kLdsRowBytes, 16, 0, 0);
    }
    const uint8_t* wsrc = static_cast<const uint8_t*>(g.w2) + (size_t(e) * H + h00 + wv * 16 + (lane >> 3)) * I;
    auto issue = [&](int v) {
        const int t = v / nkb, k = v - t * nkb;
        lds_t* slot = (lds_t*)(ring) + (v % kNB) * kLdsQSlot + wv * 2048;
        const uint8_t* src = wsrc + size_t(t) * kLdsRows * I + k * kGroup;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + ch0), slot, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + size_t(8) * I + ch1), slot + 1024, 16, 0,
                                         0);
    };
    for (int v = 0; v < D && v < V; ++v) issue(v);
    wait_vm_n<0>();
    __syncthreads();

    // fragment reads: the lane's 32 bytes (chunks 2 lk, 2 lk + 1) of row r
    const int arow = wv * 16 + lr;
    const uint32_t a0 = uint32_t(arow * kLdsRowBytes + (((2 * lk) ^ ((arow >> 1) & 7)) << 4));
    const uint32_t a1 = uint32_t(arow * kLdsRowBytes + (((2 * lk + 1) ^ ((arow >> 1) & 7)) << 4));
    f32x4 acc = {0, 0, 0, 0};
    for (int v = 0; v < V; ++v) {
        const int ahead = min(v + D - 1, V - 1) - v;
        wait_stages<2, D - 1>(ahead);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        if (v + D < V) issue(v + D);
        const int t = v / nkb, k = v - t * nkb;
        const lds_t* slot = (const lds_t*)(ring) + (v % kNB) * kLdsQSlot;
        const int brow = 16 * k + lr;
        const lds_t* tb = (const lds_t*)(tok) + brow * kLdsRowBytes;
        const i32x4 x0 = *reinterpret_cast<lds_v4*>(slot + a0);
        const i32x4 x1 = *reinterpret_cast<lds_v4*>(slot + a1);
        const i32x4 y0 = *reinterpret_cast<lds_v4*>(tb + (((2 * lk) ^ ((brow >> 1) & 7)) << 4));
        const i32x4 y1 = *reinterpret_cast<lds_v4*>(tb + (((2 * lk + 1) ^ ((brow >> 1) & 7)) << 4));
        const i32x8 av = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const i32x8 bv = {y0[0], y0[1], y0[2], y0[3], y1[0], y1[1], y1[2], y1[3]};
        const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{0, 0, 0, 0}, 0, 0, 0, 0, 0, 0);
        const float c = __fmul_rn(wsc[((t * kLdsRows + wv * 16) / kGroup) * nkb + k], tsc[lr * nkb + k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_fmaf(p[j], c, acc[j]);
        if (k == nkb - 1) {
            if (f < R) {
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = __fmul_rn(acc[j], tw);
                store_y4<true>(g.y, int64_t(f) * H + h00 + t * kLdsRows + wv * 16 + 4 * lk, o);
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
        if constexpr (NT == 1) {
            if (gemm2_lds_fp8_supported(g.H, g.I))
                return launch_tiles(gemm2_lds_fp8_kernel<3>, g, g.H / (kLdsQTiles * kLdsRows), 256, s);
        }
        if constexpr (NT <= 2) {
            if (small_gemm2_cols(g.T, g.topk, g.E, g.H, g.I, true, NT) == 256) return gemm2_fp8<NT, 4>(g, s);
        }
        return gemm2_fp8<NT, 2>(g, s);
    } else {
        // 16-row blocks stream their weights through LDS (gemm2_lds_kernel);
        // otherwise 128 output columns per workgroup, or 64 when H is not a
        // multiple of 128; 256 when a single token's experts leave the grid
        // short of waves
        if constexpr (NT == 1) {
            if (gemm2_lds_supported(g.H, g.I)) return launch_tiles(gemm2_lds_kernel<4>, g, g.H / kLdsRows, 256, s);
        }
        const int cols = small_gemm2_cols(g.T, g.topk, g.E, g.H, g.I, false, NT);
        if (cols == 256) return gemm2_bf16<NT, 4>(g, s);
        if (cols == 128) return gemm2_bf16<NT, 2>(g, s);
        return gemm2_bf16<NT, 1>(g, s);
    }
}

}  // namespace

bool gemm2_lds_supported(int H, int I) { return H % kLdsRows == 0 && I % 64 == 0; }
bool gemm2_lds_fp8_supported(int H, int I) {
    return H % (kLdsQTiles * kLdsRows) == 0 && I % kGroup == 0 && I / kGroup <= kLdsQMaxKb;
}

// GEMM2 output rows of H per workgroup on the weight-streaming path (the
// dispatch above follows the same rule)
int small_gemm2_cols(int T, int topk, int E, int H, int I, bool fp8, int NT, bool mx) {
    (void)E;
    // gemm2_lds_fp8_kernel, and gemm2_mx_lds_kernel (gemm_mx.hip) on the same shapes
    (void)mx;
    if (fp8 && NT == 1 && gemm2_lds_fp8_supported(H, I)) return kLdsRows;
    if (fp8) return (NT <= 2 && H % 256 == 0) ? 256 : 128;
    if (NT == 1 && gemm2_lds_supported(H, I)) return kLdsRows;   // gemm2_lds_kernel
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
