// LDS-tiled grouped GEMMs for many rows per expert (prefill), bf16.
//
// Same orientation as the weight-streaming path: the expert's weight rows are
// the MFMA M side, the block's tokens the N side (so the GEMM1 epilogue keeps a
// gate row and its up row in the same lane and register).  A workgroup owns a
// 256-weight-row x 128-token tile of one expert block and walks K in stages of
// 64: each stage of both operands (256x64 and 128x64 bf16) is loaded from
// global memory into registers one stage ahead, then written to one of two LDS
// buffers, so one barrier per stage separates the writers from the readers.
// LDS rows are 128 bytes; the 16-byte chunk c of row r is stored at chunk
// position c ^ (r & 7), so the 32 lanes of an MFMA fragment read that walk 32
// consecutive rows hit different banks.
//
// MFMA v_mfma_f32_32x32x16_bf16 (layout checked on gfx950): lane l holds row
// (l % 32) of A / column (l % 32) of B at K offset (l / 32) * 8; the 32x32
// result gives lane l column (l % 32) and rows (i / 4) * 8 + (l / 32) * 4 + i % 4.
//
// Token sub-tiles of 32 rows that hold only padding (the tail of an expert's
// last block) are neither loaded nor multiplied.
//
//   GEMM1 (a4+a5): tile = 128 intermediate columns: gate rows c0..c0+127 and
//                  up rows I+c0..; wave w owns gate rows c0+32w.. and the
//                  matching up rows; epilogue a = bf16(bf16(silu(bf16 g)) *
//                  bf16 u) stored in expert-sorted order (P2 sections 1.1, 1.2).
//   GEMM2 (a6):    tile = 256 output columns h; wave w owns h0+64w..+63;
//                  epilogue y[f] = tw[f] * acc in fp32 (P2 section 1.1).
#include "common.h"

namespace moe {

namespace {

constexpr int kTM = 256;           // weight rows per workgroup
constexpr int kBM = 128;           // tokens per workgroup (= block_m of the alignment)
constexpr int kKB = 64;            // K per stage (bf16 elements)
constexpr int kRowBytes = kKB * 2; // 128 bytes per LDS row
constexpr int kThreads = 256;
constexpr int kABytes = kTM * kRowBytes;   // 32 KiB
constexpr int kBBytes = kBM * kRowBytes;   // 16 KiB
constexpr int kALoads = kABytes / 16 / kThreads;   // 8 x 16 B per thread per stage
constexpr int kBLoads = kBBytes / 16 / kThreads;   // 4 x 16 B per thread per stage

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ bool map_tile(int num_blocks, int ntiles, int& blk, int& tile) {
    // hardware deals workgroups round-robin over the 8 XCDs; give each XCD a
    // contiguous run of logical tiles, ordered tile-major so the blocks of one
    // expert (same weight tile) run together on one XCD and share its L2
    const int per_xcd = gridDim.x >> 3;
    const int wg = blockIdx.x;
    const int logical = (wg & 7) * per_xcd + (wg >> 3);
    if (logical >= num_blocks * ntiles) return false;
    tile = logical / num_blocks;
    blk = logical - tile * num_blocks;
    return true;
}

template <int GEMM>
__global__ __launch_bounds__(kThreads, 1) void gemm_large_kernel(GemmArgs g, int ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][kABytes + kBBytes];
    __shared__ int s_valid;

    int blk, tile;
    if (!map_tile(g.num_blocks, ntiles, blk, tile)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int R = g.T * g.topk;
    const int K = GEMM == 1 ? g.H : g.I;
    const int nst = K / kKB;

    // rows of this block that hold real slots (a prefix: padding sits at the end)
    if (tid < 64) {
        const int f0 = g.sorted_ids[blk * kBM + tid];
        const int f1 = g.sorted_ids[blk * kBM + 64 + tid];
        const int n = __popcll(__ballot(f0 < R)) + __popcll(__ballot(f1 < R));
        if (tid == 0) s_valid = n;
    }
    __syncthreads();
    const int nvalid = s_valid;
    const int ntok_tiles = (nvalid + 31) >> 5;   // 32-token sub-tiles with real rows

    // ---- global source pointers --------------------------------------------
    // A: thread tid loads chunk (tid & 7) of rows j*32 + tid/8, j = 0..7
    const int a_chunk = tid & 7;
    const int a_row0 = tid >> 3;
    const uint8_t* a_src[kALoads];
    {
        const uint8_t* w = static_cast<const uint8_t*>(GEMM == 1 ? g.w13 : g.w2);
#pragma unroll
        for (int j = 0; j < kALoads; ++j) {
            const int r = j * 32 + a_row0;   // tile row 0..255
            int grow;
            if (GEMM == 1) {
                // rows 0..127 gate c0+r, 128..255 up I+c0+r-128; wave w reads gate rows
                // [32w, 32w+32) at tile rows [64w, 64w+32) and up rows at [64w+32, 64w+64)
                const int ww = r >> 6, half = (r >> 5) & 1, rr = r & 31;
                const int col = tile * 128 + ww * 32 + rr;
                grow = half ? g.I + col : col;
                grow += e * 2 * g.I;
            } else {
                grow = e * g.H + tile * kTM + r;
            }
            a_src[j] = w + int64_t(grow) * K * 2 + a_chunk * 16;
        }
    }
    const uint8_t* b_src[kBLoads];
    bool b_on[kBLoads];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
        const int r = j * 32 + a_row0;   // token row 0..127
        b_on[j] = r < ntok_tiles * 32;
        const int srow = blk * kBM + r;
        if (GEMM == 1) {
            const int f = g.sorted_ids[srow];
            const int tok = f < R ? f / g.topk : 0;
            b_src[j] = reinterpret_cast<const uint8_t*>(g.x) + int64_t(tok) * K * 2 + a_chunk * 16;
        } else {
            b_src[j] = static_cast<const uint8_t*>(g.inter) + int64_t(srow) * K * 2 + a_chunk * 16;
        }
    }

    i32x4 ra[kALoads], rb[kBLoads];
    auto gload = [&](int st) {
        const int64_t off = int64_t(st) * kRowBytes;
#pragma unroll
        for (int j = 0; j < kALoads; ++j) ra[j] = *reinterpret_cast<const i32x4*>(a_src[j] + off);
#pragma unroll
        for (int j = 0; j < kBLoads; ++j)
            if (b_on[j]) rb[j] = *reinterpret_cast<const i32x4*>(b_src[j] + off);
    };
    auto lstore = [&](int buf) {
        uint8_t* A = lds[buf];
        uint8_t* B = lds[buf] + kABytes;
#pragma unroll
        for (int j = 0; j < kALoads; ++j)
            *reinterpret_cast<i32x4*>(A + swz(j * 32 + a_row0, a_chunk)) = ra[j];
#pragma unroll
        for (int j = 0; j < kBLoads; ++j)
            if (b_on[j]) *reinterpret_cast<i32x4*>(B + swz(j * 32 + a_row0, a_chunk)) = rb[j];
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][u][i] = 0.0f;

    const int fr = lane & 31;   // fragment row / column
    const int fk = lane >> 5;   // fragment K half
    const int arow0 = wv * 64 + fr;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        if (st + 1 < nst) gload(st + 1);
        const uint8_t* A = lds[buf];
        const uint8_t* B = lds[buf] + kABytes;
#pragma unroll
        for (int s = 0; s < kKB / 16; ++s) {
            const int chunk = 2 * s + fk;
            bf16x8 af[2], bfr[4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                af[t] = *reinterpret_cast<const bf16x8*>(A + swz(arow0 + t * 32, chunk));
#pragma unroll
            for (int u = 0; u < 4; ++u)
                bfr[u] = *reinterpret_cast<const bf16x8*>(B + swz(u * 32 + fr, chunk));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (u < ntok_tiles) {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bfr[u], acc[t][u], 0, 0, 0);
                }
            }
        }
        if (st + 1 < nst) {
            lstore(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogues -----------------------------------------------------------
    if constexpr (GEMM == 1) {
        uint16_t* out = static_cast<uint16_t*>(g.inter);
        const int colw = tile * 128 + wv * 32;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u >= ntok_tiles) continue;
            const int row = blk * kBM + u * 32 + fr;
#pragma unroll
            for (int q = 0; q < 4; ++q) {   // groups of 4 consecutive columns
                uint32_t p[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int i0 = q * 4 + 2 * h;
                    const float a0 = silu_mul_bf16(round_bf16(acc[0][u][i0]), round_bf16(acc[1][u][i0]));
                    const float a1 = silu_mul_bf16(round_bf16(acc[0][u][i0 + 1]), round_bf16(acc[1][u][i0 + 1]));
                    p[h] = uint32_t(f32_to_bf16_rne(a0)) | (uint32_t(f32_to_bf16_rne(a1)) << 16);
                }
                const int col = colw + q * 8 + fk * 4;
                *reinterpret_cast<i32x2*>(out + int64_t(row) * g.I + col) = i32x2{int(p[0]), int(p[1])};
            }
        }
    } else {
        const int hw = tile * kTM + wv * 64;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u >= ntok_tiles) continue;
            const int f = g.sorted_ids[blk * kBM + u * 32 + fr];
            if (f >= R) continue;
            const float tw = g.topk_weights[f];
            float* yrow = g.y + int64_t(f) * g.H;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(acc[t][u][q * 4 + j], tw);
                    *reinterpret_cast<f32x4*>(yrow + hw + t * 32 + q * 8 + fk * 4) = v;
                }
        }
    }
}

template <typename Kern>
hipError_t launch(Kern kernel, const GemmArgs& g, int ntiles, hipStream_t s) {
    const int64_t n = int64_t(g.num_blocks) * ntiles;
    const int64_t grid = (n + 7) / 8 * 8;
    hipLaunchKernelGGL(kernel, dim3(unsigned(grid)), dim3(kThreads), 0, s, g, ntiles);
    return hipGetLastError();
}

}  // namespace

bool gemm_large_supported(int H, int I, bool fp8) {
    return !fp8 && I % 128 == 0 && H % kTM == 0 && H % kKB == 0 && I % kKB == 0;
}

int gemm_large_block_m() { return kBM; }

hipError_t launch_gemm1_large(const GemmArgs& g, bool fp8, hipStream_t s) {
    if (fp8 || g.block_m != kBM) return hipErrorInvalidValue;
    return launch(gemm_large_kernel<1>, g, g.I / 128, s);
}

hipError_t launch_gemm2_large(const GemmArgs& g, bool fp8, hipStream_t s) {
    if (fp8 || g.block_m != kBM) return hipErrorInvalidValue;
    return launch(gemm_large_kernel<2>, g, g.H / kTM, s);
}

}  // namespace moe
