// LDS-tiled grouped GEMMs for many rows per expert (prefill), bf16.
//
// Same orientation as the weight-streaming path: the expert's weight rows are
// the MFMA M side, the block's tokens the N side (so the GEMM1 epilogue keeps a
// gate row and its up row in the same lane and register).  A workgroup of 8
// waves owns a 256-weight-row x 256-token tile of one expert block: wave
// (wm, wn) = (w & 3, w >> 2) owns weight rows 64wm..64wm+63 and the token
// sub-tiles u (32 rows each) with u % 2 == wn, so the live sub-tiles of a
// block's partly filled tail split evenly between the two waves of a SIMD.
// K is walked in stages of 64: both operand tiles of the next stage (256x64
// bf16 each, 64 KiB; 320 token rows with a following short block, below) are
// loaded into registers while the current stage is multiplied from LDS, then
// written to the other of two LDS buffers; one barrier per stage (32 MFMAs per
// wave).  Every LDS access is ordinary code, so the compiler interleaves the
// fragment reads with the MFMAs.
//
// LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r sits at
// position c ^ ((r >> 1) & 7), which spreads the 32 rows a fragment read
// touches evenly over the banks (for 32 and for 64 four-byte banks).
//
// MFMA v_mfma_f32_32x32x16_bf16 (layout checked on gfx950): lane l holds row
// (l % 32) of A / column (l % 32) of B at K offset (l / 32) * 8; the 32x32
// result gives lane l column (l % 32) and rows (i / 4) * 8 + (l / 32) * 4 + i % 4.
//
// Token sub-tiles that hold only padding (the tail of an expert's last block)
// are neither multiplied nor stored: the main loop is instantiated per wave for
// 0..4 live sub-tiles.  An expert's last block with at most 64 real rows is
// taken by the workgroup of the expert's previous (full) block as token rows
// 256..319 (sub-tiles 8 and 9, so 4 or 5 per wave): the expert's weight tiles
// stream once for both blocks.  With routing near 256 rows per expert about
// half of the experts end in such a block, which otherwise re-streams every
// weight tile for a few rows (prefill layer: 1.52x the algorithmic HBM bytes;
// GEMM1 1.28 -> 1.20 ms, GEMM2 0.69 -> 0.66 ms).
//
//   GEMM1 (a4+a5): tile = 128 intermediate columns: gate rows c0..c0+127 and
//                  up rows I+c0..; wave (wm, .) owns gate rows c0+32wm.. and
//                  the matching up rows; epilogue a = bf16(bf16(silu(bf16 g)) *
//                  bf16 u) stored in expert-sorted order (P2 sections 1.1, 1.2).
//   GEMM2 (a6):    tile = 256 output columns h; wave (wm, .) owns h0+64wm..;
//                  epilogue y[f] = tw[f] * acc in fp32 (P2 section 1.1).
//   The layer variants (router weight on the input, SwiGLU clamp) act in the
//   epilogues as in the weight-streaming kernels.
#include "common.h"

namespace moe {

namespace {

constexpr int kTM = 256;           // weight rows per workgroup
constexpr int kBM = 256;           // tokens per workgroup (= block_m of the alignment)
constexpr int kKB = 64;            // K per stage (bf16 elements)
constexpr int kRowBytes = kKB * 2; // 128 bytes per LDS row
constexpr int kWM = 4;                         // wave groups along the weight rows
constexpr int kWaves = 2 * kWM;                // x 2 along the tokens
constexpr int kThreads = 64 * kWaves;
constexpr int kTW = kTM / kWM;                 // weight rows per wave
constexpr int kTA = kTW / 32;                  // 32-row A fragments per wave
constexpr int kXR = 64;            // rows a workgroup may take from the expert's next block
constexpr int kBR = kBM + kXR;     // token rows of the LDS token tile
constexpr int kTileBytes = kTM * kRowBytes;         // weight stage: 32 KiB
constexpr int kBTileBytes = kBR * kRowBytes;        // token stage: 40 KiB
constexpr int kStageBytes = kTileBytes + kBTileBytes;
constexpr int kLoads = kTileBytes / 16 / kThreads;  // 16-byte loads per thread per weight stage
constexpr int kLoadRows = kThreads / 8;              // tile rows one load step covers (8 chunks a row)
constexpr int kLoadsB = kBR / kLoadRows;             // token load steps with the next block's rows
static_assert(kLoads * kLoadRows == kTM, "the loader must cover the weight tile rows exactly once");
static_assert(kLoadsB == kLoads + 1 && kXR == kLoadRows, "the next block's rows take one token load step");

__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4); }

// valid: the block's real rows (a prefix).  kSkip: token rows of whole load
// steps past it are neither loaded nor written to LDS (only padding-only
// sub-tiles read those rows, and they are not multiplied); the other form
// keeps its loads unconditional.
template <int GEMM, int NU, bool kSkip, bool kExt>
__device__ __forceinline__ void run_tile(const GemmArgs& g, uint8_t* lds, int blk, int tile, int e, int valid) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv % kWM, wn = wv / kWM;
    const int R = g.T * g.topk;
    const int K = GEMM == 1 ? g.H : g.I;
    const int nst = K / kKB;
    const int64_t kbytes = int64_t(K) * 2;

    // ---- global sources: thread tid moves chunk (tid & 7) of rows j*kLoadRows + tid/8
    const int chunk = tid & 7;
    const int row0 = tid >> 3;   // 0..kLoadRows-1
    constexpr int kLB = kExt ? kLoadsB : kLoads;   // token load steps
    const uint8_t* a_src[kLoads];
    const uint8_t* b_src[kLB];
#pragma unroll
    for (int j = 0; j < kLB; ++j) {
        const int r = j * kLoadRows + row0;   // tile row 0..255 (token rows to 319 with kExt)
        if constexpr (GEMM == 1) {
            // tile row r = kTW*w + (kTW/2)*half + rr: weight-wave w's gate rows, then its up rows
            if (j < kLoads) {
                const int half = (r / (kTW / 2)) & 1, rr = r % (kTW / 2);
                const int64_t grow =
                    int64_t(e) * 2 * g.I + (half ? g.I : 0) + tile * 128 + (r / kTW) * (kTW / 2) + rr;
                a_src[j] = static_cast<const uint8_t*>(g.w13) + grow * kbytes + chunk * 16;
            }
            const int f = g.sorted_ids[blk * kBM + r];
            const int tok = f < R ? f / g.topk : 0;   // padding rows read token 0 (never stored as real rows)
            b_src[j] = reinterpret_cast<const uint8_t*>(g.x) + int64_t(tok) * kbytes + chunk * 16;
        } else {
            if (j < kLoads) {
                const int64_t grow = int64_t(e) * g.H + tile * kTM + r;
                a_src[j] = static_cast<const uint8_t*>(g.w2) + grow * kbytes + chunk * 16;
            }
            b_src[j] = static_cast<const uint8_t*>(g.inter) + int64_t(blk * kBM + r) * kbytes + chunk * 16;
        }
    }
    i32x4 ra[kLoads], rb[kLB];
    auto gload = [&](int st) {
        const int64_t off = int64_t(st) * kRowBytes;
#pragma unroll
        for (int j = 0; j < kLB; ++j) {
            if (j < kLoads) ra[j] = *reinterpret_cast<const i32x4*>(a_src[j] + off);
            if (!kSkip || j * kLoadRows < valid) rb[j] = *reinterpret_cast<const i32x4*>(b_src[j] + off);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* A = lds + buf * kStageBytes;
        uint8_t* B = A + kTileBytes;
#pragma unroll
        for (int j = 0; j < kLB; ++j) {
            if (j < kLoads) *reinterpret_cast<i32x4*>(A + swz(j * kLoadRows + row0, chunk)) = ra[j];
            if (!kSkip || j * kLoadRows < valid)
                *reinterpret_cast<i32x4*>(B + swz(j * kLoadRows + row0, chunk)) = rb[j];
        }
    };

    f32x16 acc[kTA][NU > 0 ? NU : 1];
#pragma unroll
    for (int t = 0; t < kTA; ++t)
#pragma unroll
        for (int u = 0; u < (NU > 0 ? NU : 1); ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[t][u][i] = 0.0f;

    const int fr = lane & 31;   // fragment row / column
    const int fk = lane >> 5;   // fragment K half
    const int arow = wm * kTW + fr;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int st = 0; st < nst; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nst;
        if (more) gload(st + 1);
        const uint8_t* A = lds + buf * kStageBytes;
        const uint8_t* B = A + kTileBytes;
#pragma unroll
        for (int s = 0; s < kKB / 16; ++s) {
            const int c = 2 * s + fk;
            i32x4 af[kTA], bf[NU > 0 ? NU : 1];
#pragma unroll
            for (int t = 0; t < kTA; ++t) af[t] = *reinterpret_cast<const i32x4*>(A + swz(arow + t * 32, c));
#pragma unroll
            for (int u = 0; u < NU; ++u) bf[u] = *reinterpret_cast<const i32x4*>(B + swz((2 * u + wn) * 32 + fr, c));
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int t = 0; t < kTA; ++t)
                    acc[t][u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, af[t]),
                                                                        __builtin_bit_cast(bf16x8, bf[u]),
                                                                        acc[t][u], 0, 0, 0);
        }
        if (more) {
            lstore(buf ^ 1);
            __syncthreads();
        }
    }

    // ---- epilogues: wave sub-tile u sits at token rows (2u + wn) * 32 ---------
    if constexpr (GEMM == 1) {
        uint16_t* out = static_cast<uint16_t*>(g.inter);
        constexpr int kG = kTA / 2;   // gate fragments per wave; up fragment t + kG pairs with gate t
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int row = blk * kBM + (2 * u + wn) * 32 + fr;
            const float w_in = gemm1_row_weight(g, g.sorted_ids[row]);
#pragma unroll
            for (int t = 0; t < kG; ++t) {
                const int colw = tile * 128 + wm * (kTW / 2) + t * 32;
#pragma unroll
                for (int q = 0; q < 4; ++q) {   // groups of 4 consecutive columns
                    uint32_t p[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i0 = q * 4 + 2 * h;
                        const float a0 =
                            swiglu_bf16(acc[t][u][i0], acc[t + kG][u][i0], w_in, g.clamp, g.clamp_limit);
                        const float a1 =
                            swiglu_bf16(acc[t][u][i0 + 1], acc[t + kG][u][i0 + 1], w_in, g.clamp, g.clamp_limit);
                        p[h] = uint32_t(f32_to_bf16_rne(a0)) | (uint32_t(f32_to_bf16_rne(a1)) << 16);
                    }
                    const int col = colw + q * 8 + fk * 4;
                    *reinterpret_cast<i32x2*>(out + int64_t(row) * g.I + col) = i32x2{int(p[0]), int(p[1])};
                }
            }
        }
    } else {
        const int hw = tile * kTM + wm * kTW;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int f = g.sorted_ids[blk * kBM + (2 * u + wn) * 32 + fr];
            if (f >= R) continue;
            const float tw = gemm2_row_weight(g, f);
            float* yrow = g.y + int64_t(f) * g.H;
#pragma unroll
            for (int t = 0; t < kTA; ++t)
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

template <int GEMM>
__global__ __launch_bounds__(kThreads, 1) void gemm_large_kernel(GemmArgs g, int ntiles) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];
    __shared__ int s_valid;

    int blk, tile;
    // block-major: the 12-24 column tiles of one block share its token rows in
    // L2, and the blocks of one expert (adjacent) run together and share the
    // weight tiles (measured: L2 hit rate 17% -> 42% on the prefill layer)
    if (!map_active_tile<true>(g, ntiles, blk, tile)) return;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    // An expert's last block with at most kXR real rows (row kXR is padding)
    // rides along with the expert's previous block: that workgroup multiplies
    // its rows as token rows 256..319 of the same weight tiles, so the expert's
    // weights stream once for both (each output keeps its K order: results are
    // the same bits).
    const int R = g.T * g.topk;
    const int active = __builtin_amdgcn_readfirstlane(g.ntpp[0]) / kBM;
    auto short_tail = [&](int b) { return g.sorted_ids[b * kBM + kXR] >= R; };
    if (blk > 0 && g.expert_ids[blk - 1] == e && short_tail(blk)) return;
    const bool ext = blk + 1 < active && g.expert_ids[blk + 1] == e && short_tail(blk + 1);

    // rows of the token tile that hold real slots (a prefix: padding sits at the end)
    if (threadIdx.x < 64) {
        int n = 0;
#pragma unroll
        for (int q = 0; q < kBR / 64; ++q)
            if (q < kBM / 64 || ext) n += __popcll(__ballot(g.sorted_ids[blk * kBM + q * 64 + threadIdx.x] < R));
        if (threadIdx.x == 0) s_valid = n;
    }
    __syncthreads();
    // live 32-token sub-tiles of this wave: u = wn, wn + 2, ... below the count
    const int live = (s_valid + 31) >> 5;
    const int wn = (threadIdx.x >> 6) / kWM;
    const int nu = (live - wn + 1) >> 1;
    if (ext) {   // 257..320 rows: 4 or 5 sub-tiles per wave
        if (nu >= 5) run_tile<GEMM, 5, false, true>(g, lds, blk, tile, e, s_valid);
        else run_tile<GEMM, 4, false, true>(g, lds, blk, tile, e, s_valid);
        return;
    }
    if constexpr (GEMM == 2) {
        // GEMM2 reads the intermediate's padding rows from memory: a block with
        // a whole token load step of padding (at most 6 live sub-tiles, 0..3
        // per wave) skips them (the down GEMM of 16-64 rows per expert 5-14 %
        // faster); a fuller block has 3 or 4 per wave.  GEMM1's padding rows
        // all read token 0, which stays in L2: it gained nothing there.
        if (s_valid <= kBM - kLoadRows) {
            switch (nu) {
                case 0: run_tile<GEMM, 0, true, false>(g, lds, blk, tile, e, s_valid); break;
                case 1: run_tile<GEMM, 1, true, false>(g, lds, blk, tile, e, s_valid); break;
                case 2: run_tile<GEMM, 2, true, false>(g, lds, blk, tile, e, s_valid); break;
                default: run_tile<GEMM, 3, true, false>(g, lds, blk, tile, e, s_valid); break;
            }
        } else if (nu >= 4) {
            run_tile<GEMM, 4, false, false>(g, lds, blk, tile, e, s_valid);
        } else {
            run_tile<GEMM, 3, false, false>(g, lds, blk, tile, e, s_valid);
        }
    } else {
        switch (nu) {
            case 0: run_tile<GEMM, 0, false, false>(g, lds, blk, tile, e, s_valid); break;
            case 1: run_tile<GEMM, 1, false, false>(g, lds, blk, tile, e, s_valid); break;
            case 2: run_tile<GEMM, 2, false, false>(g, lds, blk, tile, e, s_valid); break;
            case 3: run_tile<GEMM, 3, false, false>(g, lds, blk, tile, e, s_valid); break;
            default: run_tile<GEMM, 4, false, false>(g, lds, blk, tile, e, s_valid); break;
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
