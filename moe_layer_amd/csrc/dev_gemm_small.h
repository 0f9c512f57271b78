// Weight-streaming grouped GEMMs for few rows per expert (decode).
//
// The transposed ("swap-AB", P1 section "Swap-AB") orientation on CDNA4: the
// expert's weight rows fill the MFMA M side and the block's tokens the N side,
// so a block of 16..64 routed rows still runs full 16x16 MFMA tiles and every
// weight byte is read from HBM once per block.  Weights are used once, so they
// go straight from HBM to VGPRs (no LDS), two register stages deep; the token
// operand is small and stays in L2.
//
//   GEMM1 (a4+a5): h = W13[e] . x_t for the block's rows; epilogue pairs gate
//                  row i with up row I+i in the same lane and register, applies
//                  a = bf16(bf16(silu(bf16 g)) * bf16 u) (P2 section 1.2) and,
//                  for fp8, the per-row 128-group pow2 scale + e4m3 codes
//                  (group amax exchanged through LDS); the intermediate stays in
//                  expert-sorted order (P2 section 1.1, sorted-A).
//   GEMM2 (a6):    y = tw * (W2[e] . a), router weight applied in fp32 after the
//                  GEMM (P2 section 1.1); rows scattered to y[f] by flat slot.
//   Variants (P2 section 1.1 names both): with the router weight on the input
//   the GEMM1 epilogue scales h by it and GEMM2 applies none; a SwiGLU clamp
//   limit clamps the rounded gate/up pair (swiglu_bf16 in common.h).
//
// MFMA operand layouts (v_mfma_f32_16x16x32_bf16, v_mfma_f32_16x16x128_f8f6f4,
// checked on gfx950): lane l holds row (l % 16) of A and column (l % 16) of B
// at K offset (l / 16) * 8 elements (bf16) or (l / 16) * 32 (fp8); the 16x16
// result gives lane l the column (l % 16), rows 4 * (l / 16) + 0..3.
// fp8 GEMM1 multiplies on the bf16 matrix cores (operands dequantised in
// registers, exactly; see compute_stage), fp8 GEMM2 on the fp8 ones.
//
// Device code only (shared by the standalone kernels in gemm_small.hip and the
// single-launch decode layer in fused.hip): the kernel bodies are the tile
// functions gemm1_small_tile / gemm2_small_tile, run by one workgroup of NW
// waves for one (expert block, column tile).
#pragma once

#include "common.h"

namespace moe {
namespace small_gemm {   // the two GEMM families' helpers share names

namespace {

template <bool FP8>
struct Op {
    static constexpr int kStepK = FP8 ? 128 : 32;       // K per MFMA
    static constexpr int kParts = FP8 ? 2 : 1;          // 16-byte loads per operand per step
    static constexpr int kStepBytes = FP8 ? 128 : 64;   // bytes of one row per step
    static constexpr int kLaneOff = FP8 ? 32 : 16;      // byte offset of lane group l/16
    static constexpr int kElem = FP8 ? 1 : 2;
};

__device__ __forceinline__ i32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const i32x4*>(p); }

// A read-only load through the scalar data cache: p must be uniform over the
// wave (built from kernel arguments, block and wave indices), so the value
// lands in a scalar register and costs no vector memory instruction.
__device__ __forceinline__ float ld_uniform(const float* p) {
    return *(const __attribute__((address_space(4))) float*)p;
}

// fp8 activation group scales are staged per workgroup in LDS, kTabSteps
// K-blocks at a time: one vector load per (token, group) per workgroup
// instead of one per (token, group) per wave.  Row stride padded by one word
// so the 16 rows of a tile read distinct banks.
constexpr int kTabSteps = 64;
constexpr int kTabStride = kTabSteps + 1;

template <bool FP8>
__device__ __forceinline__ f32x4 mfma(const i32x4 (&a)[2], const i32x4 (&b)[2], f32x4 c) {
    if constexpr (FP8) {
        i32x8 av = {a[0][0], a[0][1], a[0][2], a[0][3], a[1][0], a[1][1], a[1][2], a[1][3]};
        i32x8 bv = {b[0][0], b[0][1], b[0][2], b[0][3], b[1][0], b[1][1], b[1][2], b[1][3]};
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                       __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
    }
}

// One pipeline stage: U K-steps of operands for MT weight tiles and NT token
// tiles (plus, for fp8, the per-step scales).
template <bool FP8, int MT, int NT, int U>
struct Stage {
    i32x4 a[U][MT][2];
    i32x4 b[U][NT][2];
    float sa[U][MT];   // weight block scale of each A tile (fp8)
    float sb[U][NT];   // activation group scale of each lane's token (fp8)
};

template <bool FP8, int MT, int NT, int U>
__device__ __forceinline__ void load_stage(Stage<FP8, MT, NT, U>& st, const uint8_t* const (&ap)[MT],
                                           const uint8_t* const (&bp)[NT],
                                           const float* const (&asp)[MT],
                                           const float* const (&bsp)[NT], int step0, int rot = 0, int nst = 0) {
    using O = Op<FP8>;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int sidx = step0 + u + rot;   // the walk's step step0 + u is K step (step0 + u + rot) mod nst
        if (sidx >= nst && rot) sidx -= nst;
        const int64_t off = int64_t(sidx) * O::kStepBytes;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int p = 0; p < O::kParts; ++p) st.a[u][m][p] = ld16(ap[m] + off + 16 * p);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int p = 0; p < O::kParts; ++p) st.b[u][n][p] = ld16(bp[n] + off + 16 * p);
        if constexpr (FP8) {
#pragma unroll
            for (int m = 0; m < MT; ++m) st.sa[u][m] = ld_uniform(asp[m] + sidx);   // weight block
#pragma unroll
            for (int n = 0; n < NT; ++n) st.sb[u][n] = bsp[n][sidx];                // LDS table
        }
    }
}

// One stage.  fp8: each 128-wide K block's partial product is scaled by
// (weight block scale) * (activation group scale).  kExact (fp8 GEMM1): the
// partial product comes from bf16 MFMAs on dequantised operands instead of one
// fp8 MFMA: the lane's 32 bytes (K 32*(l/16) .. +31) become four 8-element
// bf16 operands, the token's power-of-two group scale folded into its
// operand exactly, and four 16x16x32 bf16 MFMAs sum the block.  The fp8
// matrix-core dot product is not fp32-accurate on gfx950 (products below
// about 2^-14 of the largest in each group of eight are truncated, measured)
// while the bf16 one is, and GEMM1's results feed rounding decisions (the
// bf16 gate/up values, the intermediate's e4m3 codes).
template <bool FP8, bool kExact, int MT, int NT, int U>
__device__ __forceinline__ void compute_stage(const Stage<FP8, MT, NT, U>& st, f32x4 (&acc)[MT][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (FP8 && kExact) {
            f32x4 p[MT][NT];
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NT; ++n) p[m][n] = f32x4{0, 0, 0, 0};
            // per 8-element chunk q: convert the smaller operand set once,
            // stream the other (fewer live registers)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                auto cvt_a = [&](int m) {
                    return e4m3x8_to_bf16(st.a[u][m][q / 2][2 * (q % 2)], st.a[u][m][q / 2][2 * (q % 2) + 1], 1.0f);
                };
                auto cvt_b = [&](int n) {
                    return e4m3x8_to_bf16(st.b[u][n][q / 2][2 * (q % 2)], st.b[u][n][q / 2][2 * (q % 2) + 1],
                                          st.sb[u][n]);
                };
                if constexpr (NT <= MT) {
                    bf16x8 bv[NT];
#pragma unroll
                    for (int n = 0; n < NT; ++n) bv[n] = cvt_b(n);
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const bf16x8 av = cvt_a(m);
#pragma unroll
                        for (int n = 0; n < NT; ++n)
                            p[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[n], p[m][n], 0, 0, 0);
                    }
                } else {
                    bf16x8 av[MT];
#pragma unroll
                    for (int m = 0; m < MT; ++m) av[m] = cvt_a(m);
#pragma unroll
                    for (int n = 0; n < NT; ++n) {
                        const bf16x8 bv = cvt_b(n);
#pragma unroll
                        for (int m = 0; m < MT; ++m)
                            p[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv, p[m][n], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NT; ++n)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[m][n][j] = __builtin_fmaf(p[m][n][j], st.sa[u][m], acc[m][n][j]);
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NT; ++n) {
                    if constexpr (FP8) {
                        const f32x4 p = mfma<FP8>(st.a[u][m], st.b[u][n], f32x4{0, 0, 0, 0});
                        const float c = __fmul_rn(st.sa[u][m], st.sb[u][n]);
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[m][n][j] = __builtin_fmaf(p[j], c, acc[m][n][j]);
                    } else {
                        acc[m][n] = mfma<FP8>(st.a[u][m], st.b[u][n], acc[m][n]);
                    }
                }
        }
    }
}

// K loop over nsteps MFMA steps (nsteps % U == 0): load the next stage, then
// compute the current one.  The loads sit under a branch, so the compiler
// waits for all of them before each compute: one stage is in flight per wave,
// and HBM latency is hidden by many waves per CU (the tiles are sized for
// occupancy).  Deeper software pipelines (3-4 stages with scheduling
// barriers) cost occupancy and measured slower on every decode shape.
template <bool FP8, bool kExact, int MT, int NT, int U>
__device__ __forceinline__ void mainloop(const uint8_t* const (&ap)[MT], const uint8_t* const (&bp)[NT],
                                         const float* const (&asp)[MT], const float* const (&bsp)[NT],
                                         int nsteps, f32x4 (&acc)[MT][NT], int rot = 0) {
    Stage<FP8, MT, NT, U> s0, s1;
    load_stage<FP8, MT, NT, U>(s0, ap, bp, asp, bsp, 0, rot, nsteps);
    for (int k = 0; k < nsteps; k += 2 * U) {
        const bool has1 = k + U < nsteps;
        if (has1) load_stage<FP8, MT, NT, U>(s1, ap, bp, asp, bsp, k + U, rot, nsteps);
        compute_stage<FP8, kExact, MT, NT, U>(s0, acc);
        if (k + 2 * U < nsteps) load_stage<FP8, MT, NT, U>(s0, ap, bp, asp, bsp, k + 2 * U, rot, nsteps);
        if (has1) compute_stage<FP8, kExact, MT, NT, U>(s1, acc);
    }
}

// fp8 K loop: per chunk of kTabSteps K-blocks, stage the BM rows' activation
// scales (row_scale(r) points at row r's first group) in LDS, then run the
// mainloop over the chunk.  Every thread of the workgroup takes part.
template <bool kExact, int MT, int NT, int BM, int NTHREADS, typename RowScale>
__device__ __forceinline__ void mainloop_fp8(const uint8_t* const (&ap)[MT], const uint8_t* const (&bp)[NT],
                                             const float* const (&asp)[MT], RowScale row_scale, int nsteps,
                                             float* tab, f32x4 (&acc)[MT][NT], int rot = 0) {
    using O = Op<true>;
    if (nsteps > kTabSteps) rot = 0;   // the rotated walk stays inside one table chunk
    const int lr = threadIdx.x & 15;
    for (int c0 = 0; c0 < nsteps; c0 += kTabSteps) {
        const int cs = min(kTabSteps, nsteps - c0);
        __syncthreads();   // the previous chunk's table reads are done
        for (int i = threadIdx.x; i < BM * cs; i += NTHREADS) {
            const int r = i / cs, k = i - r * cs;
            tab[r * kTabStride + k] = row_scale(r)[c0 + k];
        }
        __syncthreads();
        const uint8_t* apc[MT];
        const float* aspc[MT];
        const uint8_t* bpc[NT];
        const float* bspc[NT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            apc[m] = ap[m] + int64_t(c0) * O::kStepBytes;
            aspc[m] = asp[m] + c0;
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            bpc[n] = bp[n] + int64_t(c0) * O::kStepBytes;
            bspc[n] = tab + (n * 16 + lr) * kTabStride;
        }
        mainloop<true, kExact, MT, NT, 1>(apc, bpc, aspc, bspc, cs, acc, rot);
    }
}

// ----------------------------------------------------------------------------
// GEMM1 + SiLU-mul (+ fp8 requant)
//   WT gate tiles and WT up tiles (16 rows each) per wave; NW waves per block
//   cover NW*WT*16 intermediate columns; BM = 16*NT tokens.
// ----------------------------------------------------------------------------
// kRot (fp8 only): walk K from k_rotation's start; the caller picks the
// instance from GemmArgs::krot, so the unrotated one keeps its plain loop.
template <bool FP8, int NT, int WT, int NW, int U, bool kRot = false>
__device__ __forceinline__ void gemm1_small_tile(const GemmArgs& g, int blk, int tile) {
    using O = Op<FP8>;
    constexpr int MT = 2 * WT;
    constexpr int BM = 16 * NT;
    constexpr int COLS = NW * WT * 16;   // intermediate columns per workgroup
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lk = lane >> 4;
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int i0 = tile * COLS + wv * WT * 16;   // first gate column of this wave

    const uint8_t* w13 = static_cast<const uint8_t*>(g.w13);
    const uint8_t* xs = FP8 ? g.xq : reinterpret_cast<const uint8_t*>(g.x);
    const uint8_t* ap[MT];
    const float* asp[MT];
    const uint8_t* bp[NT];
    const float* bsp[NT];
    const int kb_count = H / kGroup;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = (m < WT ? i0 + m * 16 : I + i0 + (m - WT) * 16);
        ap[m] = w13 + (int64_t(e) * 2 * I + row + lr) * H * O::kElem + lk * O::kLaneOff;
        asp[m] = FP8 ? static_cast<const float*>(g.w13_scale) + (int64_t(e) * (2 * I / kGroup) + row / kGroup) * kb_count
                     : nullptr;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int f = g.sorted_ids[blk * BM + n * 16 + lr];
        const int tok = f < R ? f / g.topk : 0;   // padding rows read token 0, never stored as real rows
        bp[n] = xs + int64_t(tok) * H * O::kElem + lk * O::kLaneOff;
        bsp[n] = nullptr;
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    if constexpr (FP8) {
        __shared__ float tab[BM * kTabStride];
        const int32_t* rows = g.sorted_ids + blk * BM;
        auto row_scale = [&](int r) {
            const int f = rows[r];
            return g.xs + int64_t(f < R ? f / g.topk : 0) * kb_count;
        };
        const int nst = H / O::kStepK;
        mainloop_fp8<true, MT, NT, BM, NW * 64>(ap, bp, asp, row_scale, nst, tab, acc,
                                                kRot ? k_rotation(g, e, tile, nst) : 0);
    } else {
        mainloop<FP8, false, MT, NT, U>(ap, bp, asp, bsp, H / O::kStepK, acc);
    }

    // epilogue: a = silu(g) * u with the bf16 rounding points
    float a[WT][NT][4];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const float w_in = gemm1_row_weight(g, g.sorted_ids[blk * BM + n * 16 + lr]);
#pragma unroll
        for (int m = 0; m < WT; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a[m][n][j] = swiglu_bf16(acc[m][n][j], acc[WT + m][n][j], w_in, g.clamp, g.clamp_limit);
    }

    if constexpr (!FP8) {
        uint16_t* out = static_cast<uint16_t*>(g.inter);
#pragma unroll
        for (int m = 0; m < WT; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) {
                const int row = blk * BM + n * 16 + lr;
                const int col = i0 + m * 16 + 4 * lk;
                const uint32_t lo = f32_to_bf16_rne(a[m][n][0]) | (uint32_t(f32_to_bf16_rne(a[m][n][1])) << 16);
                const uint32_t hi = f32_to_bf16_rne(a[m][n][2]) | (uint32_t(f32_to_bf16_rne(a[m][n][3])) << 16);
                *reinterpret_cast<i32x2*>(out + int64_t(row) * I + col) = i32x2{int(lo), int(hi)};
            }
    } else {
        // per token, amax over the workgroup's 128 columns (one group)
        static_assert(COLS == kGroup, "fp8 GEMM1 tile must span one 128-column group");
        __shared__ float part[NW][BM];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float m_ = 0.0f;
#pragma unroll
            for (int m = 0; m < WT; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) m_ = fmaxf(m_, __builtin_fabsf(a[m][n][j]));
            m_ = fmaxf(m_, __shfl_xor(m_, 16));
            m_ = fmaxf(m_, __shfl_xor(m_, 32));
            if (lk == 0) part[wv][n * 16 + lr] = m_;
        }
        __syncthreads();
        uint8_t* out = static_cast<uint8_t*>(g.inter);
        const int ngroups = I / kGroup;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            float amax = 0.0f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) amax = fmaxf(amax, part[w2][n * 16 + lr]);
            const float s = fp8_group_scale(amax);
            const float inv_s = __fdiv_rn(1.0f, s);
            const int row = blk * BM + n * 16 + lr;
#pragma unroll
            for (int m = 0; m < WT; ++m) {
                uint32_t packed = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) packed |= fp8_quant(a[m][n][j], inv_s) << (8 * j);
                const int col = i0 + m * 16 + 4 * lk;
                *reinterpret_cast<uint32_t*>(out + int64_t(row) * I + col) = packed;
            }
            if (wv == 0 && lk == 0) g.inter_scale[int64_t(row) * ngroups + tile] = s;
        }
    }
}

// ----------------------------------------------------------------------------
// GEMM2: y[f] = tw[f] * (W2[e] . a_row), WT tiles of 16 output columns per wave
// ----------------------------------------------------------------------------
template <bool FP8, int NT, int WT, int NW, int U>
__device__ __forceinline__ void gemm2_small_tile(const GemmArgs& g, int blk, int tile) {
    using O = Op<FP8>;
    constexpr int MT = WT;
    constexpr int BM = 16 * NT;
    constexpr int COLS = NW * WT * 16;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lk = lane >> 4;
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int h0 = tile * COLS + wv * WT * 16;
    const int kb_count = I / kGroup;

    const uint8_t* w2 = static_cast<const uint8_t*>(g.w2);
    const uint8_t* inter = static_cast<const uint8_t*>(g.inter);
    const uint8_t* ap[MT];
    const float* asp[MT];
    const uint8_t* bp[NT];
    const float* bsp[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = h0 + m * 16;
        ap[m] = w2 + (int64_t(e) * H + row + lr) * I * O::kElem + lk * O::kLaneOff;
        asp[m] = FP8 ? static_cast<const float*>(g.w2_scale) + (int64_t(e) * (H / kGroup) + row / kGroup) * kb_count
                     : nullptr;
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int row = blk * BM + n * 16 + lr;
        bp[n] = inter + int64_t(row) * I * O::kElem + lk * O::kLaneOff;
        bsp[n] = nullptr;
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    if constexpr (FP8) {
        __shared__ float tab[BM * kTabStride];
        const float* scales = g.inter_scale + int64_t(blk) * BM * kb_count;
        auto row_scale = [&](int r) { return scales + int64_t(r) * kb_count; };
        mainloop_fp8<false, MT, NT, BM, NW * 64>(ap, bp, asp, row_scale, I / O::kStepK, tab, acc);
    } else {
        mainloop<FP8, false, MT, NT, U>(ap, bp, asp, bsp, I / O::kStepK, acc);
    }

#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int f = g.sorted_ids[blk * BM + n * 16 + lr];
        if (f >= R) continue;
        const float tw = gemm2_row_weight(g, f);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const int col = h0 + m * 16 + 4 * lk;
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = __fmul_rn(acc[m][n][j], tw);
            store_y4<FP8>(g.y, int64_t(f) * H + col, v);
        }
    }
}

// GEMM2 over NTILE adjacent column tiles of one block in one workgroup.  With
// a short K (fp8 layer: I = 256, 2 K-steps) a one-tile workgroup spends much
// of its life on its prologue (token-scale table, first loads) and epilogue
// (y stores) with no weight bytes in flight.  Here the fp8 token-scale table
// is staged once and the register stages (U K-steps each) of all NTILE tiles
// form one pipeline: the next tile's loads are in flight while the current
// one is finished and stored.  Per tile the arithmetic is gemm2_small_tile's
// (same order), so the results are bitwise those of the one-tile form.  fp8
// needs I / 128 <= kTabSteps (one table for all of K).
template <bool FP8, int NT, int WT, int NW, int U, int NTILE>
__device__ __forceinline__ void gemm2_tiles(const GemmArgs& g, int blk, int tile0) {
    using O = Op<FP8>;
    constexpr int MT = WT;
    constexpr int BM = 16 * NT;
    constexpr int COLS = NW * WT * 16;
    static_assert(!FP8 || U == 1, "fp8: one K-step per stage");
    static_assert(!FP8 || COLS % kGroup == 0, "a column tile spans whole weight-scale blocks");
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lk = lane >> 4;
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int h0 = tile0 * COLS + wv * WT * 16;   // first output row of this wave, first tile
    const int kb_count = I / kGroup;
    const int ns = I / (O::kStepK * U);            // register stages per tile

    const uint8_t* w2 = static_cast<const uint8_t*>(g.w2);
    const uint8_t* inter = static_cast<const uint8_t*>(g.inter);
    const uint8_t* ap[MT];
    const float* asp[MT];
    const uint8_t* bp[NT];
    const float* bsp[NT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int row = h0 + m * 16;
        ap[m] = w2 + (int64_t(e) * H + row + lr) * I * O::kElem + lk * O::kLaneOff;
        asp[m] = FP8 ? static_cast<const float*>(g.w2_scale) + (int64_t(e) * (H / kGroup) + row / kGroup) * kb_count
                     : nullptr;
    }

    // fp8: the block's token-scale table, all of K at once (the barrier first:
    // a workgroup that ran an item before must have finished reading it)
    __shared__ float tab[FP8 ? BM * kTabStride : 1];
    if constexpr (FP8) {
        __syncthreads();
        const float* scales = g.inter_scale + int64_t(blk) * BM * kb_count;
        for (int i = threadIdx.x; i < BM * ns; i += NW * 64) {
            const int r = i / ns, k = i - r * ns;
            tab[r * kTabStride + k] = scales[int64_t(r) * kb_count + k];
        }
    }
    int f[NT];
    float tw[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int row = blk * BM + n * 16 + lr;
        bp[n] = inter + int64_t(row) * I * O::kElem + lk * O::kLaneOff;
        bsp[n] = FP8 ? tab + (n * 16 + lr) * kTabStride : nullptr;
        f[n] = g.sorted_ids[row];
        tw[n] = f[n] < R ? gemm2_row_weight(g, f[n]) : 0.0f;
    }
    if constexpr (FP8) __syncthreads();

    // virtual stage v = tile t * ns + k
    const int64_t tile_bytes = int64_t(COLS) * I * O::kElem;   // weight bytes between tiles
    const int tile_scales = (COLS / kGroup) * kb_count;          // fp8 weight-scale words between tiles
    auto load = [&](Stage<FP8, MT, NT, U>& st, int v) {
        const int t = v / ns, k = (v - t * ns) * U;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t off = int64_t(k + u) * O::kStepBytes;
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int p = 0; p < O::kParts; ++p) st.a[u][m][p] = ld16(ap[m] + t * tile_bytes + off + 16 * p);
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
                for (int p = 0; p < O::kParts; ++p) st.b[u][n][p] = ld16(bp[n] + off + 16 * p);
            if constexpr (FP8) {
#pragma unroll
                for (int m = 0; m < MT; ++m) st.sa[u][m] = ld_uniform(asp[m] + t * tile_scales + k + u);
#pragma unroll
                for (int n = 0; n < NT; ++n) st.sb[u][n] = bsp[n][k + u];
            }
        }
    };
    f32x4 acc[MT][NT];
    auto clear = [&]() {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    };
    // after stage v: a finished tile is scaled by the router weight and stored
    auto finish = [&](int v) {
        if ((v + 1) % ns != 0) return;
        const int hc = h0 + (v / ns) * COLS;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            if (f[n] >= R) continue;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                f32x4 o;
#pragma unroll
                for (int j = 0; j < 4; ++j) o[j] = __fmul_rn(acc[m][n][j], tw[n]);
                store_y4<FP8>(g.y, int64_t(f[n]) * H + hc + m * 16 + 4 * lk, o);
            }
        }
        clear();
    };

    clear();
    const int V = NTILE * ns;
    Stage<FP8, MT, NT, U> s0, s1;
    load(s0, 0);
    for (int v = 0; v < V; v += 2) {
        const bool has1 = v + 1 < V;
        if (has1) load(s1, v + 1);
        compute_stage<FP8, false, MT, NT, U>(s0, acc);
        finish(v);
        if (v + 2 < V) load(s0, v + 2);
        if (has1) {
            compute_stage<FP8, false, MT, NT, U>(s1, acc);
            finish(v + 1);
        }
    }
}

}  // namespace

}  // namespace small_gemm
}  // namespace moe
