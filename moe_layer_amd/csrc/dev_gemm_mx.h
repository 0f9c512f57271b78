// MXFP8 grouped GEMMs for few rows per expert (the weight-streaming path).
//
// MXFP8 (P3, quantisation section of "Hosting Qwen on Blackwell": the MXFP8
// scheme, weights converted statically) gives every 32 consecutive K elements
// of a row one E8M0 scale, a bare power of two.  That is the operand format of
// CDNA4's scaled matrix-core instruction.  In v_mfma_scale_f32_16x16x128_f8f6f4
// (layout measured on gfx950) lane l holds 32 e4m3 elements of row (l % 16):
// K [16g, 16g + 16) in its first 16 bytes and K [64 + 16g, 64 + 16g + 16) in
// its last 16, g = l / 16; and lane l passes, as its scale operand, the E8M0
// byte of K block g = [32g, 32g + 32) of row (l % 16).  So each K step of 128
// is one instruction that applies both operands' block scales and accumulates
// into the fp32 accumulator: no per-block rescaling on the vector ALUs.
// GEMM2 runs on it.  GEMM1, whose results feed rounding decisions, runs on
// the bf16 matrix cores instead: each lane dequantises its own MX block to
// bf16 (exact for power-of-two scales), because the fp8 instruction's dot
// product is not fp32-accurate (mx_compute).
//
// Orientation, tiles and epilogues follow the block-fp8 kernels: weights on
// the MFMA M side (swap-AB, P1 section "Swap-AB"), the block's tokens on N,
// gate/up pairs in the same lane; GEMM1's epilogue applies the SiLU-mul
// rounding points (P2 section 1.2) and re-quantises the intermediate per row
// and 32-column group (E8M0 scale + e4m3 codes, group amax exchanged through
// LDS); GEMM2's multiplies by the router weight in fp32 and writes y by flat
// slot.  The layer variants (router weight on the input, SwiGLU clamp) act in
// the epilogues as in the block-fp8 kernels.
//
// Device code only (shared by the standalone kernels in gemm_mx.hip and the
// single-launch decode layer in fused.hip): the kernel bodies are the tile
// functions gemm1_mx_tile / gemm2_mx_tile.
#pragma once

#include "common.h"

namespace moe {
namespace mx_gemm {   // the two GEMM families' helpers share names

namespace {

constexpr int kStepK = 128;                 // K per MFMA step (4 MX blocks)
constexpr int kMxBlock = 32;
constexpr int kTabSteps = 64;               // activation-scale table chunk, in K steps
constexpr int kTabStride = 4 * kTabSteps + 4;   // bytes per table row (padded by a word)

__device__ __forceinline__ i32x4 ld16(const uint8_t* p) { return *reinterpret_cast<const i32x4*>(p); }

// The lane's operand bytes of one K step.  Scaled fp8 MFMA layout (kExact =
// false): p points at K offset 16 * (l / 16), the second 16 bytes sit 64
// further.  bf16 MFMA layout (kExact = true): p points at K offset
// 32 * (l / 16), 32 contiguous bytes = the lane's MX block.
template <bool kExact>
__device__ __forceinline__ i32x8 ld32(const uint8_t* p) {
    const i32x4 lo = ld16(p), hi = ld16(p + (kExact ? 16 : 64));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int MT, int NT, int U>
struct MxStage {
    i32x8 a[U][MT];       // the lane's 32 e4m3 elements of its weight row (see ld32)
    i32x8 b[U][NT];       // ... of its token row
    uint32_t sa[U][MT];   // E8M0 byte of the lane's weight row and K block
    uint32_t sb[U][NT];   // E8M0 byte of the lane's token row and K block
};

// Operand addressing: a wave-uniform base per weight tile (scalar registers)
// plus one 32-bit lane offset shared by all weight tiles, so the loads take
// the scalar-base + vector-offset form and few vector registers hold
// addresses.  Tokens: one uniform base plus a 32-bit offset per token tile.
// Weight scales are read per lane, one byte per tile and step (staging them
// in LDS as well measured no faster): in the row-major scale layout a wave's
// 64 bytes of a step lie on 16 rows (lane offset 16-row stride, step stride 4),
// in the packed layout of moe_pack_mx_scales they are contiguous in lane order
// (lane offset = lane, step stride 64; one coalesced load, MXFP8 GEMM1 200 ->
// 168 us on the MXFP8 layer).  The tokens' scales come from an LDS table the
// workgroup fills per chunk of kTabSteps steps.
template <int MT, int NT>
struct MxAddr {
    const uint8_t* a[MT];    // weight tile bases (uniform)
    const uint8_t* as[MT];   // weight-scale tile bases (uniform)
    uint32_t aoff;           // lane offset into a weight tile, step 0
    uint32_t asoff;          // lane offset into a weight-scale tile, step 0
    uint32_t asstep;         // its advance per K step (4 row-major, 64 packed)
    const uint8_t* b;        // token operand base (uniform)
    uint32_t boff[NT];       // lane offset of each token tile, step 0
    const uint8_t* bs[NT];   // the lane's byte in the LDS token-scale table, step 0
};

// Weight-scale lane offset and step stride for lane (lr, lk) = (row in the
// 16-row tile, 32-element K block of the step); kb = scale bytes per row.
template <int MT, int NT>
__device__ __forceinline__ void set_scale_lane(MxAddr<MT, NT>& ad, const GemmArgs& g, int lr, int lk, int kb) {
    ad.asoff = g.mx_packed ? uint32_t(lr + 16 * lk) : uint32_t(lr * kb + lk);
    ad.asstep = g.mx_packed ? 64u : 4u;
}

template <bool kExact, int MT, int NT, int U>
__device__ __forceinline__ void mx_load(MxStage<MT, NT, U>& st, const MxAddr<MT, NT>& ad, int step0, int rot = 0,
                                        int nst = 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int sidx = step0 + u + rot;   // the walk's step step0 + u is K step (step0 + u + rot) mod nst (k_rotation)
        if (sidx >= nst && rot) sidx -= nst;
        const uint32_t off = uint32_t(sidx) * kStepK;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            st.a[u][m] = ld32<kExact>(ad.a[m] + (ad.aoff + off));
            st.sa[u][m] = ad.as[m][ad.asoff + ad.asstep * uint32_t(sidx)];
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            st.b[u][n] = ld32<kExact>(ad.b + (ad.boff[n] + off));
            st.sb[u][n] = ad.bs[n][4 * sidx];
        }
    }
}

// One K step.  kExact = false: one scaled fp8 MFMA per tile pair.  kExact =
// true: each lane dequantises its two MX blocks to bf16 (code * 2^(scale -
// 127), exact) and four bf16 MFMAs accumulate the 128 products: the fp8
// matrix-core dot product is not fp32-accurate on gfx950 (products smaller
// than about 2^-14 of the largest in each group of eight are truncated,
// measured), while the bf16 one is.  GEMM1 takes the exact form: its results
// feed rounding decisions (the bf16 gate/up values and the intermediate's
// e4m3 codes).
template <bool kExact, int MT, int NT, int U>
__device__ __forceinline__ void mx_compute(const MxStage<MT, NT, U>& st, f32x4 (&acc)[MT][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (kExact) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bf16x8 bv[NT];
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    bv[n] = e4m3x8_to_bf16(st.b[u][n][2 * q], st.b[u][n][2 * q + 1], e8m0_to_f32(st.sb[u][n]));
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const bf16x8 av =
                        e4m3x8_to_bf16(st.a[u][m][2 * q], st.a[u][m][2 * q + 1], e8m0_to_f32(st.sa[u][m]));
#pragma unroll
                    for (int n = 0; n < NT; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[n], acc[m][n], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < MT; ++m)
#pragma unroll
                for (int n = 0; n < NT; ++n)
                    acc[m][n] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        st.a[u][m], st.b[u][n], acc[m][n], 0, 0, 0, int(st.sa[u][m]), 0, int(st.sb[u][n]));
        }
    }
}

// K loop over nsteps steps, two register stages (the block-fp8 kernels' loop).
template <bool kExact, int MT, int NT, int U>
__device__ __forceinline__ void mx_mainloop(const MxAddr<MT, NT>& ad, int nsteps, f32x4 (&acc)[MT][NT], int rot = 0) {
    MxStage<MT, NT, U> s0, s1;
    mx_load<kExact, MT, NT, U>(s0, ad, 0, rot, nsteps);
    for (int k = 0; k < nsteps; k += 2 * U) {
        const bool has1 = k + U < nsteps;
        if (has1) mx_load<kExact, MT, NT, U>(s1, ad, k + U, rot, nsteps);
        mx_compute<kExact, MT, NT, U>(s0, acc);
        if (k + 2 * U < nsteps) mx_load<kExact, MT, NT, U>(s0, ad, k + 2 * U, rot, nsteps);
        if (has1) mx_compute<kExact, MT, NT, U>(s1, acc);
    }
}

// Per chunk of kTabSteps K steps: stage the BM token rows' scale bytes
// (row_scale(r) points at row r's first byte) in LDS, then run the K loop.
template <bool kExact, int MT, int NT, int BM, int NTHREADS, typename RowScale>
__device__ __forceinline__ void mx_kloop(MxAddr<MT, NT> ad, RowScale row_scale, int nsteps, uint8_t* tab,
                                         f32x4 (&acc)[MT][NT], int rot = 0) {
    if (nsteps > kTabSteps) rot = 0;   // the rotated walk stays inside one table chunk
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15, lk = lane >> 4;
    const uint32_t aoff0 = ad.aoff, asoff0 = ad.asoff;
    uint32_t boff0[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        boff0[n] = ad.boff[n];
        ad.bs[n] = tab + (n * 16 + lr) * kTabStride + lk;
    }
    for (int c0 = 0; c0 < nsteps; c0 += kTabSteps) {
        const int cs = min(kTabSteps, nsteps - c0);
        __syncthreads();   // the previous chunk's table reads are done
        for (int i = threadIdx.x; i < BM * cs; i += NTHREADS) {   // one 4-byte word per (row, step)
            const int r = i / cs, k = i - r * cs;
            *reinterpret_cast<uint32_t*>(tab + r * kTabStride + 4 * k) =
                *reinterpret_cast<const uint32_t*>(row_scale(r) + 4 * (c0 + k));
        }
        __syncthreads();
        ad.aoff = aoff0 + uint32_t(c0) * kStepK;
        ad.asoff = asoff0 + ad.asstep * uint32_t(c0);
#pragma unroll
        for (int n = 0; n < NT; ++n) ad.boff[n] = boff0[n] + uint32_t(c0) * kStepK;
        mx_mainloop<kExact, MT, NT, 1>(ad, cs, acc, rot);
    }
}

// ----------------------------------------------------------------------------
// GEMM1 + SiLU-mul + MXFP8 re-quantisation of the intermediate
//   WT gate + WT up tiles (16 rows each) per wave, NW waves per workgroup
//   cover COLS = NW*WT*16 intermediate columns; BM = 16*NT tokens.
// ----------------------------------------------------------------------------
template <int NT, int WT, int NW>
__device__ __forceinline__ void gemm1_mx_tile(const GemmArgs& g, int blk, int tile) {
    constexpr int MT = 2 * WT;
    constexpr int BM = 16 * NT;
    constexpr int COLS = NW * WT * 16;
    static_assert(COLS % kMxBlock == 0, "a workgroup covers whole MX groups");
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lk = lane >> 4;
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int i0 = tile * COLS + wv * WT * 16;   // first gate column of this wave
    const int kbh = H / kMxBlock;                // scale bytes per row

    const uint8_t* w13 = static_cast<const uint8_t*>(g.w13);
    const uint8_t* w13s = static_cast<const uint8_t*>(g.w13_scale);
    MxAddr<MT, NT> ad;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t row0 = int64_t(e) * 2 * I + (m < WT ? i0 + m * 16 : I + i0 + (m - WT) * 16);
        ad.a[m] = w13 + row0 * H;
        ad.as[m] = w13s + row0 * kbh;
    }
    ad.aoff = uint32_t(lr * H + lk * 32);   // bf16 MFMA layout: the lane's MX block of the step
    set_scale_lane(ad, g, lr, lk, kbh);
    ad.b = g.xq;
    const int32_t* rows = g.sorted_ids + blk * BM;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        const int f = rows[n * 16 + lr];
        const int tok = f < R ? f / g.topk : 0;   // padding rows read token 0, never stored as real rows
        ad.boff[n] = uint32_t(tok) * uint32_t(H) + uint32_t(lk * 32);
    }

    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    __shared__ __attribute__((aligned(16))) uint8_t tab[BM * kTabStride];
    const uint8_t* xs = reinterpret_cast<const uint8_t*>(g.xs);
    auto row_scale = [&](int r) {
        const int f = rows[r];
        return xs + int64_t(f < R ? f / g.topk : 0) * kbh;
    };
    mx_kloop<true, MT, NT, BM, NW * 64>(ad, row_scale, H / kStepK, tab, acc, k_rotation_start(e, tile, H / kStepK));

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

    // per token, amax over each 32-column group: the wave's columns
    // i0 .. i0 + 16*WT - 1, lanes lk = 0..3 hold 4 columns each per tile
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
    constexpr int kWavesPerGroup = WT * 16 >= kMxBlock ? 1 : kMxBlock / (WT * 16);
    constexpr int kGroupsPerWave = WT * 16 >= kMxBlock ? WT * 16 / kMxBlock : 1;
    static_assert(kGroupsPerWave == 1, "one MX group per wave or a group over several waves");
    const int wg0 = (wv / kWavesPerGroup) * kWavesPerGroup;
    uint8_t* out = static_cast<uint8_t*>(g.inter);
    uint8_t* out_s = reinterpret_cast<uint8_t*>(g.inter_scale);
    const int ngroups = I / kMxBlock;
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        float amax = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < kWavesPerGroup; ++w2) amax = fmaxf(amax, part[wg0 + w2][n * 16 + lr]);
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
        if (wv == wg0 && lk == 0) out_s[int64_t(row) * ngroups + i0 / kMxBlock] = uint8_t(__float_as_uint(s) >> 23);
    }
}

// ----------------------------------------------------------------------------
// GEMM2: y[f] = tw[f] * (W2[e] . a_row), WT tiles of 16 output columns per wave
// ----------------------------------------------------------------------------
template <int NT, int WT, int NW>
__device__ __forceinline__ void gemm2_mx_tile(const GemmArgs& g, int blk, int tile) {
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
    const int kbi = I / kMxBlock;

    const uint8_t* w2 = static_cast<const uint8_t*>(g.w2);
    const uint8_t* w2s = static_cast<const uint8_t*>(g.w2_scale);
    MxAddr<MT, NT> ad;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t row0 = int64_t(e) * H + h0 + m * 16;
        ad.a[m] = w2 + row0 * I;
        ad.as[m] = w2s + row0 * kbi;
    }
    ad.aoff = uint32_t(lr * I + lk * 16);
    set_scale_lane(ad, g, lr, lk, kbi);
    ad.b = static_cast<const uint8_t*>(g.inter) + int64_t(blk) * BM * I;
#pragma unroll
    for (int n = 0; n < NT; ++n) ad.boff[n] = uint32_t((n * 16 + lr) * I + lk * 16);

    f32x4 acc[MT][NT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    __shared__ __attribute__((aligned(16))) uint8_t tab[BM * kTabStride];
    const uint8_t* scales = reinterpret_cast<const uint8_t*>(g.inter_scale) + int64_t(blk) * BM * kbi;
    auto row_scale = [&](int r) { return scales + int64_t(r) * kbi; };
    mx_kloop<false, MT, NT, BM, NW * 64>(ad, row_scale, I / kStepK, tab, acc);

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
            store_y4<true>(g.y, int64_t(f) * H + col, v);
        }
    }
}

// GEMM2 over NTILE adjacent column tiles of one block in one workgroup: the
// token-scale table staged once, the K-steps of all tiles one register
// pipeline (the next tile's loads in flight while the current one is stored).
// Per tile the arithmetic is gemm2_mx_tile's, so the results are bitwise the
// same.  Needs I / 128 <= kTabSteps.
template <int NT, int WT, int NW, int NTILE>
__device__ __forceinline__ void gemm2_mx_tiles(const GemmArgs& g, int blk, int tile0) {
    constexpr int MT = WT;
    constexpr int BM = 16 * NT;
    constexpr int COLS = NW * WT * 16;
    const int e = __builtin_amdgcn_readfirstlane(g.expert_ids[blk]);
    if (e < 0) return;

    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lk = lane >> 4;
    const int H = g.H, I = g.I, R = g.T * g.topk;
    const int h0 = tile0 * COLS + wv * WT * 16;
    const int kbi = I / kMxBlock;
    const int ns = I / kStepK;

    const uint8_t* w2 = static_cast<const uint8_t*>(g.w2);
    const uint8_t* w2s = static_cast<const uint8_t*>(g.w2_scale);
    MxAddr<MT, NT> ad;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t row0 = int64_t(e) * H + h0 + m * 16;
        ad.a[m] = w2 + row0 * I;
        ad.as[m] = w2s + row0 * kbi;
    }
    ad.aoff = uint32_t(lr * I + lk * 16);
    set_scale_lane(ad, g, lr, lk, kbi);
    ad.b = static_cast<const uint8_t*>(g.inter) + int64_t(blk) * BM * I;

    // the block's token-scale table, all of K at once (the barrier first: a
    // workgroup that ran an item before must have finished reading it)
    __shared__ __attribute__((aligned(16))) uint8_t tab[BM * kTabStride];
    {
        __syncthreads();
        const uint8_t* scales = reinterpret_cast<const uint8_t*>(g.inter_scale) + int64_t(blk) * BM * kbi;
        for (int i = threadIdx.x; i < BM * ns; i += NW * 64) {
            const int r = i / ns, k = i - r * ns;
            *reinterpret_cast<uint32_t*>(tab + r * kTabStride + 4 * k) =
                *reinterpret_cast<const uint32_t*>(scales + int64_t(r) * kbi + 4 * k);
        }
    }
    int f[NT];
    float tw[NT];
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        ad.boff[n] = uint32_t((n * 16 + lr) * I + lk * 16);
        ad.bs[n] = tab + (n * 16 + lr) * kTabStride + lk;
        f[n] = g.sorted_ids[blk * BM + n * 16 + lr];
        tw[n] = f[n] < R ? gemm2_row_weight(g, f[n]) : 0.0f;
    }
    __syncthreads();

    // virtual step v = tile t * ns + k
    const int64_t tile_bytes = int64_t(COLS) * I;        // weight bytes between tiles
    const int64_t tile_sbytes = int64_t(COLS) * kbi;     // weight-scale bytes between tiles
    auto load = [&](MxStage<MT, NT, 1>& st, int v) {
        const int t = v / ns, k = v - t * ns;
        const uint32_t off = uint32_t(k) * kStepK;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            st.a[0][m] = ld32<false>(ad.a[m] + t * tile_bytes + (ad.aoff + off));
            st.sa[0][m] = (ad.as[m] + t * tile_sbytes)[ad.asoff + ad.asstep * uint32_t(k)];
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
            st.b[0][n] = ld32<false>(ad.b + (ad.boff[n] + off));
            st.sb[0][n] = ad.bs[n][4 * k];
        }
    };
    f32x4 acc[MT][NT];
    auto clear = [&]() {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int n = 0; n < NT; ++n) acc[m][n] = f32x4{0, 0, 0, 0};
    };
    // after K-step v: a finished tile is scaled by the router weight and stored
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
                store_y4<true>(g.y, int64_t(f[n]) * H + hc + m * 16 + 4 * lk, o);
            }
        }
        clear();
    };

    clear();
    const int V = NTILE * ns;
    MxStage<MT, NT, 1> s0, s1;
    load(s0, 0);
    for (int v = 0; v < V; v += 2) {
        const bool has1 = v + 1 < V;
        if (has1) load(s1, v + 1);
        mx_compute<false, MT, NT, 1>(s0, acc);
        finish(v);
        if (v + 2 < V) load(s0, v + 2);
        if (has1) {
            mx_compute<false, MT, NT, 1>(s1, acc);
            finish(v + 1);
        }
    }
}

}  // namespace

}  // namespace mx_gemm
}  // namespace moe
