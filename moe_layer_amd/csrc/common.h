// Shared device helpers and internal launcher declarations of libmoe_mi355x.
// Everything here targets gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------
// vector types for MFMA operands and wide memory accesses
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // 16x16x32 / 32x32x16 bf16 operand
typedef __attribute__((ext_vector_type(4))) float f32x4;     // 16x16 accumulator
typedef __attribute__((ext_vector_type(16))) float f32x16;   // 32x32 accumulator
typedef __attribute__((ext_vector_type(8))) int i32x8;       // 16x16x128 fp8 operand (32 bytes)
typedef __attribute__((ext_vector_type(4))) int i32x4;       // 16-byte load
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int kWave = 64;
constexpr int kGroup = 128;   // fp8 activation group / weight block edge

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(uint32_t(b) << 16);
}

// fp32 -> bf16, round to nearest even (a bf16 is the upper half of an fp32
// word: add half an ulp of the kept part, plus one if the kept part is odd).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

__device__ __forceinline__ float round_bf16(float f) { return bf16_to_f32(f32_to_bf16_rne(f)); }

// The down GEMM's per-slot rows y: fp32 for layers with bf16 weights, bf16
// (round to nearest even) for fp8 and MXFP8 weights, whose e4m3 intermediate
// already carries a relative error of up to 2^-4 against bf16 y's 2^-9: it
// halves the y round trip between the down GEMM and the combine.
template <bool kBf16Y>
__device__ __forceinline__ void store_y4(float* y, int64_t idx, const f32x4& v) {
    if constexpr (kBf16Y) {
        uint2 p;
        p.x = uint32_t(f32_to_bf16_rne(v[0])) | (uint32_t(f32_to_bf16_rne(v[1])) << 16);
        p.y = uint32_t(f32_to_bf16_rne(v[2])) | (uint32_t(f32_to_bf16_rne(v[3])) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(y) + idx) = p;
    } else {
        *reinterpret_cast<f32x4*>(y + idx) = v;
    }
}

// fp32 -> OCP E4M3FN byte, round to nearest even.  The input must be finite
// and within [-448, 448] (callers clamp first).  E4M3FN: exponent bias 7,
// 3 fraction bits, subnormal quantum 2^-9 below 2^-6.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    float a = __builtin_fabsf(v);
    uint32_t code;
    if (a < 0.015625f) {                       // below 2^-6: multiples of 2^-9
        code = uint32_t(__builtin_rintf(a * 512.0f));   // exact scaling, RNE
    } else {
        uint32_t ua = u & 0x7fffffffu;
        uint32_t exp = (ua >> 23) - 127u + 7u;  // biased e4m3 exponent (1..15)
        uint32_t mant = ua & 0x7fffffu;
        uint32_t keep = mant >> 20;             // top 3 fraction bits
        uint32_t rest = mant & 0xfffffu;        // 20 dropped bits
        uint32_t up = (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
        code = (exp << 3) + keep + up;          // carry into the exponent is correct
    }
    return code | sign;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
    float a = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
    return (c & 0x80u) ? -a : a;
}

// Eight E4M3FN bytes (little-endian in two words) to the bf16 operand of a
// 16x16x32 bf16 MFMA lane, element i = byte i, each value code * scale.  For a
// power-of-two scale the result is exact while it stays within bf16's normal
// range (an e4m3 value has 4 significant bits).  gfx950 converts two bytes per
// instruction (checked on all 256 codes); the pairs are moved as whole words
// (element access on bf16 vectors compiled to wrong lane moves).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(int lo, int hi, float scale) {
    const int w0 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false));
    const int w1 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true));
    const int w2 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false));
    const int w3 = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true));
    return __builtin_bit_cast(bf16x8, i32x4{w0, w1, w2, w3});
}

// The value of an E8M0 scale byte as fp32: 2^(b - 127) (b = 0 is the fp32
// subnormal 2^-127; 255, the format's NaN, gives infinity).
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
    return __uint_as_float(b ? b << 23 : 0x00400000u);
}

// Smallest power of two >= s for a positive normal fp32 s, exact.
__device__ __forceinline__ float pow2_ceil(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffu) == 0) return s;
    return __uint_as_float(((u >> 23) + 1u) << 23);
}

// Group scale from the group's absolute maximum: the fp32 product
// max(amax, 1e-10) * (1/448), rounded up to a power of two.
__device__ __forceinline__ float fp8_group_scale(float amax) {
    const float s_raw = __fmul_rn(fmaxf(amax, 1e-10f), 1.0f / 448.0f);
    return pow2_ceil(s_raw);
}

// Quantise v with a power-of-two scale s: v / s is exact, clamp, RNE.
__device__ __forceinline__ uint32_t fp8_quant(float v, float inv_s) {
    float q = __fmul_rn(v, inv_s);             // inv_s is a power of two: exact
    q = fminf(fmaxf(q, -448.0f), 448.0f);
    return f32_to_e4m3_rne(q);
}

// SiLU-gated multiply with the fused kernel's rounding points:
// g, u already bf16 values; silu rounded to bf16; product rounded to bf16.
__device__ __forceinline__ float silu_mul_bf16(float g, float u) {
    const float e = expf(-g);
    const float s = round_bf16(__fdiv_rn(g, __fadd_rn(1.0f, e)));
    return round_bf16(__fmul_rn(s, u));
}

// The gate/up pair entering the SiLU-gated multiply.  w_in multiplies the
// fp32 GEMM1 results first (the row's router weight when it applies to the
// input, which GEMM1 is linear in; else 1, an exact no-op); then the bf16
// rounding points; then, with a clamp limit, the gate is capped at L and the
// up value held to [-L, L].
__device__ __forceinline__ float swiglu_bf16(float hg, float hu, float w_in, bool clamp, float L) {
    float gv = round_bf16(__fmul_rn(hg, w_in));
    float uv = round_bf16(__fmul_rn(hu, w_in));
    if (clamp) {
        gv = fminf(gv, L);
        uv = fminf(fmaxf(uv, -L), L);
    }
    return silu_mul_bf16(gv, uv);
}

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_max_16(float v) {
    // max over aligned groups of 16 lanes
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}

// ---------------------------------------------------------------------------
// internal launchers (each .hip file owns its kernels)
// ---------------------------------------------------------------------------
hipError_t launch_route(const float* logits, int T, int E, int topk, int renormalize,
                        int32_t* ids, float* weights, hipStream_t s);

hipError_t launch_align(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* inv,
                        hipStream_t s);

// Same output as launch_align, spread over many workgroups; needs
// align_scratch_bytes(R, E) bytes of scratch (4-byte aligned).
int64_t align_scratch_bytes(int64_t R, int E);
hipError_t launch_align_wide(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* inv,
                             void* scratch, hipStream_t s);

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                            hipStream_t s);
hipError_t launch_quant_act_mx(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                               hipStream_t s);
hipError_t launch_pack_mx_scales(const uint8_t* scales, int E, int rows, int K, uint8_t* packed, hipStream_t s);

struct GemmArgs {
    int T, E, H, I, topk, block_m, num_blocks;
    const uint16_t* x;          // bf16 [T,H]
    const uint8_t* xq;          // fp8 [T,H]
    const float* xs;            // fp32 [T,H/128] (fp8) or E8M0 bytes [T,H/32] (MXFP8)
    const void* w13;
    const void* w13_scale;      // fp32 [E,2I/128,H/128] (fp8) or E8M0 [E,2I,H/32] (MXFP8)
    const void* w2;
    const void* w2_scale;       // fp32 [E,H/128,I/128] (fp8) or E8M0 [E,H,I/32] (MXFP8)
    const float* topk_weights;  // [T*topk]
    const int32_t* sorted_ids;  // [cap]
    const int32_t* expert_ids;  // [num_blocks]
    const int32_t* ntpp;        // [1]
    void* inter;                // bf16 or fp8 [cap, I]
    float* inter_scale;         // fp32 [cap, I/128] (fp8) or E8M0 bytes [cap, I/32] (MXFP8)
    float* y;                   // [T*topk, H]: fp32 (bf16 weights) or bf16 (fp8, MXFP8 weights; store_y4)
    int weight_on_input;        // router weight on GEMM1's input instead of GEMM2's output
    int mx_packed;              // MXFP8 weight scales in the tile-packed layout (moe_pack_mx_scales)
    int krot;                   // the fp8 GEMM1 walks K from a per-(expert, column tile) start (k_rotation)
    int clamp;                  // SwiGLU clamp on (limit clamp_limit)
    float clamp_limit;
};

// First K step of the fp8 and MXFP8 GEMM1 for expert e's column tile (the
// walk wraps around).  With every workgroup starting at step 0, the whole
// chip reads the same byte offset of its weight rows at the same time;
// starting the experts' tiles at spread-out steps measured 25-35 % faster
// fp8 / MXFP8 GEMM1s where experts hold about one block each (64 and 256
// tokens of the fp8 layer: 127 -> 94 and 154 -> 109 us; MXFP8 at 256 tokens
// 166 -> 110 us).  The MXFP8 GEMM1 always starts there (also faster at 1024
// and 2048 tokens: 171 -> 163 and 307 -> 302 us); the fp8 one only up to 16
// routed rows per expert (GemmArgs::krot: at 1024 tokens 164 -> 172 us); the
// bf16 decode GEMM1 ran slower with it (355 -> 402 us) and does not use it.
// It depends on (e, tile) only, so a product's K order is the same for every
// block size and both launch forms.
__device__ __forceinline__ int k_rotation_start(int e, int tile, int nsteps) { return (e * 37 + tile * 11) % nsteps; }
__device__ __forceinline__ int k_rotation(const GemmArgs& g, int e, int tile, int nsteps) {
    return g.krot ? k_rotation_start(e, tile, nsteps) : 0;
}

// Router weight a GEMM1 epilogue applies to sorted slot f (1 unless the
// weight goes on the input; 0 for padding rows, which are never stored as
// real rows), and the one GEMM2's epilogue applies.
__device__ __forceinline__ float gemm1_row_weight(const GemmArgs& g, int f) {
    if (!g.weight_on_input) return 1.0f;
    return f < g.T * g.topk ? g.topk_weights[f] : 0.0f;
}
__device__ __forceinline__ float gemm2_row_weight(const GemmArgs& g, int f) {
    return g.weight_on_input ? 1.0f : g.topk_weights[f];
}

// Workgroup -> (block, column tile) over the blocks that hold routed rows
// (the first ntpp / block_m blocks; the rest of the capacity is tail).  The
// hardware deals workgroups to the 8 XCDs round-robin (workgroup i runs on
// XCD i % 8).  The active items are cut into 8 equal contiguous ranges, one
// per XCD, so every XCD gets the same work and neighbouring items share its
// L2.  Items are ordered tile-major (blocks of one expert, same weights,
// adjacent) or block-major (the column tiles of one block, same token rows,
// adjacent).  The grid is sized for the worst case (every capacity block
// active, 8 | grid); workgroups past their XCD's range exit at once.
template <bool kBlockMajor = false>
__device__ __forceinline__ bool map_active_tile(const GemmArgs& g, int ntiles, int& blk, int& tile) {
    const int active = __builtin_amdgcn_readfirstlane(g.ntpp[0]) / g.block_m;
    const int64_t total = int64_t(active) * ntiles;
    const int xcd = blockIdx.x & 7;
    const int64_t item = xcd * total / 8 + (blockIdx.x >> 3);
    if (item >= (xcd + 1) * total / 8) return false;
    if constexpr (kBlockMajor) {
        blk = int(item / ntiles);
        tile = int(item - int64_t(blk) * ntiles);
    } else {
        tile = int(item / active);
        blk = int(item - int64_t(tile) * active);
    }
    return true;
}

hipError_t launch_gemm1_small(const GemmArgs& g, bool fp8, hipStream_t s);
// NT = block_m / 16; mx: MXFP8 weights (their own kernels, the same tiles), else fp8 = block-scaled
int small_gemm2_cols(int T, int topk, int E, int H, int I, bool fp8, int NT, bool mx = false);
bool gemm2_lds_supported(int H, int I);       // bf16 down GEMM of 16-row blocks through LDS
bool gemm2_lds_fp8_supported(int H, int I);   // its block-fp8 form
hipError_t launch_gemm2_small(const GemmArgs& g, bool fp8, hipStream_t s);
hipError_t launch_gemm1_mx(const GemmArgs& g, hipStream_t s);   // MXFP8, block_m 16/32/64
hipError_t launch_gemm2_mx(const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm1_large(const GemmArgs& g, bool fp8, hipStream_t s);
hipError_t launch_gemm2_large(const GemmArgs& g, bool fp8, hipStream_t s);
bool gemm_large_supported(int H, int I, bool fp8);   // shapes the LDS-tiled bf16 path handles
int gemm_large_block_m();                            // its rows per expert block
// the LDS-tiled path for fp8 weights (128x128 block scales, or MXFP8)
bool gemm_large_q_supported(int H, int I);
int gemm_large_q_block_m();
hipError_t launch_gemm1_large_q(const GemmArgs& g, bool mx, hipStream_t s);
hipError_t launch_gemm2_large_q(const GemmArgs& g, bool mx, hipStream_t s);

// The single-launch decode layer (fused.hip): block_m 16 and the shapes below.
bool decode_layer_supported(int T, int topk, int H, int I, int block_m);
hipError_t launch_decode_layer(const GemmArgs& g, int wdtype_fp8, int mx, const float* logits, int renormalize,
                               int32_t* route_ids, float* route_weights, const int32_t* ids, int32_t* sorted,
                               int32_t* expert_ids, int32_t* ntpp, int cap, uint8_t* xq, void* xs, uint16_t* out,
                               uint32_t* sync, hipStream_t s);

// the one-workgroup alignment (up to kAlignWideMinSlots slots) and the fp8 /
// MXFP8 quantisation of x in one launch (align.hip)
hipError_t launch_align_quant(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                              int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, const uint16_t* x, int H,
                              uint8_t* xq, void* xs, bool mx, hipStream_t s);
hipError_t launch_combine(const float* y, bool bf16_y, const int32_t* ids, int T, int topk, int E, int H,
                          uint16_t* out, hipStream_t s);

}  // namespace moe
