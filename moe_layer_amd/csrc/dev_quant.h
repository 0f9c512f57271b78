// Dynamic fp8 quantisation of activations, device code shared by quant.hip
// and the single-launch decode layer in fused.hip (description in quant.hip).
#pragma once

#include "common.h"

namespace moe {

namespace {

// Group g (row-major over rows x cols/128 groups) by 16 lanes; sub = lane
// index within the group (0..15), 8 elements each.  Lanes of an aligned group
// of 16 must call it together (the amax is a 16-lane reduction).
__device__ __forceinline__ void quant_group(const uint16_t* __restrict__ x, int rows, int cols,
                                            uint8_t* __restrict__ codes, float* __restrict__ scales, int64_t g,
                                            int sub) {
    const int groups_per_row = cols / kGroup;
    const int64_t total = int64_t(rows) * groups_per_row;
    const bool active = g < total;
    const int64_t row = active ? g / groups_per_row : 0;
    const int64_t col = active ? (g % groups_per_row) * kGroup + sub * 8 : 0;
    const int64_t off = row * cols + col;

    i32x4 raw = {0, 0, 0, 0};
    if (active) raw = *reinterpret_cast<const i32x4*>(x + off);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = uint32_t(raw[i]);
        v[2 * i] = bf16_to_f32(uint16_t(w & 0xffffu));
        v[2 * i + 1] = bf16_to_f32(uint16_t(w >> 16));
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
    amax = wave_max_16(amax);
    const float s = fp8_group_scale(amax);
    const float inv_s = __fdiv_rn(1.0f, s);   // exact: s is a power of two
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= fp8_quant(v[i], inv_s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= fp8_quant(v[4 + i], inv_s) << (8 * i);
    if (active) {
        i32x2 packed = {int(lo), int(hi)};
        *reinterpret_cast<i32x2*>(codes + off) = packed;
        if (sub == 0) scales[g] = s;
    }
}

// MXFP8: group g of 32 columns by 4 lanes (sub = 0..3); the scale, a normal
// power of two, is stored as its biased exponent, which is its E8M0 byte.
__device__ __forceinline__ void quant_group_mx(const uint16_t* __restrict__ x, int rows, int cols,
                                               uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                               int64_t g, int sub) {
    constexpr int kMx = 32;
    const int groups_per_row = cols / kMx;
    const int64_t total = int64_t(rows) * groups_per_row;
    const bool active = g < total;
    const int64_t row = active ? g / groups_per_row : 0;
    const int64_t col = active ? (g % groups_per_row) * kMx + sub * 8 : 0;
    const int64_t off = row * cols + col;

    i32x4 raw = {0, 0, 0, 0};
    if (active) raw = *reinterpret_cast<const i32x4*>(x + off);
    float v[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = uint32_t(raw[i]);
        v[2 * i] = bf16_to_f32(uint16_t(w & 0xffffu));
        v[2 * i + 1] = bf16_to_f32(uint16_t(w >> 16));
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1));
    amax = fmaxf(amax, __shfl_xor(amax, 2));
    const float s = fp8_group_scale(amax);
    const float inv_s = __fdiv_rn(1.0f, s);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= fp8_quant(v[i], inv_s) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= fp8_quant(v[4 + i], inv_s) << (8 * i);
    if (active) {
        i32x2 packed = {int(lo), int(hi)};
        *reinterpret_cast<i32x2*>(codes + off) = packed;
        if (sub == 0) scales[g] = uint8_t(__float_as_uint(s) >> 23);
    }
}

}  // namespace

}  // namespace moe
