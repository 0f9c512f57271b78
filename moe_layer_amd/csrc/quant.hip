// Dynamic fp8 quantisation of the layer input, one power-of-two scale per row
// and 128-column group (the scale rule of the fused SiLU-mul-quant kernel in
// P2 section 1.2, applied per token to x as in the block-fp8 path), or per row
// and 32-column group with the scale stored as its E8M0 byte (MXFP8).
//
// Layout: 16 (MXFP8: 4) lanes own one group, 8 bf16 = 16 bytes per lane.
// HBM-bound: 2 bytes read and 1 written per element plus the scales.
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / 16;

__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                            int rows, int cols,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    const int groups_per_row = cols / kGroup;
    const int64_t total = int64_t(rows) * groups_per_row;
    const int64_t g = int64_t(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15;
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

// MXFP8: 4 lanes per 32-column group; the scale, a normal power of two, is
// stored as its biased exponent, which is its E8M0 byte.
__global__ __launch_bounds__(kThreads) void quant_act_mx_kernel(const uint16_t* __restrict__ x, int rows,
                                                               int cols, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
    constexpr int kMx = 32;
    const int groups_per_row = cols / kMx;
    const int64_t total = int64_t(rows) * groups_per_row;
    const int64_t g = int64_t(blockIdx.x) * (kThreads / 4) + (threadIdx.x >> 2);
    const int sub = threadIdx.x & 3;
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

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                            hipStream_t s) {
    const int64_t groups = int64_t(rows) * (cols / kGroup);
    const int64_t blocks = (groups + kGroupsPerBlock - 1) / kGroupsPerBlock;
    hipLaunchKernelGGL(quant_act_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, x, rows, cols,
                       codes, scales);
    return hipGetLastError();
}

hipError_t launch_quant_act_mx(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                               hipStream_t s) {
    const int64_t groups = int64_t(rows) * (cols / 32);
    const int64_t blocks = (groups + kThreads / 4 - 1) / (kThreads / 4);
    hipLaunchKernelGGL(quant_act_mx_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, x, rows, cols, codes,
                       scales);
    return hipGetLastError();
}

}  // namespace moe
