// Dynamic fp8 quantisation of the layer input, one power-of-two scale per row
// and 128-column group (the scale rule of the fused SiLU-mul-quant kernel in
// P2 section 1.2, applied per token to x as in the block-fp8 path).
//
// Layout: 16 lanes own one 128-column group (8 bf16 = 16 bytes per lane), so a
// wave covers 4 groups and a 256-thread block 16 groups.  HBM-bound: 2 bytes
// read and 1 written per element plus 4 bytes of scale per group.
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

}  // namespace

hipError_t launch_quant_act(const uint16_t* x, int rows, int cols, uint8_t* codes, float* scales,
                            hipStream_t s) {
    const int64_t groups = int64_t(rows) * (cols / kGroup);
    const int64_t blocks = (groups + kGroupsPerBlock - 1) / kGroupsPerBlock;
    hipLaunchKernelGGL(quant_act_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, s, x, rows, cols,
                       codes, scales);
    return hipGetLastError();
}

}  // namespace moe
