// Dynamic fp8 quantisation of the layer input, one power-of-two scale per row
// and 128-column group (the scale rule of the fused SiLU-mul-quant kernel in
// P2 section 1.2, applied per token to x as in the block-fp8 path), or per row
// and 32-column group with the scale stored as its E8M0 byte (MXFP8).
//
// Layout: 16 (MXFP8: 4) lanes own one group, 8 bf16 = 16 bytes per lane.
// HBM-bound: 2 bytes read and 1 written per element plus the scales.
#include "dev_quant.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / 16;

__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t* __restrict__ x,
                                                            int rows, int cols,
                                                            uint8_t* __restrict__ codes,
                                                            float* __restrict__ scales) {
    quant_group(x, rows, cols, codes, scales, int64_t(blockIdx.x) * kGroupsPerBlock + (threadIdx.x >> 4),
                threadIdx.x & 15);
}

__global__ __launch_bounds__(kThreads) void quant_act_mx_kernel(const uint16_t* __restrict__ x, int rows,
                                                               int cols, uint8_t* __restrict__ codes,
                                                               uint8_t* __restrict__ scales) {
    quant_group_mx(x, rows, cols, codes, scales, int64_t(blockIdx.x) * (kThreads / 4) + (threadIdx.x >> 2),
                   threadIdx.x & 3);
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
