// Top-k combine kernel and launcher; the device code and its description are
// in dev_combine.h.
#include "dev_combine.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

template <bool kBf16Y>
__global__ __launch_bounds__(kThreads) void combine_kernel(const float* __restrict__ y,
                                                          const int32_t* __restrict__ ids, int T,
                                                          int topk, int E, int H,
                                                          uint16_t* __restrict__ out) {
    const int per_row = H / 8;
    const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (i >= int64_t(T) * per_row) return;
    const int t = int(i / per_row);
    combine_chunk<kBf16Y>(y, ids, topk, E, H, out, t, int(i - int64_t(t) * per_row) * 8);
}

}  // namespace

hipError_t launch_combine(const float* y, bool bf16_y, const int32_t* ids, int T, int topk, int E, int H,
                          uint16_t* out, hipStream_t s) {
    const int64_t n = int64_t(T) * (H / 8);
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    void (*kern)(const float*, const int32_t*, int, int, int, int, uint16_t*) =
        bf16_y ? combine_kernel<true> : combine_kernel<false>;
    hipLaunchKernelGGL(kern, dim3(unsigned(blocks)), dim3(kThreads), 0, s, y, ids, T, topk, E, H, out);
    return hipGetLastError();
}

}  // namespace moe
