// Router softmax + top-k kernel and launcher; the device code and its
// description are in dev_route.h.
#include "dev_route.h"

namespace moe {

namespace {

constexpr int kTokensPerBlock = 4;   // one wave per token

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                   int topk, int renormalize,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
    const int t = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;   // whole wave exits together
    route_token(logits, E, topk, renormalize, ids, weights, t);
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int topk, int renormalize,
                        int32_t* ids, float* weights, hipStream_t s) {
    const int blocks = (T + kTokensPerBlock - 1) / kTokensPerBlock;
    hipLaunchKernelGGL(route_kernel, dim3(blocks), dim3(64 * kTokensPerBlock), 0, s, logits, T, E,
                       topk, renormalize, ids, weights);
    return hipGetLastError();
}

}  // namespace moe
