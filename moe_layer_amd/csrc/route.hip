// Router softmax + top-k kernel and launcher; the device code and its
// description are in dev_route.h.
#include "dev_route.h"

namespace moe {

namespace {

constexpr int kTokensPerBlock = 4;   // one wave per token

template <int NPER>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                   int topk, int renormalize,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
    const int t = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;   // whole wave exits together
    route_token_n<NPER>(logits, E, topk, renormalize, ids, weights, t);
}

template <int NPER>
hipError_t launch_route_n(const float* logits, int T, int E, int topk, int renormalize, int32_t* ids,
                          float* weights, hipStream_t s) {
    const int blocks = (T + kTokensPerBlock - 1) / kTokensPerBlock;
    hipLaunchKernelGGL(route_kernel<NPER>, dim3(blocks), dim3(64 * kTokensPerBlock), 0, s, logits, T, E,
                       topk, renormalize, ids, weights);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, int T, int E, int topk, int renormalize,
                        int32_t* ids, float* weights, hipStream_t s) {
    switch (route_nper(E)) {
        case 1: return launch_route_n<1>(logits, T, E, topk, renormalize, ids, weights, s);
        case 2: return launch_route_n<2>(logits, T, E, topk, renormalize, ids, weights, s);
        case 4: return launch_route_n<4>(logits, T, E, topk, renormalize, ids, weights, s);
        case 8: return launch_route_n<8>(logits, T, E, topk, renormalize, ids, weights, s);
        default: return launch_route_n<kMaxPerLane>(logits, T, E, topk, renormalize, ids, weights, s);
    }
}

}  // namespace moe
