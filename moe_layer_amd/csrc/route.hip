// Router softmax + top-k (P2 section 1.1: the layer is handed topk_ids and
// softmax router weights over the selected experts).
//
// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// (up to 16 per lane for E <= 1024).  Each of the k rounds takes a wave-wide
// argmax on the key (logit descending, expert index ascending) over the
// experts not yet taken, so ties go to the lower index and the ids come out in
// descending-logit order.  Weights are exp(l_j - l_max) divided by the sum over
// the k winners (or over all experts when renormalize == 0), in fp32.
#include "common.h"

namespace moe {

namespace {

constexpr int kMaxPerLane = 16;          // MOE_MAX_EXPERTS / 64
constexpr int kTokensPerBlock = 4;       // one wave per token

// key comparison: a beats b if it has a larger logit, or the same logit and a
// lower index; an invalid candidate never beats a valid one.
__device__ __forceinline__ bool beats(bool va, float a, int ia, bool vb, float b, int ib) {
    if (va != vb) return va;
    if (a != b) return a > b;
    return ia < ib;
}

__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T, int E,
                                                   int topk, int renormalize,
                                                   int32_t* __restrict__ ids,
                                                   float* __restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= T) return;   // whole wave exits together
    const float* row = logits + int64_t(t) * E;
    const int nper = (E + 63) >> 6;

    float v[kMaxPerLane];
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
        const int e = lane + 64 * i;
        v[i] = (i < nper && e < E) ? row[e] : 0.0f;
    }
    uint32_t avail = 0;   // bit i: slot i holds an untaken expert
    for (int i = 0; i < nper; ++i)
        if (lane + 64 * i < E) avail |= 1u << i;

    const uint32_t avail0 = avail;
    float sel_v = 0.0f;   // lane j (< topk) keeps the j-th winner
    int sel_i = 0;
    for (int r = 0; r < topk; ++r) {
        // best candidate of this lane (slots ascend in expert index)
        bool bv = false;
        float b = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i) {
            const bool ok = (avail >> i) & 1u;
            if (ok && beats(true, v[i], lane + 64 * i, bv, b, bi)) {
                bv = true;
                b = v[i];
                bi = lane + 64 * i;
            }
        }
        // butterfly argmax across the wave
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const bool ov = __shfl_xor(int(bv), m) != 0;
            const float o = __shfl_xor(b, m);
            const int oi = __shfl_xor(bi, m);
            if (beats(ov, o, oi, bv, b, bi)) {
                bv = ov;
                b = o;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) avail &= ~(1u << (bi >> 6));
        if (lane == r) {
            sel_v = b;
            sel_i = bi;
        }
    }

    const float lmax = __shfl(sel_v, 0);
    float denom;
    if (renormalize) {
        // fixed order j = 0..k-1 on every lane
        float ex = lane < topk ? expf(__fsub_rn(sel_v, lmax)) : 0.0f;
        denom = 0.0f;
        for (int j = 0; j < topk; ++j) denom = __fadd_rn(denom, __shfl(ex, j));
    } else {
        float part = 0.0f;
#pragma unroll
        for (int i = 0; i < kMaxPerLane; ++i)
            if ((avail0 >> i) & 1u) part = __fadd_rn(part, expf(__fsub_rn(v[i], lmax)));
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) part = __fadd_rn(part, __shfl_xor(part, m));
        denom = part;
    }
    if (lane < topk) {
        const float ex = expf(__fsub_rn(sel_v, lmax));
        ids[int64_t(t) * topk + lane] = sel_i;
        weights[int64_t(t) * topk + lane] = __fdiv_rn(ex, denom);
    }
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
