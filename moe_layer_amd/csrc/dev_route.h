// Router softmax + top-k (P2 section 1.1: the layer is handed topk_ids and
// softmax router weights over the selected experts).
//
// One wavefront per token.  Lane l holds the logits of experts l, l+64, ...
// (up to 16 per lane for E <= 1024).  Each candidate is a 64-bit key: the
// logit's bits mapped to an order-preserving unsigned integer (-0 taken as
// +0) above the complement of the expert index, so the larger key is the
// larger logit and, on equal logits, the lower index.  Each of the k rounds
// takes the wave-wide maximum key over the experts not yet taken (DPP within
// rows of 16 lanes, two lane shuffles across rows), so the ids come out in
// descending-logit order with ties to the lower index.  Weights are
// exp(l_j - l_max) divided by the sum over the k winners (or over all experts
// when renormalize == 0), in fp32.
//
// Device code only (shared by route.hip's kernel and the single-launch decode
// layer in fused.hip).
#pragma once

#include "common.h"

namespace moe {

namespace {


constexpr int kMaxPerLane = 16;          // MOE_MAX_EXPERTS / 64

__device__ __forceinline__ uint32_t order_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0;                        // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t o = uint32_t(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t make_key(float v, int e) {
    return (uint64_t(order_key(v)) << 32) | uint32_t(0xffffu - e);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t k) {
    const int lo = __builtin_amdgcn_update_dpp(0, int(uint32_t(k)), CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, int(uint32_t(k >> 32)), CTRL, 0xf, 0xf, false);
    return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t k, int m) {
    const int lo = __shfl_xor(int(uint32_t(k)), m);
    const int hi = __shfl_xor(int(uint32_t(k >> 32)), m);
    return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

// maximum over the 64 lanes, returned on every lane
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
    uint64_t o;
    o = dpp64<0xb1>(k);  k = o > k ? o : k;     // quad_perm [1,0,3,2]
    o = dpp64<0x4e>(k);  k = o > k ? o : k;     // quad_perm [2,3,0,1]
    o = dpp64<0x141>(k); k = o > k ? o : k;     // row_half_mirror
    o = dpp64<0x140>(k); k = o > k ? o : k;     // row_mirror: row maximum on all 16 lanes
    o = shfl_xor64(k, 16); k = o > k ? o : k;
    o = shfl_xor64(k, 32); k = o > k ? o : k;
    return k;
}

// Experts per lane the routing code is instantiated for: E <= 64 * NPER.
// Fewer per lane is less code, and these one-shot kernels spend much of their
// time fetching instructions.
__host__ __device__ constexpr int route_nper(int E) {
    return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : kMaxPerLane;
}

// Route token t (< T) with the whole calling wave; E <= 64 * NPER.
template <int NPER>
__device__ __forceinline__ void route_token_n(const float* __restrict__ logits, int E, int topk,
                                              int renormalize, int32_t* __restrict__ ids,
                                              float* __restrict__ weights, int t) {
    static_assert(NPER >= 1 && NPER <= kMaxPerLane, "experts per lane");
    const int lane = threadIdx.x & 63;
    const float* row = logits + int64_t(t) * E;
    const int nper = (E + 63) >> 6;

    float v[NPER];
    uint64_t key[NPER];   // 0 = no candidate (below every real key)
#pragma unroll
    for (int i = 0; i < NPER; ++i) {
        const int e = lane + 64 * i;
        const bool ok = i < nper && e < E;
        v[i] = ok ? row[e] : 0.0f;
        key[i] = ok ? make_key(v[i], e) : 0ull;
    }

    float sel_v = 0.0f;   // lane j (< topk) keeps the j-th winner
    int sel_i = 0;
    for (int r = 0; r < topk; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < NPER; ++i) best = key[i] > best ? key[i] : best;
        const uint64_t w = wave_max_key(best);
        const int wi = int(0xffffu - uint32_t(w & 0xffffu));
        if ((wi & 63) == lane) {
#pragma unroll
            for (int i = 0; i < NPER; ++i)
                if (i == (wi >> 6)) key[i] = 0;
        }
        if (lane == r) {
            sel_v = key_value(w);
            sel_i = wi;
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
        for (int i = 0; i < NPER; ++i)
            if (i < nper && lane + 64 * i < E) part = __fadd_rn(part, expf(__fsub_rn(v[i], lmax)));
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

// route_token_n for any E <= MOE_MAX_EXPERTS (one instance per experts-per-lane count)
__device__ __forceinline__ void route_token(const float* __restrict__ logits, int E, int topk,
                                            int renormalize, int32_t* __restrict__ ids,
                                            float* __restrict__ weights, int t) {
    switch (route_nper(E)) {
        case 1: route_token_n<1>(logits, E, topk, renormalize, ids, weights, t); break;
        case 2: route_token_n<2>(logits, E, topk, renormalize, ids, weights, t); break;
        case 4: route_token_n<4>(logits, E, topk, renormalize, ids, weights, t); break;
        case 8: route_token_n<8>(logits, E, topk, renormalize, ids, weights, t); break;
        default: route_token_n<kMaxPerLane>(logits, E, topk, renormalize, ids, weights, t); break;
    }
}

}  // namespace

}  // namespace moe
