// Token-to-expert alignment, device code shared by align.hip and the
// single-launch decode layer in fused.hip: the ballot multisplit and the
// one-wave form for up to kTinyMaxSlots slots (descriptions in align.hip).
#pragma once

#include "common.h"

namespace moe {

namespace {

constexpr int kMaxE = 1024;
constexpr int kTinyBatches = 4;
constexpr int kTinyMaxSlots = 64 * kTinyBatches;

// Mask of the lanes whose (valid) expert id equals this lane's: one ballot per
// bit of the id.
__device__ __forceinline__ uint64_t peers(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

// The alignment of R <= 64 * NB (NB <= kTinyBatches) slots by one wave.
// Called by every wave of a workgroup (its barriers are workgroup barriers);
// only waves with act set do the work, so pass act for exactly one wave.
// cnt[kMaxE] and offs[kMaxE + 1] are LDS scratch.
template <int NB = kTinyBatches>
__device__ __forceinline__ void align_tiny_wg(const int32_t* __restrict__ ids, int R, int E, int B, int cap,
                                              int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids,
                                              int32_t* __restrict__ ntpp, int32_t* __restrict__ inv, int* cnt,
                                              int* offs, bool act) {
    static_assert(NB >= 1 && NB <= kTinyBatches, "64-slot batches");
    const int lane = threadIdx.x & 63;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    int ev[NB];
    uint64_t m[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int f = 64 * u + lane;
        ev[u] = act && f < R ? ids[f] : -1;
        m[u] = 0;
    }
    if (act)
        for (int e = lane; e < E; e += 64) cnt[e] = 0;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        if (act) {
            const int e = ev[u];
            const bool valid = e >= 0 && e < E;
            m[u] = peers(e, valid, nbits);
            if (valid && (m[u] & lt_mask) == 0) cnt[e] += __popcll(m[u]);
        }
        __syncthreads();   // batches of one expert update its count in order
    }
    if (act) {
        // lane owns experts [lane * per, lane * per + per): padded sizes, scan
        const int per = (E + 63) / 64;
        const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
        int mine = 0;
        for (int e = e0; e < e1; ++e) mine += (cnt[e] + B - 1) / B * B;
        int incl = mine;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            if (lane >= d) incl += o;
        }
        int run = incl - mine;
        for (int e = e0; e < e1; ++e) {
            const int c = cnt[e];
            const int padded = (c + B - 1) / B * B;
            offs[e] = run;
            for (int p = run + c; p < run + padded; ++p) sorted[p] = R;            // padding
            for (int b = run / B; b < (run + padded) / B; ++b) expert_ids[b] = e;  // its blocks
            cnt[e] = run;
            run += padded;
        }
        const int total = __shfl(incl, 63);
        if (lane == 0) {
            offs[E] = total;
            ntpp[0] = total;
        }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int f = 64 * u + lane;
        const int e = ev[u];
        const bool valid = e >= 0 && e < E;
        if (act) {
            if (valid) {
                const int pos = cnt[e] + __popcll(m[u] & lt_mask);
                sorted[pos] = f;
                if (inv) inv[f] = pos;
            } else if (f < R && inv) {
                inv[f] = -1;
            }
        }
        __syncthreads();
        if (act && valid && (m[u] & lt_mask) == 0) cnt[e] += __popcll(m[u]);
        __syncthreads();
    }
    if (act) {
        const int total = offs[E];
        for (int p = total + lane; p < cap; p += 64) sorted[p] = R;
        const int nblocks = (cap + B - 1) / B;
        for (int b = total / B + lane; b < nblocks; b += 64) expert_ids[b] = -1;
    }
}

}  // namespace

}  // namespace moe
