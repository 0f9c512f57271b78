// Token-to-expert alignment (P2 section 1.1: sorted_token_ids,
// num_tokens_post_padded and the per-block expert of the block-sorted GEMM).
//
// One workgroup of 16 waves.  The flat slots f = t*topk + j are cut into 16
// contiguous chunks, one per wave, and every wave walks its chunk 64 slots at
// a time in ascending order.  A ballot multisplit (one ballot per bit of the
// expert id) gives each lane the mask of lanes holding the same expert, so
// ranks inside a 64-slot batch need no atomics:
//   phase 1  per-wave expert counts cnt[w][e]
//   phase 2  padded sizes, exclusive scan over experts, per-(wave, expert)
//            start positions; padding slots of each expert get the sentinel
//   phase 3  stable scatter: position = start[w][e] + rank inside the batch
//   phase 4  tail of sorted_token_ids and expert_ids of every block
// The output is a pure function of the input: rows of one expert appear in
// ascending flat order because waves own ascending chunks and batches are
// walked in order.
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 1024;
constexpr int kBatchUnroll = 4;   // batches whose loads are issued together

__device__ __forceinline__ uint64_t peers(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (e >> b) & 1;
        const uint64_t bb = __ballot(valid && bit);
        m &= bit ? bb : ~bb;
    }
    return valid ? m : 0ull;
}

__global__ __launch_bounds__(kThreads) void align_kernel(const int32_t* __restrict__ ids, int R,
                                                        int E, int B, int cap,
                                                        int32_t* __restrict__ sorted,
                                                        int32_t* __restrict__ expert_ids,
                                                        int32_t* __restrict__ ntpp,
                                                        int32_t* __restrict__ inv) {
    __shared__ int cnt[kWaves * kMaxE];   // counts, then running start positions
    __shared__ int offs[kMaxE + 1];       // exclusive scan of padded sizes
    __shared__ int wsum[kWaves];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;

    for (int i = tid; i < kWaves * E; i += kThreads) cnt[i] = 0;
    __syncthreads();

    const int chunk = (((R + kWaves - 1) / kWaves) + 63) & ~63;
    const int begin = min(R, w * chunk);
    const int end = min(R, begin + chunk);
    int* my = cnt + w * E;

    // ---- phase 1: per-wave counts ------------------------------------------
    for (int base = begin; base < end; base += 64 * kBatchUnroll) {
        int ev[kBatchUnroll];
#pragma unroll
        for (int u = 0; u < kBatchUnroll; ++u) {
            const int f = base + 64 * u + lane;
            ev[u] = f < end ? ids[f] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatchUnroll; ++u) {
            const int e = ev[u];
            const bool valid = e >= 0 && e < E;
            const uint64_t m = peers(e, valid, nbits);
            if (valid && (m & lt_mask) == 0) my[e] += __popcll(m);
        }
    }
    __syncthreads();

    // ---- phase 2: padded sizes, scan, start positions ------------------------
    int padded = 0;
    if (tid < E) {
        int total = 0;
        for (int ww = 0; ww < kWaves; ++ww) total += cnt[ww * E + tid];
        padded = (total + B - 1) / B * B;
    }
    int incl = padded;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(incl, d);
        if (lane >= d) incl += o;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    if (w == 0) {
        int s = lane < kWaves ? wsum[lane] : 0;
        int si = s;
#pragma unroll
        for (int d = 1; d < kWaves; d <<= 1) {
            const int o = __shfl_up(si, d);
            if (lane >= d) si += o;
        }
        if (lane < kWaves) wsum[lane] = si - s;   // exclusive wave offsets
    }
    __syncthreads();
    if (tid < E) {
        const int excl = incl - padded + wsum[w];
        offs[tid] = excl;
        if (tid == E - 1) offs[E] = excl + padded;
    }
    __syncthreads();
    if (tid < E) {
        int run = offs[tid];
        for (int ww = 0; ww < kWaves; ++ww) {
            const int c = cnt[ww * E + tid];
            cnt[ww * E + tid] = run;
            run += c;
        }
        for (int p = run; p < offs[tid + 1]; ++p) sorted[p] = R;   // padding of expert tid
    }
    if (tid == 0) ntpp[0] = offs[E];
    __syncthreads();

    // ---- phase 3: stable scatter ---------------------------------------------
    for (int base = begin; base < end; base += 64 * kBatchUnroll) {
        int ev[kBatchUnroll];
#pragma unroll
        for (int u = 0; u < kBatchUnroll; ++u) {
            const int f = base + 64 * u + lane;
            ev[u] = f < end ? ids[f] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatchUnroll; ++u) {
            const int f = base + 64 * u + lane;
            const int e = ev[u];
            const bool valid = e >= 0 && e < E;
            const uint64_t m = peers(e, valid, nbits);
            if (valid) {
                const int pos = my[e] + __popcll(m & lt_mask);
                sorted[pos] = f;
                if (inv) inv[f] = pos;
            } else if (f < end && inv) {
                inv[f] = -1;
            }
            // all reads of my[] above precede the leader's update (same wave, in order)
            if (valid && (m & lt_mask) == 0) my[e] += __popcll(m);
        }
    }

    // ---- phase 4: tail and block experts ---------------------------------------
    const int total = offs[E];
    for (int p = total + tid; p < cap; p += kThreads) sorted[p] = R;
    const int nblocks = (cap + B - 1) / B;
    for (int b = tid; b < nblocks; b += kThreads) {
        const int row = b * B;
        int e = -1;
        if (row < total) {
            int lo = 0, hi = E;   // first index u in [0, E] with offs[u] > row
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (offs[mid] > row) hi = mid; else lo = mid + 1;
            }
            e = lo - 1;
        }
        expert_ids[b] = e;
    }
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* inv,
                        hipStream_t s) {
    hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), 0, s, ids, T * topk, E, block_m,
                       int(cap), sorted_ids, expert_ids, ntpp, inv);
    return hipGetLastError();
}

}  // namespace moe
