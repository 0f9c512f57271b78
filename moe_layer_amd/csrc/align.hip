// Token-to-expert alignment (P2 section 1.1: sorted_token_ids,
// num_tokens_post_padded and the per-block expert of the block-sorted GEMM).
//
// Flat slots f = t*topk + j are cut into chunks that waves walk 64 slots at a
// time in ascending order.  A ballot multisplit (one ballot per bit of the
// expert id) gives each lane the mask of lanes holding the same expert, so
// ranks inside a 64-slot batch need no atomics.  Rows of one expert end up in
// ascending flat order because chunks are ascending and batches are walked in
// order: the output is a pure function of the input.
//
// Three forms with the same output:
//   align_tiny_kernel    one wave, up to 256 slots (decode): counts, scan over
//                        experts, stable scatter, tail; no scratch memory
//   align_kernel         one workgroup of 16 waves (no scratch memory):
//                        per-wave counts, scan, stable scatter, tail
//   align_count_kernel   many workgroups of 4 waves x 256 slots (1024 per
//   align_scan_kernel    workgroup): per-workgroup counts to scratch; one
//   align_scatter_kernel workgroup scans them into per-workgroup start
//                        positions, padding, tail and block experts; many
//                        workgroups scatter.  Used above 8192 slots, where
//                        one CU's ALUs would be the bottleneck.
// align_quant_kernel runs align_kernel (or the one-wave form) in workgroup 0
// and the fp8 / MXFP8 quantisation of the layer input in the others.
#include "dev_align.h"
#include "dev_quant.h"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBatchUnroll = 4;   // batches whose loads are issued together


__device__ __forceinline__ void align_one_wg(const int32_t* __restrict__ ids, int R, int E, int B, int cap,
                                             int32_t* __restrict__ sorted, int32_t* __restrict__ expert_ids,
                                             int32_t* __restrict__ ntpp, int32_t* __restrict__ inv) {
    __shared__ int cnt[kWaves * kMaxE];   // counts, then running start positions
    __shared__ int offs[kMaxE + 1];       // exclusive scan of padded sizes
    __shared__ int pstart[kMaxE];         // first padding slot of each expert
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
        pstart[tid] = run;
    }
    if (tid == 0) ntpp[0] = offs[E];
    __syncthreads();
    // padding: one wave per expert, consecutive lanes on consecutive slots (a
    // thread per expert writing its own run made every store touch 64 lines)
    for (int ee = w; ee < E; ee += kWaves)
        for (int p = pstart[ee] + lane; p < offs[ee + 1]; p += 64) sorted[p] = R;

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

__global__ __launch_bounds__(kThreads) void align_kernel(const int32_t* __restrict__ ids, int R,
                                                        int E, int B, int cap,
                                                        int32_t* __restrict__ sorted,
                                                        int32_t* __restrict__ expert_ids,
                                                        int32_t* __restrict__ ntpp,
                                                        int32_t* __restrict__ inv) {
    align_one_wg(ids, R, E, B, cap, sorted, expert_ids, ntpp, inv);
}

// The one-workgroup alignment and the layer input's fp8 quantisation in one
// launch: workgroup 0 aligns (on one CU), the others quantise x in a
// grid-stride loop (16 lanes per 128-column group, or 4 per 32-column MXFP8
// group), so the quantisation runs beside the alignment instead of after it.
// Up to kTinyMaxSlots slots workgroup 0 runs the one-wave alignment.
template <bool MX, bool TINY>
__global__ __launch_bounds__(kThreads) void align_quant_kernel(const int32_t* __restrict__ ids, int R, int E, int B,
                                                              int cap, int32_t* __restrict__ sorted,
                                                              int32_t* __restrict__ expert_ids,
                                                              int32_t* __restrict__ ntpp,
                                                              const uint16_t* __restrict__ x, int T, int H,
                                                              uint8_t* __restrict__ xq, void* __restrict__ xs) {
    if (blockIdx.x == 0) {
        if constexpr (TINY) {
            __shared__ int cnt[kMaxE];
            __shared__ int offs[kMaxE + 1];
            align_tiny_wg<kTinyBatches>(ids, R, E, B, cap, sorted, expert_ids, ntpp, nullptr, cnt, offs,
                                        threadIdx.x < 64);
        } else {
            align_one_wg(ids, R, E, B, cap, sorted, expert_ids, ntpp, nullptr);
        }
        return;
    }
    constexpr int kLanes = MX ? 4 : 16;
    constexpr int kPer = kThreads / kLanes;   // groups per workgroup and pass
    const int64_t groups = int64_t(T) * (H / (MX ? 32 : kGroup));
    for (int64_t base = int64_t(blockIdx.x - 1) * kPer; base < groups; base += int64_t(gridDim.x - 1) * kPer) {
        if constexpr (MX)
            quant_group_mx(x, T, H, xq, static_cast<uint8_t*>(xs), base + threadIdx.x / kLanes,
                           threadIdx.x % kLanes);
        else
            quant_group(x, T, H, xq, static_cast<float*>(xs), base + threadIdx.x / kLanes, threadIdx.x % kLanes);
    }
}

// ---------------------------------------------------------------------------
// one-wave form for few slots (decode): no cross-wave synchronisation
// ---------------------------------------------------------------------------
// NB 64-slot batches (R <= 64 * NB): less code for fewer slots, which is most
// of this one-shot kernel's time
template <int NB>
__global__ __launch_bounds__(64) void align_tiny_kernel(const int32_t* __restrict__ ids, int R, int E, int B,
                                                       int cap, int32_t* __restrict__ sorted,
                                                       int32_t* __restrict__ expert_ids,
                                                       int32_t* __restrict__ ntpp,
                                                       int32_t* __restrict__ inv) {
    __shared__ int cnt[kMaxE];
    __shared__ int offs[kMaxE + 1];
    align_tiny_wg<NB>(ids, R, E, B, cap, sorted, expert_ids, ntpp, inv, cnt, offs, true);
}

// ---------------------------------------------------------------------------
// multi-workgroup form
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 256;                  // 4 waves
constexpr int kWideWaves = kWideThreads / 64;
constexpr int kWideBatches = 4;                    // 64-slot batches per wave
constexpr int kWideSlots = kWideThreads * kWideBatches;   // slots per workgroup

__device__ __forceinline__ int expert_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// Per-wave expert counts of one workgroup's slots into cnt[w * E + e]
// (cnt zeroed by the caller); ev holds each lane's ids of its 4 batches.
__device__ __forceinline__ void wide_count(const int (&ev)[kWideBatches], int E, int* cnt) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const int nbits = expert_bits(E);
    int* my = cnt + w * E;
#pragma unroll
    for (int u = 0; u < kWideBatches; ++u) {
        const int e = ev[u];
        const bool valid = e >= 0 && e < E;
        const uint64_t m = peers(e, valid, nbits);
        if (valid && (m & lt_mask) == 0) my[e] += __popcll(m);
    }
}

__device__ __forceinline__ void wide_load(const int32_t* ids, int R, int (&ev)[kWideBatches]) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int base = blockIdx.x * kWideSlots + w * 64 * kWideBatches;
#pragma unroll
    for (int u = 0; u < kWideBatches; ++u) {
        const int f = base + 64 * u + lane;
        ev[u] = f < R ? ids[f] : -1;
    }
}

// counts[g * E + e] = slots of expert e among workgroup g's slots
__global__ __launch_bounds__(kWideThreads) void align_count_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                   int32_t* __restrict__ counts) {
    __shared__ int cnt[kWideWaves * kMaxE];
    const int tid = threadIdx.x;
    int ev[kWideBatches];
    wide_load(ids, R, ev);
    for (int i = tid; i < kWideWaves * E; i += kWideThreads) cnt[i] = 0;
    __syncthreads();
    wide_count(ev, E, cnt);
    __syncthreads();
    for (int e = tid; e < E; e += kWideThreads) {
        int c = 0;
#pragma unroll
        for (int w = 0; w < kWideWaves; ++w) c += cnt[w * E + e];
        counts[int64_t(blockIdx.x) * E + e] = c;
    }
}

// One workgroup: padded sizes, exclusive scan over experts, the start of
// every (workgroup, expert) run, padding and tail sentinels, block experts,
// padded total.  Threads are split as (expert, part): the parts of one
// expert cover consecutive ranges of workgroups.
__global__ __launch_bounds__(kThreads) void align_scan_kernel(const int32_t* __restrict__ counts, int ngroups,
                                                              int R, int E, int B, int cap,
                                                              int32_t* __restrict__ starts,
                                                              int32_t* __restrict__ sorted,
                                                              int32_t* __restrict__ expert_ids,
                                                              int32_t* __restrict__ ntpp) {
    __shared__ int part_sum[kThreads];
    __shared__ int offs[kMaxE + 1];
    __shared__ int pstart[kMaxE];
    __shared__ int wsum[kWaves];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    int ep = 1;
    while (ep < E) ep <<= 1;                       // experts rounded up to a power of two
    const int parts = kThreads / ep;
    const int e = tid & (ep - 1), part = tid / ep;
    const int per = (ngroups + parts - 1) / parts;
    const int q0 = min(ngroups, part * per), q1 = min(ngroups, q0 + per);
    int local = 0;
    if (e < E) {
#pragma unroll 8
        for (int q = q0; q < q1; ++q) local += counts[int64_t(q) * E + e];
    }
    part_sum[tid] = local;
    __syncthreads();

    int padded = 0, total = 0;
    if (tid < E) {
        for (int pp = 0; pp < parts; ++pp) total += part_sum[pp * ep + tid];
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
        if (lane < kWaves) wsum[lane] = si - s;
    }
    __syncthreads();
    if (tid < E) {
        const int excl = incl - padded + wsum[w];
        offs[tid] = excl;
        if (tid == E - 1) offs[E] = excl + padded;
    }
    __syncthreads();

    if (e < E) {
        const int beg = offs[e], end = offs[e + 1];
        int run = beg;
        int filled = 0;                            // rows of expert e over all parts
        for (int pp = 0; pp < parts; ++pp) {
            const int c = part_sum[pp * ep + e];
            if (pp < part) run += c;
            filled += c;
        }
#pragma unroll 8
        for (int q = q0; q < q1; ++q) {
            const int64_t i = int64_t(q) * E + e;
            starts[i] = run;
            run += counts[i];
        }
        if (part == 0) pstart[e] = beg + filled;
    }
    __syncthreads();
    // padding and block experts: one wave per expert, consecutive lanes on
    // consecutive slots (threads of different experts made every store touch
    // 64 lines: 17.5 us for the fp8 layer's 256 experts)
    for (int ee = w; ee < E; ee += kWaves) {
        const int beg = offs[ee], end = offs[ee + 1];
        for (int p = pstart[ee] + lane; p < end; p += 64) sorted[p] = R;
        for (int b = beg / B + lane; b < end / B; b += 64) expert_ids[b] = ee;
    }
    const int all = offs[E];
    if (tid == 0) ntpp[0] = all;
    for (int p = all + tid; p < cap; p += kThreads) sorted[p] = R;
    const int nblocks = (cap + B - 1) / B;
    for (int b = all / B + tid; b < nblocks; b += kThreads) expert_ids[b] = -1;
}

// Scatter: the workgroup's per-wave counts again (its slots), each wave's
// start per expert = the workgroup's start + the counts of the waves before
// it, then the stable scatter.
__global__ __launch_bounds__(kWideThreads) void align_scatter_kernel(const int32_t* __restrict__ ids, int R, int E,
                                                                     const int32_t* __restrict__ starts,
                                                                     int32_t* __restrict__ sorted,
                                                                     int32_t* __restrict__ inv) {
    __shared__ int cnt[kWideWaves * kMaxE];
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    const int nbits = expert_bits(E);
    int ev[kWideBatches];
    wide_load(ids, R, ev);
    for (int i = tid; i < kWideWaves * E; i += kWideThreads) cnt[i] = 0;
    __syncthreads();
    wide_count(ev, E, cnt);
    __syncthreads();
    const int32_t* st = starts + int64_t(blockIdx.x) * E;
    for (int e = tid; e < E; e += kWideThreads) {
        int run = st[e];
#pragma unroll
        for (int ww = 0; ww < kWideWaves; ++ww) {
            const int c = cnt[ww * E + e];
            cnt[ww * E + e] = run;
            run += c;
        }
    }
    __syncthreads();
    int* my = cnt + w * E;
    const int base = blockIdx.x * kWideSlots + w * 64 * kWideBatches;
#pragma unroll
    for (int u = 0; u < kWideBatches; ++u) {
        const int f = base + 64 * u + lane;
        const int e = ev[u];
        const bool valid = e >= 0 && e < E;
        const uint64_t m = peers(e, valid, nbits);
        if (valid) {
            const int pos = my[e] + __popcll(m & lt_mask);
            sorted[pos] = f;
            if (inv) inv[f] = pos;
        } else if (f < R && inv) {
            inv[f] = -1;
        }
        if (valid && (m & lt_mask) == 0) my[e] += __popcll(m);
    }
}

}  // namespace

hipError_t launch_align(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                        int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* inv,
                        hipStream_t s) {
    const int R = T * topk;
    if (R <= kTinyMaxSlots) {
        auto k = R <= 64 ? align_tiny_kernel<1> : R <= 128 ? align_tiny_kernel<2> : align_tiny_kernel<kTinyBatches>;
        hipLaunchKernelGGL(k, dim3(1), dim3(64), 0, s, ids, R, E, block_m, int(cap), sorted_ids, expert_ids, ntpp,
                           inv);
    } else {
        hipLaunchKernelGGL(align_kernel, dim3(1), dim3(kThreads), 0, s, ids, R, E, block_m, int(cap), sorted_ids,
                           expert_ids, ntpp, inv);
    }
    return hipGetLastError();
}

int64_t align_scratch_bytes(int64_t R, int E) {
    const int64_t groups = (R + kWideSlots - 1) / kWideSlots;
    return 2 * groups * E * int64_t(sizeof(int32_t));
}

hipError_t launch_align_quant(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                              int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, const uint16_t* x, int H,
                              uint8_t* xq, void* xs, bool mx, hipStream_t s) {
    const int R = T * topk;
    const int64_t groups = int64_t(T) * (H / (mx ? 32 : kGroup));
    const int64_t per = kThreads / (mx ? 4 : 16);
    const int64_t qwg = std::min<int64_t>(std::max<int64_t>((groups + per - 1) / per, 1), 2048);
    const bool tiny = R <= kTinyMaxSlots;
    void (*k)(const int32_t*, int, int, int, int, int32_t*, int32_t*, int32_t*, const uint16_t*, int, int,
              uint8_t*, void*) = mx ? (tiny ? align_quant_kernel<true, true> : align_quant_kernel<true, false>)
                                    : (tiny ? align_quant_kernel<false, true> : align_quant_kernel<false, false>);
    hipLaunchKernelGGL(k, dim3(unsigned(1 + qwg)), dim3(kThreads), 0, s, ids, R, E, block_m, int(cap), sorted_ids,
                       expert_ids, ntpp, x, T, H, xq, xs);
    return hipGetLastError();
}

hipError_t launch_align_wide(const int32_t* ids, int T, int topk, int E, int block_m, int64_t cap,
                             int32_t* sorted_ids, int32_t* expert_ids, int32_t* ntpp, int32_t* inv,
                             void* scratch, hipStream_t s) {
    const int R = T * topk;
    const int groups = (R + kWideSlots - 1) / kWideSlots;
    int32_t* counts = static_cast<int32_t*>(scratch);
    int32_t* starts = counts + int64_t(groups) * E;
    hipLaunchKernelGGL(align_count_kernel, dim3(groups), dim3(kWideThreads), 0, s, ids, R, E, counts);
    hipLaunchKernelGGL(align_scan_kernel, dim3(1), dim3(kThreads), 0, s, counts, groups, R, E, block_m, int(cap),
                       starts, sorted_ids, expert_ids, ntpp);
    hipLaunchKernelGGL(align_scatter_kernel, dim3(groups), dim3(kWideThreads), 0, s, ids, R, E, starts,
                       sorted_ids, inv);
    return hipGetLastError();
}

}  // namespace moe
