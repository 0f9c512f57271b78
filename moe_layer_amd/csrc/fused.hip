// The whole layer for few tokens (decode) as one persistent kernel: router
// top-k (from logits, optional) and activation quantisation -> alignment ->
// GEMM1 + SiLU-mul epilogue -> GEMM2 -> top-k combine, the phases separated by
// grid-wide barriers instead of kernel boundaries.  P3 (section on MoE
// dispatch/combine) fuses its decode-side kernel into one for the same reason:
// at a few tokens per step the per-kernel latency of the short phases (route,
// align, combine: a few microseconds each) is a visible share of the layer.
//
// Measured on MI355X, this is slower than the kernel-per-stage sequence of
// moe_forward (one token, 8 of 256 experts, H 7168, I 2048: 0.215 against
// 0.141 ms): a grid barrier across the 8 XCDs (write-back of the writer's L2,
// invalidation of the reader's, cross-XCD atomics) costs about as much as a
// kernel boundary, the short phases stay latency-bound inside the kernel
// (route and align take 10-14 us each including their barrier), the GEMM
// phases run 15-20 % slower at the persistent kernel's occupancy, and a
// cooperative launch costs ~17 us more than a plain one.  It is kept as the
// single-launch form of the layer, bitwise equal to the other, for callers
// that need one launch.
//
// Every phase runs the same device code as the standalone kernels (dev_*.h),
// so the output is bitwise that of moe_forward on the same routing.  The
// workgroups are persistent: a cooperative launch of at most as many
// workgroups as fit on the device at once (so every barrier is reached), each
// taking the GEMM items of its XCD's contiguous range in turn (the same
// XCD-balanced split as the standalone kernels).
//
// Grid barrier: thread 0 of each workgroup releases the workgroup's writes to
// device scope (L2 write-back), arrives, and polls with device-scope atomic
// loads until every workgroup has arrived, then acquires (L2/L1 invalidate):
// the XCDs' L2s are not coherent with each other, so both fences are needed
// for data written on one XCD and read on another.  Arrival is two-level (the
// workgroups of each eighth of the grid on their own counter, the last of
// them on a global one) and the release is a generation number written to
// eight words, so no single memory line takes every arrival and every poll.
// The words live in a small caller-owned buffer that must be zero before the
// first call; the kernel leaves it zero (counters are reset by the arrival
// that completes them, the generations by the last workgroup to leave).  A
// wait is bounded by wall time (the 100 MHz real-time counter): past the bound
// the workgroup sets the error word and goes on, so the kernel always ends.
#include <algorithm>

#include "moe.h"
#include "dev_align.h"
#include "dev_combine.h"
#include "dev_gemm_mx.h"
#include "dev_gemm_small.h"
#include "dev_quant.h"
#include "dev_route.h"

namespace moe {

namespace {

constexpr int kThreads = 256;               // 4 waves, the GEMM tiles' workgroup
constexpr int kBlockM = 16;                 // rows per expert block (one 16-token MFMA tile)
constexpr uint64_t kWaitTicks = 200000000;  // 2 s of the 100 MHz real-time counter
// Barrier words, each on its own 128-byte line: per-XCD arrival counters and
// per-XCD release generations (so arrivals and polls spread over 16 lines),
// the count of XCDs arrived, and the exit counter.
constexpr int kLine = 32;                               // words per 128-byte line
constexpr int kXcdCount = 0;                            // lines 0..7
constexpr int kXcdGen = 8;                              // lines 8..15
constexpr int kGlobal = 16;
constexpr int kExit = 17;
static_assert(MOE_SYNC_ERROR >= (kExit + 1) * kLine && MOE_SYNC_ERROR < MOE_SYNC_WORDS,
              "barrier words and the error word fit the sync buffer without sharing a line");

struct FusedArgs {
    GemmArgs g;                   // the layer, block_m 16, workspace pointers
    const float* logits;          // fp32 [T, E] router logits, or null (routing given)
    int renormalize;
    int32_t* route_ids;           // route outputs when logits is set
    float* route_weights;
    const int32_t* ids;           // the routing the layer uses: [T, topk]
    int32_t* sorted;              // workspace: alignment outputs
    int32_t* expert_ids;
    int32_t* ntpp;
    int cap;
    uint8_t* xq;                  // workspace: quantised activations (fp8 paths)
    void* xs;
    uint16_t* out;
    uint32_t* sync;               // MOE_SYNC_WORDS words, zero on entry and on exit
    int ntiles1, ntiles2;         // column tiles of GEMM1 and GEMM2
};

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t add_agent(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Grid barrier number gen (1, 2, ...).  The counters only grow during a call:
// barrier gen is complete for group x (the workgroups with blockIdx % 8 == x)
// when its counter reaches gen * nwg / 8; the arrival that completes it adds
// one to the global counter, and the arrival that brings that to 8 * gen
// publishes gen to every group's generation word, which the group polls.
__device__ __forceinline__ void grid_barrier(uint32_t* sync, uint32_t gen, int nwg) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const int x = blockIdx.x & 7;
        const uint32_t per = uint32_t(nwg) / 8;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // this workgroup's writes to device scope
        if (add_agent(&sync[(kXcdCount + x) * kLine], 1u) == gen * per - 1) {
            if (add_agent(&sync[kGlobal * kLine], 1u) == 8 * gen - 1)
                for (int y = 0; y < 8; ++y)
                    __hip_atomic_store(&sync[(kXcdGen + y) * kLine], gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t* gw = &sync[(kXcdGen + x) * kLine];
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (load_agent(gw) < gen) {
            __builtin_amdgcn_s_sleep(1);
            if (__builtin_amdgcn_s_memrealtime() - t0 > kWaitTicks) {
                __hip_atomic_fetch_or(&sync[MOE_SYNC_ERROR], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // later reads see every workgroup's writes
    }
    __syncthreads();
}

// After the last barrier: the last workgroup out zeroes every barrier word
// (every workgroup has passed every barrier by then).
__device__ __forceinline__ void grid_exit(uint32_t* sync, int nwg) {
    if (threadIdx.x == 0) {
        uint32_t* ex = &sync[kExit * kLine];
        if (add_agent(ex, 1u) == uint32_t(nwg) - 1) {
            for (int w = 0; w < kExit; ++w)
                __hip_atomic_store(&sync[w * kLine], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(ex, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Workgroup wg's items of [0, total) in the XCD-balanced order of the
// standalone kernels: XCD x = wg % 8 owns [x*total/8, (x+1)*total/8), taken by
// its nwg/8 workgroups in turn.
template <typename F>
__device__ __forceinline__ void for_items(int64_t total, int wg, int nwg, F f) {
    const int xcd = wg & 7;
    const int64_t end = (xcd + 1) * total / 8;
    for (int64_t item = xcd * total / 8 + (wg >> 3); item < end; item += nwg >> 3) f(item);
}

// W: 0 bf16, 1 fp8 (128x128 block scales), 2 MXFP8.
template <int W>
__global__ __launch_bounds__(kThreads) void decode_layer_kernel(FusedArgs a) {
    const GemmArgs& g = a.g;
    const int wg = blockIdx.x, nwg = gridDim.x;
    const int wv = threadIdx.x >> 6;
    const int R = g.T * g.topk;
    uint32_t bar = 0;   // barriers passed

    // phase 0: routing from logits, activation quantisation (independent)
    if (a.logits) {
        for (int t = wg * 4 + wv; t < g.T; t += nwg * 4)
            route_token(a.logits, g.E, g.topk, a.renormalize, a.route_ids, a.route_weights, t);
    }
    if constexpr (W == 1) {   // 16 lanes per 128-column group, 16 groups per pass
        const int64_t groups = int64_t(g.T) * (g.H / kGroup);
        for (int64_t base = int64_t(wg) * (kThreads / 16); base < groups; base += int64_t(nwg) * (kThreads / 16))
            quant_group(g.x, g.T, g.H, a.xq, static_cast<float*>(a.xs), base + (threadIdx.x >> 4), threadIdx.x & 15);
    } else if constexpr (W == 2) {   // 4 lanes per 32-column group, 64 groups per pass
        const int64_t groups = int64_t(g.T) * (g.H / 32);
        for (int64_t base = int64_t(wg) * (kThreads / 4); base < groups; base += int64_t(nwg) * (kThreads / 4))
            quant_group_mx(g.x, g.T, g.H, a.xq, static_cast<uint8_t*>(a.xs), base + (threadIdx.x >> 2),
                           threadIdx.x & 3);
    }
    if (a.logits) grid_barrier(a.sync, ++bar, nwg);

    // phase 1: alignment by one wave of workgroup 0
    if (wg == 0) {
        __shared__ int cnt[kMaxE];
        __shared__ int offs[kMaxE + 1];
        align_tiny_wg(a.ids, R, g.E, kBlockM, a.cap, a.sorted, a.expert_ids, a.ntpp, nullptr, cnt, offs, wv == 0);
    }
    grid_barrier(a.sync, ++bar, nwg);

    // phase 2: GEMM1 + SiLU-mul (+ quantisation of the intermediate)
    const int active = __builtin_amdgcn_readfirstlane(a.ntpp[0]) / kBlockM;
    for_items(int64_t(active) * a.ntiles1, wg, nwg, [&](int64_t item) {
        const int tile = int(item / active), blk = int(item - int64_t(tile) * active);
        if constexpr (W == 0) small_gemm::gemm1_small_tile<false, 1, 1, 4, 4>(g, blk, tile);
        else if constexpr (W == 1) {
            if (g.krot) small_gemm::gemm1_small_tile<true, 1, 2, 4, 1, true>(g, blk, tile);
            else small_gemm::gemm1_small_tile<true, 1, 2, 4, 1>(g, blk, tile);
        }
        else mx_gemm::gemm1_mx_tile<1, 2, 4>(g, blk, tile);
    });
    grid_barrier(a.sync, ++bar, nwg);

    // phase 3: GEMM2 with the router weight
    for_items(int64_t(active) * a.ntiles2, wg, nwg, [&](int64_t item) {
        const int tile = int(item / active), blk = int(item - int64_t(tile) * active);
        if constexpr (W == 0) small_gemm::gemm2_small_tile<false, 1, 2, 4, 4>(g, blk, tile);
        else if constexpr (W == 1) small_gemm::gemm2_small_tile<true, 1, 4, 4, 1>(g, blk, tile);
        else mx_gemm::gemm2_mx_tile<1, 4, 4>(g, blk, tile);
    });
    grid_barrier(a.sync, ++bar, nwg);

    // phase 4: top-k combine, 8 outputs per thread
    const int per_row = g.H / 8;
    for (int64_t i = int64_t(wg) * kThreads + threadIdx.x; i < int64_t(g.T) * per_row;
         i += int64_t(nwg) * kThreads) {
        const int t = int(i / per_row);
        combine_chunk<(W > 0)>(g.y, a.ids, g.topk, g.E, g.H, a.out, t, int(i - int64_t(t) * per_row) * 8);
    }
    grid_exit(a.sync, nwg);
}

template <int W>
hipError_t launch_w(const FusedArgs& a, hipStream_t s) {
    int dev = 0, cus = 0, coop = 0, per_cu = 0;
    hipError_t e;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev)) != hipSuccess) return e;
    if (!coop) return hipErrorNotSupported;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_layer_kernel<W>, kThreads, 0)) !=
        hipSuccess)
        return e;
    // every workgroup resident at once; a multiple of 8 (the XCD split), no
    // more than the largest phase has items for
    // (an expert block holds at least one routed slot: at most T * topk blocks)
    const int64_t blocks = std::min<int64_t>((a.cap + kBlockM - 1) / kBlockM, int64_t(a.g.T) * a.g.topk);
    const int64_t most = std::max<int64_t>(blocks * std::max(a.ntiles1, a.ntiles2), 8);
    int nwg = int(std::min<int64_t>(int64_t(cus) * per_cu, (most + 7) / 8 * 8));
    nwg = nwg / 8 * 8;
    if (nwg < 8) return hipErrorNotSupported;
    FusedArgs arg = a;
    void* params[] = {&arg};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(decode_layer_kernel<W>), dim3(nwg),
                                      dim3(kThreads), params, 0, s);
}

}  // namespace

bool decode_layer_supported(int T, int topk, int H, int I, int block_m) {
    return block_m == kBlockM && int64_t(T) * topk <= kTinyMaxSlots && H % 256 == 0 && I % 128 == 0;
}

hipError_t launch_decode_layer(const GemmArgs& g, int wdtype_fp8, int mx, const float* logits, int renormalize,
                               int32_t* route_ids, float* route_weights, const int32_t* ids, int32_t* sorted,
                               int32_t* expert_ids, int32_t* ntpp, int cap, uint8_t* xq, void* xs, uint16_t* out,
                               uint32_t* sync, hipStream_t s) {
    FusedArgs a;
    a.g = g;
    a.logits = logits;
    a.renormalize = renormalize;
    a.route_ids = route_ids;
    a.route_weights = route_weights;
    a.ids = ids;
    a.sorted = sorted;
    a.expert_ids = expert_ids;
    a.ntpp = ntpp;
    a.cap = cap;
    a.xq = xq;
    a.xs = xs;
    a.out = out;
    a.sync = sync;
    if (mx) {
        a.ntiles1 = g.I / 128;   // 4 waves x (32 gate + 32 up) rows
        a.ntiles2 = g.H / 256;
        return launch_w<2>(a, s);
    }
    if (wdtype_fp8) {
        a.ntiles1 = g.I / 128;
        a.ntiles2 = g.H / 256;
        return launch_w<1>(a, s);
    }
    a.ntiles1 = g.I / 64;        // 4 waves x (16 gate + 16 up) rows
    a.ntiles2 = g.H / 128;
    return launch_w<0>(a, s);
}

}  // namespace moe
