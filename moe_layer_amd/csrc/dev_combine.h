// Router-weighted top-k combine (the "expert aggregation" step of P1, section
// "Backend-Wechsel für FP8-Modelle"): out[t] = bf16( sum_j y[t*topk + j] ),
// summed in fp32 in slot order j = 0..topk-1; slots whose id is outside
// [0, E) were not routed and are skipped.  The down GEMM already applied the
// router weight and wrote y by flat slot (fp32, or bf16 for fp8 and MXFP8
// weights), so the k rows of a token are contiguous and every access here is
// a coalesced 16-byte vector.  HBM-bound: topk*H*4 (bf16 y: topk*H*2) bytes
// read and H*2 written per token.
//
// Device code shared by combine.hip and the single-launch decode layer in
// fused.hip.
#pragma once

#include "common.h"

namespace moe {

namespace {

// Output columns h .. h+7 of token t by one thread.
template <bool kBf16Y>
__device__ __forceinline__ void combine_chunk(const float* __restrict__ y, const int32_t* __restrict__ ids,
                                              int topk, int E, int H, uint16_t* __restrict__ out, int t, int h) {
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // slots in groups of 8: the ids first, then every y load of the group at
    // once (an unrouted slot's row is loaded from slot 0's and added as +0.0,
    // which leaves the sum unchanged bit for bit: it starts at +0.0, so no
    // partial sum is -0.0)
    for (int j0 = 0; j0 < topk; j0 += 8) {
        bool ok[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const int e = j < topk ? ids[int64_t(t) * topk + j] : -1;
            ok[u] = e >= 0 && e < E;
        }
        f32x4 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int64_t idx = (int64_t(t) * topk + (ok[u] ? j0 + u : 0)) * H + h;
            if constexpr (kBf16Y) {
                const i32x4 r = *reinterpret_cast<const i32x4*>(reinterpret_cast<const uint16_t*>(y) + idx);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    a[u][2 * q] = __uint_as_float(uint32_t(r[q]) << 16);
                    a[u][2 * q + 1] = __uint_as_float(uint32_t(r[q]) & 0xffff0000u);
                    b[u][2 * q] = __uint_as_float(uint32_t(r[2 + q]) << 16);
                    b[u][2 * q + 1] = __uint_as_float(uint32_t(r[2 + q]) & 0xffff0000u);
                }
            } else {
                a[u] = *reinterpret_cast<const f32x4*>(y + idx);
                b[u] = *reinterpret_cast<const f32x4*>(y + idx + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[q] = __fadd_rn(acc[q], ok[u] ? a[u][q] : 0.0f);
                acc[4 + q] = __fadd_rn(acc[4 + q], ok[u] ? b[u][q] : 0.0f);
            }
    }
    i32x4 packed;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        packed[q] = int(uint32_t(f32_to_bf16_rne(acc[2 * q])) | (uint32_t(f32_to_bf16_rne(acc[2 * q + 1])) << 16));
    *reinterpret_cast<i32x4*>(out + int64_t(t) * H + h) = packed;
}

}  // namespace

}  // namespace moe
