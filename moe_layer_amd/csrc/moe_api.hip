// C ABI of libmoe_mi355x: argument validation, planning and the launch
// sequence of the fused MoE layer.  Declarations, argument meaning and error
// behaviour are documented in include/moe.h.
#include "moe.h"

#include <algorithm>
#include <climits>
#include <cstddef>
#include <mutex>

#include "common.h"

using namespace moe;

namespace {

constexpr int kVersionMajor = 1;
constexpr int kVersionMinor = 6;   // 1.1: MXFP8 weights; 1.2: layer variants; 1.3: moe_decode_layer;
                                   // 1.4: packed MXFP8 scales (moe_pack_mx_scales);
                                   // 1.5: multi-workgroup alignment (moe_align_ws);
                                   // 1.6: moe_forward_noalloc
// Rows per expert (on average) from which the LDS-tiled path beats weight
// streaming.  Measured with bf16 weights (align + GEMM1 + GEMM2): E 128, H
// 4096, I 1536 at 8 rows 0.90 ms streaming vs 1.08 tiled, 16 rows 1.14 vs 1.09,
// 32 rows 1.49 vs 1.11; E 256, H 7168, I 2048 at 16 rows 5.3 vs 4.9 ms.  The
// tiled path skips a block's padding-only 32-token sub-tiles, so its 256-row
// blocks cost little when an expert has few rows.  It also needs enough
// GEMM1 workgroups (one per expert and 128 intermediate columns) to cover the
// CUs: on a layer as small as 8 experts, H 256, I 512 (16 rows per expert) the
// tiled path's 32 workgroups took 0.037 ms against streaming's 0.025.
constexpr double kLargeMinRowsPerExpert = 12.0;
// fp8 and MXFP8 weights take their LDS-tiled path from this many rows per
// expert (E 256, H 4096, I 256, layer ms, weight streaming vs tiled: fp8 at
// 8 rows 0.196 vs 0.229, 16 rows 0.250 vs 0.257, 24 rows 0.297 vs 0.286, 32
// rows 0.317 vs 0.305, 256 rows 1.77 vs 1.16; MXFP8 0.200 vs 0.240, 0.259 vs
// 0.260, 0.283 vs 0.287, 0.323 vs 0.305, 1.78 vs 1.15)
constexpr double kLargeQMinRowsPerExpert = 20.0;
constexpr double kLargeMxMinRowsPerExpert = 28.0;
constexpr int64_t kLargeMinGemm1Tiles = 256;
// Above 8192 routed slots the alignment runs on many workgroups (one
// workgroup's ALUs bound it beyond; align stage us, one workgroup vs many:
// 2048 slots 14.6 vs 24.3, 4096 14.8 vs 23.8, 8192 21.9 vs 25.5, 16384 35.3
// vs 27.0, 32768 63 vs 27).
constexpr int64_t kAlignWideMinSlots = 8193;
// The fp8 GEMM1 walks K from a per-(expert, tile) start up to this many
// routed rows per expert (k_rotation; fp8 layer: 64 tokens 127 -> 94 us, 256
// tokens 154 -> 109 us, 512 tokens 143 -> 138 us; the MXFP8 GEMM1 always does).
constexpr int64_t kRotateMaxRowsPerExpert = 16;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

// Planner: rows per expert decide the block size and the tile path.
struct Plan {
    int path;
    int block_m;
    int64_t cap;
    int num_blocks;
    int gemm1_cols, gemm2_cols;
    int64_t off_sorted, off_eids, off_ntpp, off_xq, off_xs, off_inter, off_inter_scale, off_y, total;
};

int validate_forward_scalars(const moe_forward_args* a) {
    if (!a) return MOE_ERR_INVALID_ARG;
    if (a->T < 0 || a->E < 1 || a->E > MOE_MAX_EXPERTS || a->topk < 1 || a->topk > MOE_MAX_TOPK ||
        a->H <= 0 || a->I <= 0)
        return MOE_ERR_INVALID_ARG;
    if (a->wdtype != MOE_WDTYPE_BF16 && a->wdtype != MOE_WDTYPE_FP8_E4M3 && a->wdtype != MOE_WDTYPE_MXFP8)
        return MOE_ERR_INVALID_ARG;
    if (a->path < MOE_PATH_AUTO || a->path > MOE_PATH_LARGE_M) return MOE_ERR_INVALID_ARG;
    if ((a->flags & ~(MOE_FLAG_WEIGHT_ON_INPUT | MOE_FLAG_MX_PACKED_SCALES)) != 0) return MOE_ERR_INVALID_ARG;
    if ((a->flags & MOE_FLAG_MX_PACKED_SCALES) && a->wdtype != MOE_WDTYPE_MXFP8) return MOE_ERR_INVALID_ARG;
    if (!(a->clamp_limit >= 0.0f)) return MOE_ERR_INVALID_ARG;   // negative or NaN
    if (a->block_m != 0 && a->block_m != 16 && a->block_m != 32 && a->block_m != 64 && a->block_m != 128 &&
        a->block_m != 256)
        return MOE_ERR_UNSUPPORTED;
    const int q = a->wdtype == MOE_WDTYPE_BF16 ? 64 : MOE_QUANT_GROUP;
    if (a->H % q != 0 || a->I % q != 0) return MOE_ERR_UNSUPPORTED;
    if (int64_t(a->T) * a->topk > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    // the MXFP8 kernels address the quantised activations with 32-bit offsets
    if (a->wdtype == MOE_WDTYPE_MXFP8 && int64_t(a->T) * a->H >= (int64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int make_plan(const moe_forward_args* a, Plan* p) {
    int st = validate_forward_scalars(a);
    if (st != MOE_OK) return st;
    const int64_t R = int64_t(a->T) * a->topk;
    const bool fp8 = a->wdtype != MOE_WDTYPE_BF16;          // block-scaled fp8 or MXFP8
    const bool mx = a->wdtype == MOE_WDTYPE_MXFP8;
    const double rows_per_expert = double(R) / a->E;
    const bool large_ok = fp8 ? gemm_large_q_supported(a->H, a->I) : gemm_large_supported(a->H, a->I, false);
    const int large_bm = fp8 ? gemm_large_q_block_m() : gemm_large_block_m();
    int path = a->path;
    // AUTO with an explicit block size of the weight-streaming path stays on it
    const bool bm_ok = a->block_m == 0 || a->block_m == large_bm;
    const bool wide = std::min<int64_t>(a->E, R) * (a->I / 128) >= kLargeMinGemm1Tiles;
    const double min_rows = !fp8 ? kLargeMinRowsPerExpert
                            : a->wdtype == MOE_WDTYPE_MXFP8 ? kLargeMxMinRowsPerExpert : kLargeQMinRowsPerExpert;
    if (path == MOE_PATH_AUTO)
        path = (large_ok && bm_ok && wide && rows_per_expert >= min_rows) ? MOE_PATH_LARGE_M : MOE_PATH_SMALL_M;
    int bm = a->block_m;
    if (path == MOE_PATH_LARGE_M) {
        if (!large_ok) return MOE_ERR_UNSUPPORTED;
        if (bm == 0) bm = large_bm;
        if (bm != large_bm) return MOE_ERR_UNSUPPORTED;
    } else {
        if (bm == 0) bm = rows_per_expert <= 16.0 ? 16 : rows_per_expert <= 32.0 ? 32 : 64;
        if (bm > 64) return MOE_ERR_UNSUPPORTED;
    }
    p->path = path;
    p->block_m = bm;
    p->cap = R + int64_t(a->E) * (bm - 1);
    if (p->cap > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    p->num_blocks = int((p->cap + bm - 1) / bm);
    if (path == MOE_PATH_LARGE_M) {
        p->gemm1_cols = 256;   // 128 gate + 128 up rows
        p->gemm2_cols = 256;
    } else {
        p->gemm1_cols = fp8 ? 256 : 128;   // gate + up rows per workgroup
        p->gemm2_cols = small_gemm2_cols(a->T, a->topk, a->E, a->H, a->I, fp8, bm / 16, mx);
    }

    const int64_t rows = int64_t(p->num_blocks) * bm;   // every row a block can touch
    const int64_t es = fp8 ? 1 : 2;
    int64_t off = 0;
    auto take = [&](int64_t bytes) { const int64_t o = off; off = round_up(off + bytes, 256); return o; };
    p->off_sorted = take(p->cap * 4);
    p->off_eids = take(int64_t(p->num_blocks) * 4);
    p->off_ntpp = take(4);
    p->off_xq = fp8 ? take(int64_t(a->T) * a->H) : -1;
    p->off_xs = mx ? take(int64_t(a->T) * (a->H / MOE_MX_BLOCK)) : fp8 ? take(int64_t(a->T) * (a->H / MOE_QUANT_GROUP) * 4) : -1;
    p->off_inter = take(rows * a->I * es);
    p->off_inter_scale = mx    ? take(rows * (a->I / MOE_MX_BLOCK))
                         : fp8 ? take(rows * (a->I / MOE_QUANT_GROUP) * 4)
                               : -1;
    // y (fp32, or bf16 for fp8 and MXFP8 weights) also serves as the wide
    // alignment's scratch (used before GEMM2 writes y)
    p->off_y = take(std::max(R * a->H * (fp8 ? 2 : 4), align_scratch_bytes(R, a->E)));
    p->total = off;
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The GEMM kernels' arguments for a validated plan and workspace.
GemmArgs gemm_args(const moe_forward_args* a, const Plan& p, uint8_t* ws) {
    const bool fp8 = a->wdtype != MOE_WDTYPE_BF16;
    GemmArgs g{};
    g.T = a->T;
    g.E = a->E;
    g.H = a->H;
    g.I = a->I;
    g.topk = a->topk;
    g.block_m = p.block_m;
    g.num_blocks = p.num_blocks;
    g.x = static_cast<const uint16_t*>(a->x);
    g.xq = fp8 ? ws + p.off_xq : nullptr;
    g.xs = fp8 ? reinterpret_cast<const float*>(ws + p.off_xs) : nullptr;
    g.w13 = a->w13;
    g.w13_scale = a->w13_scale;
    g.w2 = a->w2;
    g.w2_scale = a->w2_scale;
    g.topk_weights = a->topk_weights;
    g.sorted_ids = reinterpret_cast<const int32_t*>(ws + p.off_sorted);
    g.expert_ids = reinterpret_cast<const int32_t*>(ws + p.off_eids);
    g.ntpp = reinterpret_cast<const int32_t*>(ws + p.off_ntpp);
    g.inter = ws + p.off_inter;
    g.inter_scale = fp8 ? reinterpret_cast<float*>(ws + p.off_inter_scale) : nullptr;
    g.y = reinterpret_cast<float*>(ws + p.off_y);
    g.weight_on_input = (a->flags & MOE_FLAG_WEIGHT_ON_INPUT) != 0;
    g.mx_packed = (a->flags & MOE_FLAG_MX_PACKED_SCALES) != 0;
    // the fp8 GEMM1's rotated K walk: on while experts hold about one block each
    g.krot = int64_t(a->T) * a->topk <= kRotateMaxRowsPerExpert * int64_t(a->E);
    g.clamp = a->clamp_limit > 0.0f;
    g.clamp_limit = a->clamp_limit;
    return g;
}

}  // namespace

extern "C" {

MOE_API const char* moe_status_string(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or option";
        case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
        case MOE_ERR_HIP: return "HIP launch failure";
        default: return "unknown status";
    }
}

MOE_API int moe_version(void) { return (kVersionMajor << 16) | kVersionMinor; }

MOE_API int moe_route(const float* logits, int32_t T, int32_t E, int32_t topk, int32_t renormalize,
                      int32_t* topk_ids, float* topk_weights, hipStream_t stream) {
    if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || topk < 1 || topk > E || topk > MOE_MAX_TOPK)
        return MOE_ERR_INVALID_ARG;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_weights || !aligned(logits, 4) || !aligned(topk_ids, 4) ||
        !aligned(topk_weights, 4))
        return MOE_ERR_INVALID_ARG;
    return hip_status(launch_route(logits, T, E, topk, renormalize, topk_ids, topk_weights, stream));
}

MOE_API int64_t moe_align_capacity(int32_t T, int32_t topk, int32_t E, int32_t block_m) {
    if (T < 0 || topk < 1 || topk > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS || block_m < 1 ||
        block_m > 1024)
        return MOE_ERR_INVALID_ARG;
    const int64_t cap = int64_t(T) * topk + int64_t(E) * (block_m - 1);
    if (cap > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return cap;
}

MOE_API int moe_align(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E, int32_t block_m,
                      int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                      int32_t* inv, hipStream_t stream) {
    const int64_t cap = moe_align_capacity(T, topk, E, block_m);
    if (cap < 0) return int(cap);
    if (!sorted_token_ids || !expert_ids || !num_tokens_post_padded || !aligned(sorted_token_ids, 4) ||
        !aligned(expert_ids, 4) || !aligned(num_tokens_post_padded, 4) || (inv && !aligned(inv, 4)))
        return MOE_ERR_INVALID_ARG;
    if (T > 0 && (!topk_ids || !aligned(topk_ids, 4))) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_align(topk_ids, T, topk, E, block_m, cap, sorted_token_ids, expert_ids,
                                   num_tokens_post_padded, inv, stream));
}

MOE_API int64_t moe_align_scratch_bytes(int32_t T, int32_t topk, int32_t E) {
    if (T < 0 || topk < 1 || topk > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_INVALID_ARG;
    const int64_t R = int64_t(T) * topk;
    if (R > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    return R >= kAlignWideMinSlots ? round_up(align_scratch_bytes(R, E), 256) : 0;
}

MOE_API int moe_align_ws(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E, int32_t block_m,
                         int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         int32_t* inv, void* scratch, int64_t scratch_bytes, hipStream_t stream) {
    const int64_t cap = moe_align_capacity(T, topk, E, block_m);
    if (cap < 0) return int(cap);
    const int64_t need = moe_align_scratch_bytes(T, topk, E);
    if (need < 0) return int(need);
    if (need == 0)
        return moe_align(topk_ids, T, topk, E, block_m, sorted_token_ids, expert_ids, num_tokens_post_padded, inv,
                         stream);
    if (!sorted_token_ids || !expert_ids || !num_tokens_post_padded || !aligned(sorted_token_ids, 4) ||
        !aligned(expert_ids, 4) || !aligned(num_tokens_post_padded, 4) || (inv && !aligned(inv, 4)) ||
        !topk_ids || !aligned(topk_ids, 4))
        return MOE_ERR_INVALID_ARG;
    if (!scratch || !aligned(scratch, 4) || scratch_bytes < need) return MOE_ERR_WORKSPACE;
    return hip_status(launch_align_wide(topk_ids, T, topk, E, block_m, cap, sorted_token_ids, expert_ids,
                                        num_tokens_post_padded, inv, scratch, stream));
}

MOE_API int moe_quant_act(const void* x, int32_t rows, int32_t cols, uint8_t* codes, float* scales,
                          hipStream_t stream) {
    if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
    if (cols % MOE_QUANT_GROUP != 0) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4))
        return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_act(static_cast<const uint16_t*>(x), rows, cols, codes, scales, stream));
}

MOE_API int moe_quant_act_mx(const void* x, int32_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                             hipStream_t stream) {
    if (rows < 0 || cols <= 0) return MOE_ERR_INVALID_ARG;
    if (cols % MOE_MX_BLOCK != 0) return MOE_ERR_UNSUPPORTED;
    if (rows == 0) return MOE_OK;
    if (!x || !codes || !scales || !aligned(x, 16) || !aligned(codes, 8) || !aligned(scales, 4))
        return MOE_ERR_INVALID_ARG;
    return hip_status(launch_quant_act_mx(static_cast<const uint16_t*>(x), rows, cols, codes, scales, stream));
}

MOE_API int moe_pack_mx_scales(const uint8_t* scales, int32_t E, int32_t rows, int32_t K, uint8_t* packed,
                               hipStream_t stream) {
    if (E < 0 || rows < 0 || K < 0) return MOE_ERR_INVALID_ARG;
    if (E < 1 || rows % 16 != 0 || K % 128 != 0) return MOE_ERR_UNSUPPORTED;
    const int64_t bytes = int64_t(E) * rows * (K / MOE_MX_BLOCK);
    if (bytes == 0) return MOE_OK;
    if (!scales || !packed) return MOE_ERR_INVALID_ARG;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(scales), b0 = reinterpret_cast<uintptr_t>(packed);
    if (a0 < b0 + uintptr_t(bytes) && b0 < a0 + uintptr_t(bytes)) return MOE_ERR_INVALID_ARG;   // overlap
    return hip_status(launch_pack_mx_scales(scales, E, rows, K, packed, stream));
}

MOE_API int moe_plan(const moe_forward_args* a, moe_plan_info* out) {
    if (!out) return MOE_ERR_INVALID_ARG;
    Plan p;
    const int st = make_plan(a, &p);
    if (st != MOE_OK) return st;
    out->path = p.path;
    out->block_m = p.block_m;
    out->capacity = p.cap;
    out->num_blocks = p.num_blocks;
    out->gemm1_cols = p.gemm1_cols;
    out->gemm2_cols = p.gemm2_cols;
    out->decode_layer = p.path == MOE_PATH_SMALL_M && decode_layer_supported(a->T, a->topk, a->H, a->I, p.block_m);
    out->workspace_bytes = p.total;
    out->off_sorted_ids = p.off_sorted;
    out->off_expert_ids = p.off_eids;
    out->off_num_post_padded = p.off_ntpp;
    out->off_xq = p.off_xq;
    out->off_xs = p.off_xs;
    out->off_inter = p.off_inter;
    out->off_inter_scale = p.off_inter_scale;
    out->off_y = p.off_y;
    return MOE_OK;
}

MOE_API int64_t moe_forward_workspace(const moe_forward_args* a) {
    Plan p;
    const int st = make_plan(a, &p);
    return st != MOE_OK ? int64_t(st) : p.total;
}

}  // extern "C"

namespace {

int run_forward(const moe_forward_args* a, void* workspace, int64_t workspace_bytes, hipStream_t stream,
                hipEvent_t* ev) {
    Plan p;
    int st = make_plan(a, &p);
    if (st != MOE_OK) return st;
    if (a->T == 0) return MOE_OK;
    const bool fp8 = a->wdtype != MOE_WDTYPE_BF16;          // block-scaled fp8 or MXFP8
    const bool mx = a->wdtype == MOE_WDTYPE_MXFP8;
    if (!a->x || !a->w13 || !a->w2 || !a->topk_ids || !a->topk_weights || !a->out ||
        !aligned(a->x, 16) || !aligned(a->w13, 16) || !aligned(a->w2, 16) || !aligned(a->out, 16) ||
        !aligned(a->topk_ids, 4) || !aligned(a->topk_weights, 4))
        return MOE_ERR_INVALID_ARG;
    if (fp8 && (!a->w13_scale || !a->w2_scale || !aligned(a->w13_scale, 4) || !aligned(a->w2_scale, 4)))
        return MOE_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    GemmArgs g = gemm_args(a, p, ws);
    auto mark = [&](int i) { return ev ? hip_status(hipEventRecord(ev[i], stream)) : MOE_OK; };
    if ((st = mark(0)) != MOE_OK) return st;
    int32_t* sorted = reinterpret_cast<int32_t*>(ws + p.off_sorted);
    int32_t* eids = reinterpret_cast<int32_t*>(ws + p.off_eids);
    int32_t* ntpp = reinterpret_cast<int32_t*>(ws + p.off_ntpp);
    const bool wide = int64_t(a->T) * a->topk >= kAlignWideMinSlots;
    // fp8 and MXFP8 with the one-workgroup alignment: the quantisation of x
    // runs in the same launch on the other CUs (its stage time is then 0)
    const bool joint = fp8 && !wide;
    const hipError_t ae =
        wide    ? launch_align_wide(a->topk_ids, a->T, a->topk, a->E, p.block_m, p.cap, sorted, eids, ntpp, nullptr,
                                    ws + p.off_y, stream)
        : joint ? launch_align_quant(a->topk_ids, a->T, a->topk, a->E, p.block_m, p.cap, sorted, eids, ntpp, g.x,
                                     a->H, ws + p.off_xq, ws + p.off_xs, mx, stream)
                : launch_align(a->topk_ids, a->T, a->topk, a->E, p.block_m, p.cap, sorted, eids, ntpp, nullptr,
                               stream);
    if ((st = hip_status(ae)) != MOE_OK) return st;
    if ((st = mark(1)) != MOE_OK) return st;
    if (fp8 && !joint) {
        const hipError_t qe = mx ? launch_quant_act_mx(g.x, a->T, a->H, ws + p.off_xq, ws + p.off_xs, stream)
                                 : launch_quant_act(g.x, a->T, a->H, ws + p.off_xq,
                                                    reinterpret_cast<float*>(ws + p.off_xs), stream);
        if ((st = hip_status(qe)) != MOE_OK) return st;
    }
    if ((st = mark(2)) != MOE_OK) return st;
    const bool large = p.path == MOE_PATH_LARGE_M;
    const hipError_t g1 = large ? (fp8 ? launch_gemm1_large_q(g, mx, stream) : launch_gemm1_large(g, false, stream))
                          : mx  ? launch_gemm1_mx(g, stream)
                                : launch_gemm1_small(g, fp8, stream);
    if ((st = hip_status(g1)) != MOE_OK) return st;
    if ((st = mark(3)) != MOE_OK) return st;
    const hipError_t g2 = large ? (fp8 ? launch_gemm2_large_q(g, mx, stream) : launch_gemm2_large(g, false, stream))
                          : mx  ? launch_gemm2_mx(g, stream)
                                : launch_gemm2_small(g, fp8, stream);
    if ((st = hip_status(g2)) != MOE_OK) return st;
    if ((st = mark(4)) != MOE_OK) return st;
    if ((st = hip_status(launch_combine(g.y, fp8, a->topk_ids, a->T, a->topk, a->E, a->H,
                                        static_cast<uint16_t*>(a->out), stream))) != MOE_OK)
        return st;
    return mark(5);
}

}  // namespace

extern "C" {

MOE_API int moe_forward(const moe_forward_args* a, void* workspace, int64_t workspace_bytes,
                        hipStream_t stream) {
    return run_forward(a, workspace, workspace_bytes, stream, nullptr);
}

MOE_API int moe_forward_profiled(const moe_forward_args* a, void* workspace, int64_t workspace_bytes,
                                 hipStream_t stream, hipEvent_t* events, int32_t n_events) {
    if (!events || n_events < MOE_NUM_STAGES + 1) return MOE_ERR_INVALID_ARG;
    return run_forward(a, workspace, workspace_bytes, stream, events);
}

MOE_API int moe_decode_layer(const moe_forward_args* a, const float* router_logits, int32_t renormalize,
                             int32_t* topk_ids_out, float* topk_weights_out, uint32_t* sync, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
    Plan p;
    int st = make_plan(a, &p);
    if (st != MOE_OK) return st;
    if (p.path != MOE_PATH_SMALL_M || !decode_layer_supported(a->T, a->topk, a->H, a->I, p.block_m))
        return MOE_ERR_UNSUPPORTED;
    if (a->T == 0) return MOE_OK;
    const bool fp8 = a->wdtype != MOE_WDTYPE_BF16;
    const bool mx = a->wdtype == MOE_WDTYPE_MXFP8;
    if (router_logits) {
        if (a->topk > a->E || !aligned(router_logits, 4) || !topk_ids_out || !topk_weights_out ||
            !aligned(topk_ids_out, 4) || !aligned(topk_weights_out, 4))
            return MOE_ERR_INVALID_ARG;
    } else if (!a->topk_ids || !a->topk_weights || !aligned(a->topk_ids, 4) || !aligned(a->topk_weights, 4)) {
        return MOE_ERR_INVALID_ARG;
    }
    if (!a->x || !a->w13 || !a->w2 || !a->out || !aligned(a->x, 16) || !aligned(a->w13, 16) ||
        !aligned(a->w2, 16) || !aligned(a->out, 16) || !sync || !aligned(sync, 4))
        return MOE_ERR_INVALID_ARG;
    if (fp8 && (!a->w13_scale || !a->w2_scale || !aligned(a->w13_scale, 4) || !aligned(a->w2_scale, 4)))
        return MOE_ERR_INVALID_ARG;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;

    uint8_t* ws = static_cast<uint8_t*>(workspace);
    GemmArgs g = gemm_args(a, p, ws);
    const int32_t* ids = router_logits ? topk_ids_out : a->topk_ids;
    if (router_logits) g.topk_weights = topk_weights_out;
    return hip_status(launch_decode_layer(
        g, fp8, mx, router_logits, renormalize, topk_ids_out, topk_weights_out, ids,
        reinterpret_cast<int32_t*>(ws + p.off_sorted), reinterpret_cast<int32_t*>(ws + p.off_eids),
        reinterpret_cast<int32_t*>(ws + p.off_ntpp), int(p.cap), fp8 ? ws + p.off_xq : nullptr,
        fp8 ? static_cast<void*>(ws + p.off_xs) : nullptr, static_cast<uint16_t*>(a->out), sync, stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// moe_forward_noalloc: moe_forward with its workspace in a static device
// array of MOE_NOALLOC_MAX_BYTES that the library holds on every GPU it runs
// on, for callers that cannot allocate device memory.  Host code never passes
// the array's name to a kernel or a copy: in host code that name is a host
// stand-in, not the device address.  The device address is looked up once per
// device with hipGetSymbolAddress and used from then on.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's copy of the scratch array (nullptr on failure).
void* scratch_for_current_device(int* status) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = MOE_ERR_HIP;
        return nullptr;
    }
    std::call_once(g_scratch_once[dev], [dev] {
        void* ptr = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        *status = MOE_ERR_HIP;
        return nullptr;
    }
    *status = MOE_OK;
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" MOE_API int moe_forward_noalloc(const moe_forward_args* a, hipStream_t stream) {
    Plan p;
    int st = make_plan(a, &p);
    if (st != MOE_OK) return st;
    if (p.total > MOE_NOALLOC_MAX_BYTES) return MOE_ERR_WORKSPACE;   // beyond the static array
    if (a->T == 0) return MOE_OK;
    void* ws = scratch_for_current_device(&st);
    if (!ws) return st;
    return run_forward(a, ws, MOE_NOALLOC_MAX_BYTES, stream, nullptr);
}
