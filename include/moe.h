/*
 * moe.h — C ABI of libmoe_mi355x.so, a fused Mixture-of-Experts layer for
 * AMD MI355X (CDNA4, gfx950).
 *
 * The layer follows the fused-MoE pipeline described in
 *   [P1] kinachrichten.com, "AWS erklärt zwei Kernel-Optimierungen, die den
 *        Durchsatz von SageMaker AI auf H200 steigern" (sections "Warum
 *        MoE-Kernel so wichtig sind", "Swap-AB", "Backend-Wechsel für
 *        FP8-Modelle"), and
 *   [P2] blog.secrett2633.cloud, analysis of vLLM PR #64760 "sorted-A TMA
 *        for FP8 MoE" (section 1.1: the sorted-A path and its block-fp8
 *        test; section 1.2: the fused SiLU-mul-FP8-quant kernel).
 *
 * Conventions shared by every entry point
 *   - All tensors are dense and row-major.  Device pointers must be 16-byte
 *     aligned.  bf16 tensors are passed as raw 16-bit words, fp8 tensors as
 *     raw OCP E4M3FN bytes (max 448, no infinities).
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     retains a pointer, keeps no state between calls and may be called from
 *     several host threads at once.
 *   - All device work is enqueued on the caller's stream, in order; nothing
 *     synchronises the host.  Results are valid once the stream reaches them.
 *     Calls that share a workspace or output buffer must be ordered by the
 *     caller (same stream, or events).
 *   - Every entry point validates its arguments on the host before enqueuing
 *     any work and returns a status; on an error nothing is enqueued, except
 *     MOE_ERR_HIP, which reports a failed launch.  T == 0 is a valid no-op.
 *   - Expert ids outside [0, E) are "not routed": they take no row, contribute
 *     nothing to the output, and their inverse-permutation entry is -1 (the
 *     expert_map convention of P2 section 1.1).  Duplicate ids within a token
 *     are allowed and each slot counts.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

/* status codes */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1)  /* null/misaligned pointer, negative size, topk out of range ... */
#define MOE_ERR_UNSUPPORTED (-2)  /* valid request outside what the kernels implement (see limits) */
#define MOE_ERR_WORKSPACE   (-3)  /* workspace smaller than moe_forward_workspace() */
#define MOE_ERR_HIP         (-4)  /* a kernel launch failed */

/* weight element types */
#define MOE_WDTYPE_BF16      0   /* w13/w2 are bf16 */
#define MOE_WDTYPE_FP8_E4M3  1   /* w13/w2 are E4M3FN with 128x128 fp32 block scales */
#define MOE_WDTYPE_MXFP8     2   /* w13/w2 are E4M3FN with one E8M0 scale per row and
                                    32 consecutive K elements (MXFP8) */

/* GEMM tile path (moe_forward_args.path) */
#define MOE_PATH_AUTO        0   /* the planner decides from rows per expert */
#define MOE_PATH_SMALL_M     1   /* weight-streaming path: few rows per expert (decode) */
#define MOE_PATH_LARGE_M     2   /* LDS-tiled path: many rows per expert (prefill) */

/* layer variants and operand layouts (moe_forward_args.flags) */
#define MOE_FLAG_WEIGHT_ON_INPUT 1   /* router weight on GEMM1's input, none after GEMM2 */
#define MOE_FLAG_MX_PACKED_SCALES 2  /* MXFP8 only: w13_scale and w2_scale are in the
                                        layout moe_pack_mx_scales writes */

/* limits */
#define MOE_MAX_EXPERTS      1024
#define MOE_MAX_TOPK         64
#define MOE_QUANT_GROUP      128  /* fp8 activation group and weight block edge */
#define MOE_MX_BLOCK         32   /* MXFP8 block: elements sharing one E8M0 scale */

/* Human-readable name of a status code (static storage, never NULL). */
MOE_API const char* moe_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
MOE_API int moe_version(void);

/*
 * moe_route — router softmax with top-k and renormalised weights.
 *
 * P2 section 1.1: the layer receives topk_ids / topk_weights from the router,
 * and its block-fp8 test builds the weights with a softmax over the selected
 * experts.  For each token t the k largest logits are selected (a tie goes to
 * the lower expert index; ids are written in descending-logit order), and
 *   renormalize != 0: w_j = exp(l_j - l_max) / sum over the k selected
 *                     (softmax -> top-k -> renormalise; the full softmax
 *                     denominator cancels)
 *   renormalize == 0: w_j = exp(l_j - l_max) / sum over all E experts
 * computed in fp32.  Selection compares the fp32 logits exactly.
 *
 *   logits        device, fp32 [T, E]   (finite values; NaN gives an
 *                                        unspecified selection)
 *   topk_ids      device, int32 [T, topk]  (output)
 *   topk_weights  device, fp32  [T, topk]  (output)
 * Requires 1 <= E <= MOE_MAX_EXPERTS, 1 <= topk <= min(E, MOE_MAX_TOPK).
 */
MOE_API int moe_route(const float* logits, int32_t T, int32_t E, int32_t topk,
                      int32_t renormalize, int32_t* topk_ids, float* topk_weights,
                      hipStream_t stream);

/*
 * moe_align_capacity — length of sorted_token_ids for moe_align:
 * T*topk + E*(block_m - 1), the padded row count when every expert wastes
 * block_m - 1 rows.  Host only.  Returns a negative status on invalid
 * arguments or when the capacity exceeds INT32_MAX.
 */
MOE_API int64_t moe_align_capacity(int32_t T, int32_t topk, int32_t E, int32_t block_m);

/*
 * moe_align — token-to-expert alignment into expert-sorted, block-padded
 * order (P2 section 1.1: sorted_token_ids, num_tokens_post_padded, and the
 * per-block expert of the block-sorted GEMM, which computes the padding rows
 * of the blocks it runs).
 *
 * With flat slot ids f = t*topk + j, c_e = #{f : topk_ids[f] == e} and
 * P_e = ceil(c_e / block_m) * block_m, o_e = sum_{e' < e} P_e':
 *   sorted_token_ids[o_e + r] = the r-th smallest f routed to e (r < c_e);
 *       padding slots o_e + c_e .. o_e + P_e - 1 and the tail
 *       [o_E, capacity) hold the sentinel T*topk;
 *   expert_ids[b] = e for blocks b in [o_e / block_m, (o_e + P_e) / block_m),
 *       -1 for the blocks past o_E (experts with no rows get no block);
 *   num_tokens_post_padded[0] = o_E;
 *   inv[f] = position of f in sorted_token_ids, -1 for unrouted slots.
 * Every element of every output is written, so the result is a pure
 * function of the inputs (bit-exact and deterministic).
 *
 *   topk_ids                device, int32 [T, topk]
 *   sorted_token_ids        device, int32 [moe_align_capacity(...)]  (output)
 *   expert_ids              device, int32 [ceil(capacity / block_m)] (output)
 *   num_tokens_post_padded  device, int32 [1]                         (output)
 *   inv                     device, int32 [T*topk] or NULL            (output)
 * Requires 1 <= E <= MOE_MAX_EXPERTS, 1 <= topk <= MOE_MAX_TOPK,
 * 1 <= block_m <= 1024.
 */
MOE_API int moe_align(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E,
                      int32_t block_m, int32_t* sorted_token_ids, int32_t* expert_ids,
                      int32_t* num_tokens_post_padded, int32_t* inv, hipStream_t stream);

/*
 * moe_align_scratch_bytes — device scratch bytes moe_align_ws needs for
 * T * topk routed slots over E experts: 0 up to 8192 slots (one workgroup
 * aligns them, as moe_align does), else the per-workgroup expert counts and
 * starts of the multi-workgroup form (2 * ceil(T*topk / 1024) * E int32,
 * rounded up to 256 bytes).  Host only; negative status on invalid arguments.
 */
MOE_API int64_t moe_align_scratch_bytes(int32_t T, int32_t topk, int32_t E);

/*
 * moe_align_ws — moe_align (same definition, same outputs bit for bit) on
 * many workgroups: above 8192 routed slots, one workgroup per 1024 slots
 * counts its slots per expert, one workgroup scans the counts into padded
 * expert offsets and per-workgroup starts, and the counting workgroups
 * scatter their slots (stable: ascending flat index within an expert).
 * Up to 8192 slots it is moe_align.  One workgroup's ALUs bound moe_align
 * above that (16384 slots: 35 against 27 us; the prefill layer's 32768
 * slots: 63 against 27 us for the multi-workgroup form).
 *
 *   scratch        device, >= moe_align_scratch_bytes(T, topk, E) bytes,
 *                  4-byte aligned (may be NULL when that is 0); contents on
 *                  entry do not matter; owned by the caller
 *   other arguments as for moe_align.
 * MOE_ERR_WORKSPACE when the scratch is missing, misaligned or too small.
 */
MOE_API int moe_align_ws(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E, int32_t block_m,
                         int32_t* sorted_token_ids, int32_t* expert_ids, int32_t* num_tokens_post_padded,
                         int32_t* inv, void* scratch, int64_t scratch_bytes, hipStream_t stream);

/*
 * moe_quant_act — dynamic fp8 quantisation of bf16 activations, one
 * power-of-two scale per row and 128-column group (P2 section 1.2, the fused
 * kernel's scale rule, applied to the layer input as in the block-fp8 path):
 *   s = smallest power of two >= fl32(max(amax, 1e-10) * fl32(1/448)),
 *   q = E4M3FN_RNE(clamp(x / s, -448, 448))   (x / s is exact).
 *
 *   x       device, bf16 [rows, cols]
 *   codes   device, E4M3FN [rows, cols]            (output)
 *   scales  device, fp32 [rows, cols / 128]        (output)
 * Requires cols % 128 == 0.
 */
MOE_API int moe_quant_act(const void* x, int32_t rows, int32_t cols, uint8_t* codes,
                          float* scales, hipStream_t stream);

/*
 * moe_quant_act_mx — the same quantisation on 1x32 groups, scales stored as
 * E8M0 bytes (value 2^(byte - 127)): the activation side of the MXFP8 layer
 * (P3, the quantisation section of "Hosting Qwen on Blackwell": MXFP8, the
 * successor of block scaling; the scale rule is P2 section 1.2's, whose
 * power-of-two scales E8M0 holds exactly).
 *
 *   x       device, bf16 [rows, cols]
 *   codes   device, E4M3FN [rows, cols]            (output)
 *   scales  device, E8M0 bytes [rows, cols / 32]   (output)
 * Requires cols % 32 == 0; codes 8-byte and scales 4-byte aligned.
 */
MOE_API int moe_quant_act_mx(const void* x, int32_t rows, int32_t cols, uint8_t* codes,
                             uint8_t* scales, hipStream_t stream);

/*
 * moe_pack_mx_scales — reorder an MXFP8 weight's E8M0 scale bytes (P3's MXFP8
 * scheme: one scale per weight row and 32 consecutive K elements) for the
 * matrix-core kernels, once per weight as part of its static conversion.  The
 * kernels multiply 16 weight rows by 128 K elements per step, and each of a
 * wave's 64 lanes needs the scale of one row (lane % 16) and one 32-element
 * block (lane / 16); in the row-major layout those 64 bytes lie on 16 rows,
 * packed they are contiguous in lane order:
 *   packed[((e * rows/16 + t) * K/128 + s) * 64 + g * 16 + r]
 *       = scales[(e * rows + 16 t + r) * K/32 + 4 s + g]
 * for r < 16 and g < 4.  Every 16-row group keeps its byte range, so the
 * packed array has the row-major one's size and offsets at 16-row bounds.
 * Pass the results as w13_scale / w2_scale with MOE_FLAG_MX_PACKED_SCALES.
 *
 *   scales  device, E8M0 bytes [E, rows, K / 32] (row-major)
 *   packed  device, E8M0 bytes, E * rows * K / 32 of them (output; must not
 *           overlap scales)
 * Requires E >= 1, rows % 16 == 0 (w13: rows = 2I; w2: rows = H) and
 * K % 128 == 0 (w13: K = H; w2: K = I); else MOE_ERR_UNSUPPORTED (sizes) or
 * MOE_ERR_INVALID_ARG (null pointers, overlap, negative sizes).
 */
MOE_API int moe_pack_mx_scales(const uint8_t* scales, int32_t E, int32_t rows, int32_t K, uint8_t* packed,
                               hipStream_t stream);

/* Arguments of moe_forward (the pages' `apply(x, w1, w2, topk_weights,
 * topk_ids, activation=SiLU, expert_map=None,
 * apply_router_weight_on_input=False)`, P2 section 1.1). */
typedef struct moe_forward_args {
    int32_t T;            /* tokens */
    int32_t E;            /* experts */
    int32_t H;            /* hidden size (GEMM1 K, GEMM2 N) */
    int32_t I;            /* expert intermediate size (GEMM2 K) */
    int32_t topk;         /* routed experts per token */
    int32_t wdtype;       /* MOE_WDTYPE_* */
    const void* x;        /* device bf16 [T, H] */
    const void* w13;      /* device [E, 2I, H]: rows [0, I) gate, [I, 2I) up */
    const void* w13_scale;  /* FP8_E4M3: device fp32 [E, 2I/128, H/128];
                               MXFP8: device E8M0 bytes [E, 2I, H/32] (packed
                               by moe_pack_mx_scales with
                               MOE_FLAG_MX_PACKED_SCALES); else NULL */
    const void* w2;       /* device [E, H, I] */
    const void* w2_scale;   /* FP8_E4M3: device fp32 [E, H/128, I/128];
                               MXFP8: device E8M0 bytes [E, H, I/32] (packed
                               as w13_scale); else NULL */
    const int32_t* topk_ids;   /* device int32 [T, topk] */
    const float* topk_weights; /* device fp32 [T, topk] */
    void* out;            /* device bf16 [T, H] (output) */
    int32_t path;         /* MOE_PATH_*; AUTO unless a test forces a path */
    int32_t block_m;      /* rows per expert block; 0 lets the planner choose;
                             small-M path: 16, 32 or 64; large-M path: 256
                             (bf16) or 128 (fp8 and MXFP8) */
    int32_t flags;        /* MOE_FLAG_* bits; 0 is the layer of the pages' test */
    float clamp_limit;    /* SwiGLU clamp limit L: 0 for none, else L > 0
                             (+inf allowed, the same as none) */
} moe_forward_args;

/* What moe_forward will do for a set of arguments: the tile path, block size
 * and launch shapes it picks, so that a test can check which path a shape
 * takes without timing it (the role of the spy that P2 section 1.1's test
 * patches onto the A_is_sorted decision to see whether the sorted-A path
 * ran), plus the workspace offsets of the intermediates. */
typedef struct moe_plan_info {
    int32_t path;          /* MOE_PATH_SMALL_M or MOE_PATH_LARGE_M */
    int32_t block_m;       /* rows per expert block */
    int64_t capacity;      /* sorted rows incl. worst-case padding */
    int32_t num_blocks;    /* ceil(capacity / block_m): GEMM grid rows */
    int32_t gemm1_cols;    /* GEMM1 weight rows (of 2I, gate + up) per workgroup */
    int32_t gemm2_cols;    /* GEMM2 weight rows (of H) per column tile; a workgroup
                              may walk several adjacent tiles of its block */
    int32_t decode_layer;  /* 1 if moe_decode_layer takes these arguments */
    int64_t workspace_bytes;
    /* byte offsets of the forward's intermediates inside the workspace */
    int64_t off_sorted_ids, off_expert_ids, off_num_post_padded;
    int64_t off_xq, off_xs, off_inter, off_inter_scale, off_y;
} moe_plan_info;

/* moe_plan — fill *out for these arguments (host only, no device work):
 * the decisions moe_forward takes for them, reported instead of observed
 * (P2 section 1.1's test spies on the sorted-A decision; here the planner's
 * choice is a pure function a test can call).  Pointers in *a are not
 * inspected.  Returns a status. */
MOE_API int moe_plan(const moe_forward_args* a, moe_plan_info* out);

/* moe_forward_workspace — workspace bytes moe_forward needs for these
 * arguments (host only); negative status on invalid arguments. */
MOE_API int64_t moe_forward_workspace(const moe_forward_args* a);

/*
 * moe_forward — the fused MoE layer on one GPU:
 *   align (block_m from the plan) -> [fp8: quantise x per token and
 *   128-group] -> GEMM1 h = W13[e] . x_t over expert-sorted rows with the
 *   SiLU-mul epilogue a = bf16(bf16(silu(bf16 h_gate)) * bf16 h_up)
 *   [fp8: + per-row 128-group pow2 scale and E4M3 codes], kept in sorted
 *   order (P2 sections 1.1 and 1.2) -> GEMM2 y = tw * (W2[e] . a) with the
 *   router weight applied in fp32 after the GEMM (P2 section 1.1), one row
 *   per slot, kept in fp32 (bf16 weights) or bf16 (fp8 and MXFP8 weights) ->
 *   out_t = bf16(sum_j y_{t,j}) summed in fp32 in slot order j = 0..topk-1
 *   (the expert aggregation of P1, "Backend-Wechsel").
 * MXFP8: the same with x and the intermediate quantised per row and
 * 32-group, scales as E8M0 bytes, and every 32-element block of a product
 * scaled by its two E8M0 scales (inside the matrix-core instruction in the
 * weight-streaming down GEMM, folded into exact bf16 conversions elsewhere).
 * fp8 and MXFP8 weights arrive pre-quantised with their scales; the library
 * never quantises weights.
 * Layer variants (P2 section 1.1 names both switches: the
 * apply_router_weight_on_input argument and the activation config's clamp
 * limit):
 *   MOE_FLAG_WEIGHT_ON_INPUT  the slot's router weight scales the token's
 *       (quantised) input row of GEMM1 instead of GEMM2's output; GEMM1 being
 *       linear in that row, it is applied to GEMM1's fp32 accumulator before
 *       the bf16 rounding of h, and GEMM2's rows are left unweighted;
 *   clamp_limit L > 0  after their bf16 rounding the gate is capped at L and
 *       the up value held to [-L, L] before the SiLU-gated multiply.
 * MOE_FLAG_MX_PACKED_SCALES (MXFP8 only, else MOE_ERR_INVALID_ARG): both
 *       weight-scale arrays are in moe_pack_mx_scales's layout; the results
 *       are bitwise those of the row-major layout, and the weight-streaming
 *       kernels read the scales with one coalesced load per tile and step.
 *
 *   workspace  device buffer of at least moe_forward_workspace(a) bytes,
 *              256-byte aligned; its contents on entry do not matter and on
 *              exit hold the intermediates (layout in moe_plan_info).
 * Limits: bf16 requires H % 64 == 0 and I % 64 == 0; fp8 and MXFP8 require
 * H % 128 == 0 and I % 128 == 0; MXFP8 also T * H < 2^32 (else
 * MOE_ERR_UNSUPPORTED).  The large-M
 * path needs H % 256 == 0 and I % 128 == 0 (fp8 and MXFP8 also H, I <= 8192);
 * it runs 256-row blocks for bf16 weights and 128-row blocks for fp8 and MXFP8
 * weights.  AUTO takes it from 12 (bf16), 20 (fp8) or 28 (MXFP8) routed rows
 * per expert (on average) on when min(E, T * topk) * I / 128 >= 256, unless
 * block_m names a size of the weight-streaming path (16, 32, 64); forcing it
 * elsewhere is MOE_ERR_UNSUPPORTED.
 * The workspace's activation scales (off_xs, off_inter_scale) are fp32 for
 * FP8_E4M3 and E8M0 bytes for MXFP8; its y rows (off_y, [T*topk, H] by flat
 * slot) fp32 for bf16 weights and bf16 for FP8_E4M3 and MXFP8.  Unknown flag bits, and a clamp limit
 * that is negative or NaN, are MOE_ERR_INVALID_ARG.
 */
MOE_API int moe_forward(const moe_forward_args* a, void* workspace, int64_t workspace_bytes,
                        hipStream_t stream);

/*
 * moe_forward_profiled — moe_forward that also records HIP events on the
 * caller's stream around its stages, for timing each kernel where it runs:
 * events[i] is recorded before stage i and events[MOE_NUM_STAGES] after the
 * last one.  Stages: 0 align, 1 fp8 activation quantisation (empty for bf16),
 * 2 GEMM1 + SiLU-mul epilogue, 3 GEMM2, 4 combine.  The events are created by
 * the caller (hipEventCreate); n_events must be at least MOE_NUM_STAGES + 1.
 * Same results and errors as moe_forward, plus MOE_ERR_INVALID_ARG for a
 * missing event array.
 */
#define MOE_NUM_STAGES 5
MOE_API int moe_forward_profiled(const moe_forward_args* a, void* workspace, int64_t workspace_bytes,
                                 hipStream_t stream, hipEvent_t* events, int32_t n_events);

/*
 * moe_forward_noalloc — moe_forward for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Its workspace is a static device array inside the
 * library, MOE_NOALLOC_MAX_BYTES long, of which every GPU the library runs
 * on holds one copy until the process ends; the call itself allocates
 * nothing.  The caller still passes the inputs and the output in *a.
 *
 * Same results as moe_forward (the same kernels, bit for bit) and the same
 * argument errors, plus MOE_ERR_WORKSPACE when moe_forward_workspace(a)
 * exceeds MOE_NOALLOC_MAX_BYTES (64 MiB: decode-sized layers, e.g. 16 tokens
 * of 128 experts with H 4096 and I 1536 need 8.4 MB), and MOE_ERR_HIP if the
 * array's device address cannot be found (looked up once per device, on the
 * first call there).  Every call on one GPU uses the same array: calls that
 * overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller.  The array's contents on entry do not matter; it
 * keeps the last call's intermediates.
 */
#define MOE_NOALLOC_MAX_BYTES (64 << 20)
MOE_API int moe_forward_noalloc(const moe_forward_args* a, hipStream_t stream);

/*
 * moe_decode_layer — the whole layer for few tokens (decode) in ONE kernel
 * launch: [router top-k from logits] and [fp8 activation quantisation] ->
 * alignment -> GEMM1 + SiLU-mul epilogue -> GEMM2 -> top-k combine, the phases
 * separated by grid-wide barriers inside a persistent cooperative kernel
 * (P3, section on MoE dispatch/combine: the decode-side kernels are fused
 * into one, since per-kernel latency is a visible share at a few tokens per
 * step).  Results are bitwise those of moe_route + moe_forward.  On MI355X
 * it measures slower than that pair (one token, 8 of 256 experts, H 7168,
 * I 2048: 0.215 against 0.141 ms): a grid barrier across the 8 XCDs costs
 * about what a kernel boundary does, and a cooperative launch more than a
 * plain one; it is for callers that need the layer in one launch.
 *
 *   a                  as for moe_forward (layer variants included);
 *   router_logits      device fp32 [T, E], or NULL.  With logits the layer
 *                      routes them as moe_route(renormalize) does and writes
 *                      the routing to topk_ids_out / topk_weights_out (device
 *                      int32 / fp32 [T, topk]; a->topk_ids and
 *                      a->topk_weights are not read).  With NULL, the routing
 *                      is a->topk_ids / a->topk_weights and the outputs are
 *                      not written.
 *   sync               device uint32 [MOE_SYNC_WORDS], all zero before the
 *                      first call; every call leaves it zero.  Calls sharing a
 *                      sync buffer must be ordered on one stream.  If a
 *                      grid-barrier wait ever exceeds 2 s (the device could
 *                      not keep every workgroup resident), the kernel sets
 *                      sync[MOE_SYNC_ERROR] and finishes with an undefined
 *                      output; the buffer must then be zeroed again.
 *   workspace          as for moe_forward (same size and layout).
 * Supported where moe_plan reports decode_layer = 1: the weight-streaming
 * path with block_m 16, T * topk <= 256, H % 256 == 0, I % 128 == 0 (else
 * MOE_ERR_UNSUPPORTED); with logits also topk <= E.  The device must support
 * cooperative launches (else MOE_ERR_HIP).
 */
#define MOE_SYNC_WORDS 640   /* 2560 bytes */
#define MOE_SYNC_ERROR 576
MOE_API int moe_decode_layer(const moe_forward_args* a, const float* router_logits, int32_t renormalize,
                             int32_t* topk_ids_out, float* topk_weights_out, uint32_t* sync, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
