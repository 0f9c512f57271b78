"""Reference oracle for the fused Mixture-of-Experts layer (plain, slow, fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import or run this module.  The product
path (the HIP library and its Python binding) never calls it, and this module
imports nothing from the product package.

What it computes, step by step, with the passage each step follows
("P2" is the blog analysis of vLLM PR #64760, "sorted-A TMA for FP8 MoE";
"P1" is the kinachrichten.com article on AWS's two fused-MoE kernel
optimisations for SageMaker AI on H200):

  route        softmax over the experts, top-k, renormalised weights.  The
               layer receives ``topk_ids``/``topk_weights`` from the router
               (P2, section 1.1, the test that builds ``topk_weights`` with a
               softmax and calls ``kernel.apply``).  Softmax -> top-k ->
               renormalise equals a softmax over the k selected logits, since
               the full denominator cancels; that plain definition is what is
               written below.
  align        expert histogram, padding of each expert's row count to a
               multiple of the block size, exclusive prefix sum and a stable
               scatter of flat slot ids into expert-sorted, block-padded order
               (P2, section 1.1: ``sorted_token_ids``, ``num_tokens_post_padded``,
               and the GEMM computing the padding rows of the blocks it runs).
  quant_act    dynamic fp8-e4m3 quantisation with one power-of-two scale per
               row and 128-column group (P2, section 1.2, the fused
               SiLU-mul-quant kernel: amax, floor 1e-10, times 1/448, rounded up
               to a power of two, divide, clamp to +-448, cast to e4m3).  The
               MXFP8 variant (the successor scheme of P3, section on
               quantisation for Blackwell) uses the same rule on 1x32 groups;
               its power-of-two scales are E8M0 bytes.
  forward      grouped gate/up GEMM, SiLU-gated multiply with the rounding
               points of P2 section 1.2 (gate/up rounded to the activation dtype,
               SiLU rounded before the multiply, product rounded), optional fp8
               re-quantisation of the intermediate, grouped down GEMM, router
               weight applied after the down GEMM (P2 section 1.1,
               ``apply_router_weight_on_input=False`` and the weight multiplied
               inside GEMM2), and the sum over the k routed rows of each token
               (the "expert aggregation" of P1, section on the backend switch).

Readings where the pages leave a step open (each is also a decision the GPU
path must follow):
  * ties in top-k go to the lower expert index; ids are emitted in descending
    logit order; selection compares logits, never exponentiated values;
  * rows of one expert keep ascending flat slot order f = t*topk + j; padding
    slots and the tail of ``sorted_token_ids`` hold the sentinel T*topk; the
    tail of ``expert_ids`` holds -1; experts with no rows get no block;
  * expert ids outside [0, E) are not routed and contribute nothing;
    duplicate ids in one token each count;
  * w13 holds gate rows [0, I) then up rows [I, 2I) (P2 section 1.2 reads
    gate from the first half of each 2I row and up from the second);
  * the power-of-two scale is the smallest power of two >= the fp32 product,
    computed exactly (never through an approximate log2);
  * fp8 is OCP E4M3FN (max 448, no infinities), round to nearest even;
  * the layer output is returned in fp64, unrounded;
  * layer variants (P2 section 1.1 names both switches, nothing more):
    with the router weight on the input, the token's (quantised) input row is
    multiplied by the slot's weight before the gate/up GEMM and the down GEMM
    output is not weighted; a SwiGLU clamp limit L caps the gate at L and
    holds the up value to [-L, L], after their bf16 rounding.

Every input of the method is exact in fp64: bf16 values and e4m3 codes times
fp32 block scales promote without error, so the oracle and the GPU consume the
same real numbers.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "round_bf16", "bf16_bits_to_f64", "round_e4m3", "e4m3_decode",
    "e4m3_encode", "fl32", "pow2_ceil", "fp8_group_scale", "quant_act",
    "route", "align", "align_capacity", "dequant_block", "forward", "expert_rows",
    "expert_intermediate",
    "MX_BLOCK", "e8m0_decode", "e8m0_encode", "dequant_mx",
]

# ----------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------

_BF16_MIN_NORMAL_EXP = -126   # smallest normal binade of bf16 (same as fp32)
_BF16_MANT_BITS = 7           # explicit fraction bits of bf16
_E4M3_MIN_NORMAL_EXP = -6     # OCP E4M3FN: exponent bias 7, min normal 2^-6
_E4M3_MANT_BITS = 3
E4M3_MAX = 448.0              # 1.75 * 2^8, the largest finite E4M3FN value


def _binade(v: np.ndarray) -> np.ndarray:
    """floor(log2|v|) for nonzero finite v, exact (from frexp)."""
    _, e = np.frexp(v)
    return e.astype(np.int64) - 1


def _round_to_grid(v: np.ndarray, min_normal_exp: int, mant_bits: int) -> np.ndarray:
    """Round fp64 values to the nearest value with ``mant_bits`` fraction bits
    (normal range) or the subnormal quantum below ``min_normal_exp``; ties to
    even.  Division and multiplication by the power-of-two quantum are exact.
    A zero keeps its sign, and so does a value that rounds to zero, as in an
    IEEE conversion (a cast of -0.0 gives the negative-zero code)."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    np.copysign(out, v, out=out)
    nz = (v != 0) & np.isfinite(v)
    e = np.maximum(_binade(v[nz]), min_normal_exp)
    q = np.ldexp(1.0, (e - mant_bits).astype(np.int64))
    out[nz] = np.copysign(np.rint(v[nz] / q) * q, v[nz])   # np.rint rounds half to even
    out[~np.isfinite(v)] = v[~np.isfinite(v)]
    return out


def round_bf16(v) -> np.ndarray:
    """Round to the nearest bf16 value (RNE); overflow goes to +-inf."""
    r = _round_to_grid(v, _BF16_MIN_NORMAL_EXP, _BF16_MANT_BITS)
    r[np.abs(r) >= 2.0 ** 128] = np.copysign(np.inf, r[np.abs(r) >= 2.0 ** 128])
    return r


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to fp64: a bf16 value is the upper
    half of an fp32 word."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def round_e4m3(v) -> np.ndarray:
    """Round to the nearest E4M3FN value (RNE).  Inputs must already lie in
    [-448, 448] (the method clamps before the cast)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or not np.all(np.isfinite(v)):
        raise ValueError("round_e4m3 expects finite values within +-448")
    return _round_to_grid(v, _E4M3_MIN_NORMAL_EXP, _E4M3_MANT_BITS)


def e4m3_decode(codes) -> np.ndarray:
    """Decode E4M3FN bytes: sign bit, 4 exponent bits (bias 7), 3 fraction
    bits; exponent field 0 is subnormal (m * 2^-9); 0x7F/0xFF are NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    mf = c & 0x7
    val = np.where(ef == 0, mf * 2.0 ** -9,
                   (1.0 + mf / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((ef == 0xF) & (mf == 0x7), np.nan, val)
    return sign * val


def e4m3_encode(v) -> np.ndarray:
    """Encode values that lie exactly on the E4M3FN grid to their bytes."""
    v = np.asarray(v, dtype=np.float64)
    if not np.array_equal(round_e4m3(v), v):
        raise ValueError("e4m3_encode expects values on the E4M3FN grid")
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.int64)
    code = np.zeros(v.shape, dtype=np.int64)
    sub = a < 2.0 ** _E4M3_MIN_NORMAL_EXP
    code[sub] = (a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = ~sub
    e = _binade(a[nrm])
    m = (a[nrm] / np.ldexp(1.0, e) - 1.0) * 8.0
    code[nrm] = ((e + 7) << 3) | m.astype(np.int64)
    return (code | sign).astype(np.uint8)


def fl32(v) -> np.ndarray:
    """Round to fp32 (numpy's cast rounds to nearest even) and widen again."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def pow2_ceil(v) -> np.ndarray:
    """Smallest power of two >= v, for positive finite v, exact via frexp."""
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                          # v = m * 2^e, m in [0.5, 1)
    return np.where(m == 0.5, v, np.ldexp(1.0, e))


# ----------------------------------------------------------------------------
# Dynamic fp8 activation quantisation (P2, section 1.2)
# ----------------------------------------------------------------------------

_EPS32 = float(np.float32(1e-10))          # the 1e-10 floor as an fp32 constant
_INV448_32 = float(np.float32(1.0 / 448.0))  # 1/448 as an fp32 constant


def fp8_group_scale(amax) -> np.ndarray:
    """Scale of one 128-wide group from its absolute maximum: the fp32
    product max(amax, 1e-10) * (1/448), rounded up to a power of two."""
    a = fl32(np.maximum(fl32(amax), _EPS32))
    s_raw = fl32(a * _INV448_32)               # one correctly rounded fp32 multiply
    return pow2_ceil(s_raw)


def quant_act(v, group: int = 128):
    """Quantise each row of ``v`` ([rows, cols], cols % group == 0) per
    ``group`` columns.  Returns (codes uint8, scales fp64 [rows, cols/group],
    dequantised fp64 values = e4m3(code) * scale)."""
    v = np.asarray(v, dtype=np.float64)
    rows, cols = v.shape
    if cols % group:
        raise ValueError("column count must be a multiple of the group size")
    g = v.reshape(rows, cols // group, group)
    s = fp8_group_scale(np.max(np.abs(g), axis=2))
    q = round_e4m3(np.clip(g / s[:, :, None], -E4M3_MAX, E4M3_MAX))
    codes = e4m3_encode(q).reshape(rows, cols)
    deq = (q * s[:, :, None]).reshape(rows, cols)
    return codes, s, deq


# ----------------------------------------------------------------------------
# MXFP8 (P3, quantisation section: MXFP8 weights, converted statically):
# e4m3 elements with one E8M0 scale (a bare power of two) per 1x32 block along
# the reduction dimension.  Reading: activations (x and the intermediate) are
# quantised with the P2 section 1.2 rule on 1x32 groups (quant_act(v, 32)),
# which never saturates; weights arrive already converted by the caller.
# ----------------------------------------------------------------------------

MX_BLOCK = 32


def e8m0_decode(s) -> np.ndarray:
    """E8M0 scale byte -> 2^(s - 127); 255 is NaN."""
    s = np.asarray(s).astype(np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def e8m0_encode(scale) -> np.ndarray:
    """Power of two in [2^-127, 2^127] -> its E8M0 byte (exact, via frexp)."""
    m, e = np.frexp(np.asarray(scale, dtype=np.float64))
    if not np.all(m == 0.5):
        raise ValueError("E8M0 holds powers of two only")
    b = e - 1 + 127
    if np.any((b < 0) | (b > 254)):
        raise ValueError("power of two outside the E8M0 range")
    return b.astype(np.uint8)


def dequant_mx(codes, scales, block: int = MX_BLOCK) -> np.ndarray:
    """MXFP8 weights from e4m3 codes [.., N, K] and E8M0 scales [.., N, K/block]:
    value = e4m3(code) * 2^(s - 127) of its row's K block."""
    w = e4m3_decode(codes)
    return w * np.repeat(e8m0_decode(scales), block, axis=-1)


# ----------------------------------------------------------------------------
# Routing: softmax over experts, top-k, renormalise
# ----------------------------------------------------------------------------

def route(logits, topk: int, renormalize: bool = True):
    """Per token, the ``topk`` largest logits (ties to the lower expert index),
    in descending order, and their weights.

    renormalize=True : w_j = exp(l_j - l_max) / sum over the selected experts
                       (softmax, top-k, renormalise).
    renormalize=False: w_j = exp(l_j - l_max) / sum over all experts
                       (the softmax probabilities of the winners).
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= topk <= E:
        raise ValueError("need 1 <= topk <= E")
    idx = np.arange(E)
    ids = np.empty((T, topk), dtype=np.int32)
    w = np.empty((T, topk), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((idx, -lg[t]))       # primary: logit desc; then index asc
        sel = order[:topk]
        ids[t] = sel
        ex = np.exp(lg[t, sel] - lg[t, sel[0]])
        denom = ex.sum() if renormalize else np.exp(lg[t] - lg[t, sel[0]]).sum()
        w[t] = ex / denom
    return ids, w


# ----------------------------------------------------------------------------
# Alignment: expert-sorted, block-padded order
# ----------------------------------------------------------------------------

def align_capacity(T: int, topk: int, E: int, block_m: int) -> int:
    """Upper bound on the padded row count: every expert may waste B-1 rows."""
    return T * topk + E * (block_m - 1)


def align(topk_ids, E: int, block_m: int):
    """Returns a dict with
      sorted_token_ids [cap] int32 : flat slot ids f = t*topk + j, grouped by
                                     expert in ascending expert order, ascending
                                     f inside an expert, each expert's group
                                     padded to a multiple of block_m with the
                                     sentinel T*topk; tail [padded, cap) holds it
                                     too;
      expert_ids [ceil(cap/B)] int32 : expert of each block, -1 past the end;
      num_tokens_post_padded int     : total padded row count;
      inv [T*topk] int32             : position of f in sorted_token_ids, -1 for
                                       slots whose id is outside [0, E).
    """
    ids = np.asarray(topk_ids).astype(np.int64)
    T, k = ids.shape
    R = T * k
    B = int(block_m)
    cap = align_capacity(T, k, E, B)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    padded = -(-counts // B) * B
    offsets = np.concatenate([[0], np.cumsum(padded)])
    sorted_ids = np.full(cap, R, dtype=np.int32)
    inv = np.full(R, -1, dtype=np.int32)
    for e in range(E):
        members = np.nonzero(flat == e)[0]          # ascending flat index
        pos = offsets[e] + np.arange(len(members))
        sorted_ids[pos] = members
        inv[members] = pos
    nblocks = -(-cap // B)
    expert_ids = np.full(nblocks, -1, dtype=np.int32)
    for e in range(E):
        expert_ids[offsets[e] // B: offsets[e + 1] // B] = e
    return dict(sorted_token_ids=sorted_ids, expert_ids=expert_ids,
                num_tokens_post_padded=int(offsets[E]), inv=inv, capacity=cap)


# ----------------------------------------------------------------------------
# The expert computation
# ----------------------------------------------------------------------------

def dequant_block(codes, scales, block: int = 128) -> np.ndarray:
    """Weights from e4m3 codes [.., N, K] and fp32 block scales
    [.., N/block, K/block]: value = e4m3(code) * scale of its block."""
    w = e4m3_decode(codes)
    s = np.asarray(scales, dtype=np.float64)
    s = np.repeat(np.repeat(s, block, axis=-2), block, axis=-1)
    return w * s


def _silu_mul(g, u, method: bool, clamp_limit=None):
    """SiLU(gate) * up; in method mode with the rounding points of the fused
    kernel: gate/up in bf16, SiLU rounded to bf16 before the multiply, product
    rounded to bf16.  With a clamp limit L (the activation config's
    ``clamp_limit``, P2 section 1.1), the gate is capped at L and the up value
    held to [-L, L] (after their bf16 rounding in method mode)."""
    if method:
        g = round_bf16(g)
        u = round_bf16(u)
    if clamp_limit is not None:
        g = np.minimum(g, clamp_limit)
        u = np.clip(u, -clamp_limit, clamp_limit)
    if method:
        s = round_bf16(g / (1.0 + np.exp(-g)))
        return round_bf16(s * u)
    return g / (1.0 + np.exp(-g)) * u


def forward(x, w13, w2, topk_ids, topk_weights, *, mode: str = "method",
            fp8: bool = False, group: int = 128, weight_on_input: bool = False,
            clamp_limit=None):
    """The layer output out[t] = sum_j tw[t,j] * W2[e] . act(W13[e] . x_t) for
    the valid experts e = topk_ids[t, j], returned unrounded in fp64.

    x            [T, H] fp64 (the bf16 activations, exact)
    w13          [E, 2I, H] fp64 (gate rows [0, I), up rows [I, 2I)); for fp8
                 pass the dequantised block-scaled weights
    w2           [E, H, I] fp64
    topk_ids     [T, k] integer; ids outside [0, E) are skipped
    topk_weights [T, k] float
    mode         "method": the rounding points of the fused kernel;
                 "pure": no rounding beyond the inputs
    fp8          quantise x and the intermediate per row and ``group`` columns
                 (128: block-scaled fp8; 32: MXFP8)
    weight_on_input
                 apply the router weight to the token's input row before the
                 gate/up GEMM instead of after the down GEMM (P2 section 1.1,
                 ``apply_router_weight_on_input``); the input is the quantised
                 row when fp8, and the scaled row itself is not rounded
    clamp_limit  None, or the SwiGLU clamp limit L > 0 (see ``_silu_mul``)
    """
    if mode not in ("method", "pure"):
        raise ValueError(mode)
    method = mode == "method"
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E, twoI, H2 = w13.shape
    I = twoI // 2
    if H2 != H or w2.shape != (E, H, I):
        raise ValueError("shape mismatch")
    ids = np.asarray(topk_ids).astype(np.int64)
    tw = np.asarray(topk_weights, dtype=np.float64)
    k = ids.shape[1]
    xh = quant_act(x, group)[2] if (fp8 and method) else x
    out = np.zeros((T, H), dtype=np.float64)
    flat = ids.reshape(-1)
    for e in range(E):
        slots = np.nonzero(flat == e)[0]
        if slots.size == 0:
            continue
        tok = slots // k
        w_rows = tw.reshape(-1)[slots][:, None]
        xin = xh[tok] * w_rows if weight_on_input else xh[tok]
        h = xin @ np.asarray(w13[e], dtype=np.float64).T             # [rows, 2I]
        a = _silu_mul(h[:, :I], h[:, I:], method, clamp_limit)
        if fp8 and method:
            a = quant_act(a, group)[2]
        y = a @ np.asarray(w2[e], dtype=np.float64).T                # [rows, H]
        if not weight_on_input:
            y *= w_rows
        np.add.at(out, tok, y)
    return out


def expert_intermediate(x, w13_e, rows_tok, rows_tw, *, mode="method", fp8=False,
                        group: int = 128, weight_on_input: bool = False, clamp_limit=None):
    """The rows one expert hands its down GEMM, for the given tokens: the
    gate/up GEMM, the SiLU-gated multiply with its rounding points and, with
    ``fp8``, the per-row re-quantisation of P2 section 1.2 (options as for
    ``forward``).  Returns a dict with
      h       fp64 [rows, 2I]   gate/up results before any rounding;
      a       fp64 [rows, I]    the SiLU-gated product (bf16 values in method mode);
      codes   uint8 [rows, I]   e4m3 codes of ``a`` (fp8 and method mode only);
      scales  fp64 [rows, I/group] their power-of-two group scales;
      deq     fp64 [rows, I]    what the down GEMM multiplies (codes * scales,
                                or ``a``)."""
    method = mode == "method"
    xt = np.asarray(x, dtype=np.float64)[rows_tok]
    if fp8 and method:
        xt = quant_act(xt, group)[2]
    if weight_on_input:
        xt = xt * np.asarray(rows_tw, dtype=np.float64)[:, None]
    I = w13_e.shape[0] // 2
    h = xt @ np.asarray(w13_e, dtype=np.float64).T
    a = _silu_mul(h[:, :I], h[:, I:], method, clamp_limit)
    out = dict(h=h, a=a, codes=None, scales=None, deq=a)
    if fp8 and method:
        out["codes"], out["scales"], out["deq"] = quant_act(a, group)
    return out


def expert_rows(x, w13_e, w2_e, rows_tok, rows_tw, *, mode="method", fp8=False,
                group: int = 128, weight_on_input: bool = False, clamp_limit=None):
    """Contribution y = tw * W2[e] . act(W13[e] . x_t) of one expert to the
    given tokens (used to evaluate sampled outputs of large layers one expert
    at a time), with the options of ``forward``.  Returns [len(rows_tok), H]
    fp64."""
    a = expert_intermediate(x, w13_e, rows_tok, rows_tw, mode=mode, fp8=fp8, group=group,
                            weight_on_input=weight_on_input, clamp_limit=clamp_limit)["deq"]
    y = a @ np.asarray(w2_e, dtype=np.float64).T
    w_rows = np.asarray(rows_tw, dtype=np.float64)[:, None]
    return y if weight_on_input else y * w_rows
