"""The intermediate checker (tests/intermediate_check.py) on the CPU.

A stand-in workspace is filled from the oracle (the alignment and the
expert intermediate rows in sorted order, laid out as moe_plan describes it),
and the checker must pass it; then one rounding point at a time is dropped or
changed in a CPU stand-in for the epilogue, and the checker must flag it.
This is what lets the GPU test see each rounding point of P2 section 1.2.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_layer_amd.workloads import exact_sum_layer

from intermediate_check import check_workspace, group_of

_LIMIT = float(np.float32(0.4))


def _layer(wdtype, T=48, E=4, H=256, I=256, k=2, pow2=False):
    d = exact_sum_layer(T, E, H, I, k, wdtype, pow2_route_weights=pow2)
    x64 = O.bf16_bits_to_f64(d["x_bits"])
    if wdtype == "bf16":
        w13 = np.stack([O.bf16_bits_to_f64(w[0]) for w in d["experts"]])
    elif wdtype == "fp8":
        w13 = np.stack([O.dequant_block(w[0], w[1]) for w in d["experts"]])
    else:
        w13 = np.stack([O.dequant_mx(w[0], w[1]) for w in d["experts"]])
    return x64, w13, d["ids"], d["tw"]


def _stand_in(x64, w13e, toks, tws, wdtype, woi, clamp, planted):
    """The epilogue's rows computed on the CPU, with one planted mistake."""
    fp8 = wdtype != "bf16"
    group = group_of(wdtype)
    if planted is None:
        r = O.expert_intermediate(x64, w13e, toks, tws, fp8=fp8, group=group, weight_on_input=woi,
                                  clamp_limit=clamp)
        return r["codes"] if fp8 else r["a"], r["scales"]
    xt = x64[toks]
    if fp8:
        xt = O.quant_act(xt, group)[2]
    if woi:
        xt = xt * tws[:, None]
    I = w13e.shape[0] // 2
    h = xt @ w13e.T
    rnd = O.round_bf16
    g, u = (h[:, :I], h[:, I:]) if planted == "no_h_round" else (rnd(h[:, :I]), rnd(h[:, I:]))
    if planted == "swap_gate_up":
        g, u = u, g
    if clamp:
        g = np.minimum(g, clamp) if planted != "clamp_gate_both_ways" else np.clip(g, -clamp, clamp)
        u = np.clip(u, -clamp, clamp)
    s = g / (1.0 + np.exp(-g))
    if planted != "no_silu_round":
        s = rnd(s)
    a = s * u
    if planted != "no_product_round":
        a = rnd(a)
    if not fp8:
        return rnd(a), None
    if planted == "scale_not_pow2":
        amax = np.abs(a.reshape(len(a), -1, group)).max(axis=2)
        sc = O.fl32(np.maximum(amax, 1e-10) / 448.0)
        if wdtype == "mxfp8":       # E8M0 holds powers of two only: round down instead of up
            m, ex = np.frexp(sc)
            sc = np.ldexp(1.0, ex - 1)
        q = O.round_e4m3(np.clip(a.reshape(len(a), -1, group) / sc[:, :, None], -448, 448))
        return O.e4m3_encode(q).reshape(a.shape), sc
    c, sc, _ = O.quant_act(a, group)
    return c, sc


def _workspace(x64, w13, ids, tw, wdtype, B, woi=False, clamp=None, planted=None):
    """A byte workspace laid out like moe_forward's (offsets in the plan dict)."""
    T, k = ids.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    al = O.align(ids, E, B)
    cap = al["capacity"]
    nblk = -(-cap // B)
    rows = nblk * B
    group = group_of(wdtype)
    es = 2 if wdtype == "bf16" else 1
    off_inter = ((4 * cap + 255) // 256) * 256
    off_sc = off_inter + ((rows * I * es + 255) // 256) * 256
    ws = np.zeros(off_sc + rows * (I // group) * 4 + 256, np.uint8)
    ws[: 4 * cap] = al["sorted_token_ids"].view(np.uint8)
    sorted_ids = al["sorted_token_ids"]
    R = T * k
    inter = np.zeros((rows, I), np.uint16 if wdtype == "bf16" else np.uint8)
    scales = np.zeros((rows, I // group), np.float32 if wdtype == "fp8" else np.uint8)
    valid = np.nonzero(sorted_ids < R)[0]
    f = sorted_ids[valid]
    e = ids[f // k, f % k]
    for ex in np.unique(e):
        sel = e == ex
        vals, sc = _stand_in(x64, w13[ex], (f // k)[sel], tw[(f // k)[sel], (f % k)[sel]].astype(np.float64),
                             wdtype, woi, clamp, planted)
        if wdtype == "bf16":
            inter[valid[sel]] = torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16) \
                .view(torch.int16).numpy().view(np.uint16)
        else:
            inter[valid[sel]] = vals
            scales[valid[sel]] = sc if wdtype == "fp8" else O.e8m0_encode(sc)
    ws[off_inter: off_inter + inter.nbytes] = inter.view(np.uint8).reshape(-1)
    if wdtype != "bf16":
        ws[off_sc: off_sc + scales.nbytes] = scales.view(np.uint8).reshape(-1)
    plan = dict(num_blocks=nblk, block_m=B, capacity=cap, off_sorted_ids=0, off_inter=off_inter,
                off_inter_scale=off_sc)
    return torch.from_numpy(ws), plan


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("variant", ["plain", "clamp", "on_input"])
def test_checker_passes_the_oracle(wdtype, variant):
    woi = variant == "on_input"
    clamp = _LIMIT if variant == "clamp" else None
    x64, w13, ids, tw = _layer(wdtype, pow2=woi)
    ws, plan = _workspace(x64, w13, ids, tw, wdtype, 16, woi, clamp)
    n, amb, bad, nrows = check_workspace(ws, plan, w13.shape[1] // 2, x64, w13, ids, tw, wdtype, woi,
                                         clamp or 0.0)
    assert nrows == int(((ids >= 0) & (ids < w13.shape[0])).sum())
    assert bad == 0 and n > 0


_PLANTED = ["no_h_round", "no_silu_round", "swap_gate_up", "no_product_round", "scale_not_pow2",
            "clamp_gate_both_ways"]


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("planted", _PLANTED)
def test_checker_catches_planted_mistakes(wdtype, planted):
    if planted == "scale_not_pow2" and wdtype == "bf16":
        pytest.skip("bf16 has no intermediate scale")
    if planted == "no_product_round" and wdtype == "bf16":
        pytest.skip("a stored bf16 value is rounded anyway")
    clamp = _LIMIT if planted == "clamp_gate_both_ways" else None
    x64, w13, ids, tw = _layer(wdtype)
    ws, plan = _workspace(x64, w13, ids, tw, wdtype, 16, False, clamp, planted)
    _, _, bad, _ = check_workspace(ws, plan, w13.shape[1] // 2, x64, w13, ids, tw, wdtype, False, clamp or 0.0)
    assert bad > 0, planted


def test_exact_sum_layer_sums_are_exact_in_fp32():
    """The fixture's premise: fp32 accumulation in two different orders gives
    the fp64 gate/up products exactly, and x survives the fp8 activation
    quantisation (128- and 32-groups) unchanged."""
    for wdtype in ("bf16", "fp8", "mxfp8"):
        x64, w13, _, _ = _layer(wdtype, T=8, E=2, H=512, I=128)
        for e in range(w13.shape[0]):
            prod = (x64[:, None, :] * w13[e][None, :, :]).astype(np.float32)   # exact products
            h64 = x64 @ w13[e].T
            fwd = np.zeros(h64.shape, np.float32)
            for kk in range(prod.shape[2]):
                fwd += prod[:, :, kk]
            rev = np.zeros(h64.shape, np.float32)
            for kk in reversed(range(prod.shape[2])):
                rev += prod[:, :, kk]
            assert np.array_equal(fwd.astype(np.float64), h64)
            assert np.array_equal(rev.astype(np.float64), h64)
        assert np.array_equal(O.quant_act(x64, 128)[2], x64)
        assert np.array_equal(O.quant_act(x64, 32)[2], x64)
