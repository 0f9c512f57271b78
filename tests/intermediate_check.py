"""Reading the fused epilogue's intermediate out of a moe_forward workspace
and comparing it with the oracle's ``expert_intermediate`` (used by the GPU
tests, and on the CPU by the checker's own tests).

Rows are mapped through the sorted slot ids in the same workspace: row r holds
slot f = sorted[r] (token f // k, slot f % k, expert ids[t, j]) when f < T*k.
bf16 values must equal the oracle's bit for bit; fp8 / MXFP8 codes and group
scales likewise, per group.  The one freedom a correct kernel has is the
exp inside SiLU (a few fp32 ulps): where the exact SiLU lies within a
relative 2^-19 of a bf16 rounding boundary either neighbour is correct, and
the product (for fp8: the group's codes and scale) of either is accepted;
such elements are counted.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle as O

AMBIG_REL = 2.0 ** -19     # relative error bound of a GPU SiLU in fp32, with margin


def group_of(wdtype: str) -> int:
    return 32 if wdtype == "mxfp8" else 128


def read_intermediate(ws: torch.Tensor, plan: dict, I: int, wdtype: str):
    """(sorted ids [cap], values-or-codes [rows, I], scales [rows, I/group] or None)
    from a workspace."""
    rows = plan["num_blocks"] * plan["block_m"]
    cap = plan["capacity"]
    sorted_ids = ws[plan["off_sorted_ids"]: plan["off_sorted_ids"] + 4 * cap].cpu().numpy().view(np.int32)
    o = plan["off_inter"]
    if wdtype == "bf16":
        vals = ws[o: o + rows * I * 2].cpu().numpy().view(np.uint16).reshape(rows, I)
        return sorted_ids, O.bf16_bits_to_f64(vals), None
    codes = ws[o: o + rows * I].cpu().numpy().reshape(rows, I)
    so = plan["off_inter_scale"]
    if wdtype == "mxfp8":
        sb = ws[so: so + rows * (I // 32)].cpu().numpy().reshape(rows, I // 32)
        return sorted_ids, codes, O.e8m0_decode(sb)
    sc = ws[so: so + rows * (I // 128) * 4].cpu().numpy().view(np.float32).reshape(rows, I // 128)
    return sorted_ids, codes, sc.astype(np.float64)


def _silu_candidates(g, u):
    """Per element the bf16 SiLU-gated products a correct kernel may give:
    (a_lo, a_hi, ambiguous), where a_lo != a_hi only when the exact SiLU of g
    lies within AMBIG_REL of a bf16 rounding boundary."""
    s = g / (1.0 + np.exp(-g))
    r1 = O.round_bf16(s * (1.0 - AMBIG_REL))
    r2 = O.round_bf16(s * (1.0 + AMBIG_REL))
    return O.round_bf16(r1 * u), O.round_bf16(r2 * u), r1 != r2


def compare_rows(gpu_vals, gpu_scales, ref: dict, wdtype: str, clamp_limit):
    """Compare one expert's rows.  Returns (elements compared, near-boundary
    elements, mismatches) and asserts nothing (the caller decides)."""
    I = ref["a"].shape[1]
    h = ref["h"]
    g = O.round_bf16(h[:, :I])
    u = O.round_bf16(h[:, I:])
    if clamp_limit:
        g = np.minimum(g, clamp_limit)
        u = np.clip(u, -clamp_limit, clamp_limit)
    a_lo, a_hi, amb = _silu_candidates(g, u)
    # unambiguous elements: the two candidates agree with the oracle's product
    assert np.array_equal(np.where(amb, ref["a"], a_lo), ref["a"])
    if wdtype == "bf16":
        ok = (gpu_vals == ref["a"]) | (amb & ((gpu_vals == a_lo) | (gpu_vals == a_hi)))
        return gpu_vals.size, int(amb.sum()), int((~ok).sum())
    group = group_of(wdtype)
    ng = I // group
    bad = 0
    for r in range(gpu_vals.shape[0]):
        for q in range(ng):
            sl = slice(q * group, (q + 1) * group)
            want_c, want_s = ref["codes"][r, sl], ref["scales"][r, q]
            got_c, got_s = gpu_vals[r, sl], gpu_scales[r, q]
            if np.array_equal(got_c, want_c) and got_s == want_s:
                continue
            pos = np.nonzero(amb[r, sl])[0]
            if len(pos) == 0 or len(pos) > 6:
                bad += 1
                continue
            found = False
            for choice in itertools.product((0, 1), repeat=len(pos)):
                alt = ref["a"][r, sl].copy()
                for p, c in zip(pos, choice):
                    alt[p] = (a_lo if c == 0 else a_hi)[r, q * group + p]
                c_alt, s_alt, _ = O.quant_act(alt[None, :], group)
                if np.array_equal(got_c, c_alt[0]) and got_s == s_alt[0, 0]:
                    found = True
                    break
            bad += not found
    return gpu_vals.size, int(amb.sum()), bad


def check_workspace(ws, plan, I, x64, w13_64, ids, tw, wdtype, weight_on_input=False, clamp_limit=0.0,
                    rows_subset=None):
    """Map the workspace intermediate rows to (token, expert, weight) through
    the sorted ids and compare each expert's rows with the oracle.  Returns
    (compared, near-boundary, mismatches, rows checked)."""
    T, k = ids.shape
    R = T * k
    sorted_ids, vals, scales = read_intermediate(ws, plan, I, wdtype)
    rows = np.nonzero(sorted_ids < R)[0]
    rows = rows[rows < vals.shape[0]]
    if rows_subset is not None:
        rows = rows[rows_subset(rows)]
    f = sorted_ids[rows]
    t, j = f // k, f % k
    e = ids[t, j]
    assert np.all(e >= 0)
    fp8 = wdtype != "bf16"
    n = amb = bad = 0
    for ex in np.unique(e):
        sel = e == ex
        w13e = w13_64(ex) if callable(w13_64) else w13_64[ex]
        ref = O.expert_intermediate(x64, w13e, t[sel], tw[t[sel], j[sel]].astype(np.float64), fp8=fp8,
                                    group=group_of(wdtype), weight_on_input=weight_on_input,
                                    clamp_limit=clamp_limit if clamp_limit > 0 else None)
        gv = vals[rows[sel]]
        gs = scales[rows[sel]] if scales is not None else None
        c, a, b = compare_rows(gv, gs, ref, wdtype, clamp_limit)
        n, amb, bad = n + c, amb + a, bad + b
    return n, amb, bad, len(rows)
