"""Pins of the oracle's layer forward.

* E=1, k=1 in pure mode equals the dense SwiGLU MLP computed with torch's
  fp64 CPU ops (silu, matmul);
* a dense masked evaluation sum_e G[t,e] FFN_e(x_t), evaluated token by token
  with scalar loops (a different algorithm from the oracle's per-expert
  gather), agrees in both modes, bf16 and fp8, with duplicate and invalid ids;
* hand-derived worked examples pin the rounding points;
* invariants: linear in the router weights, token-permutation equivariant,
  zero weights give zero, a duplicated id equals the summed weight;
* the layer variants (router weight on the input, SwiGLU clamp limit) against
  slot-by-slot scalar loops, a dense MLP of the scaled input, hand-derived
  examples and their special cases (unit weights, a limit nothing reaches).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _bf16(a):
    return O.round_bf16(np.asarray(a, dtype=np.float64))


def _layer(T, E, H, I, k, seed, fp8=False):
    rng = np.random.default_rng(seed)
    x = _bf16(rng.standard_normal((T, H)) * 0.1)
    if fp8 == "mx":
        w13 = O.dequant_mx(rng.integers(0, 256, (E, 2 * I, H)).astype(np.uint8) & 0x77,
                           rng.integers(110, 125, (E, 2 * I, H // 32)).astype(np.uint8))
        w2 = O.dequant_mx(rng.integers(0, 256, (E, H, I)).astype(np.uint8) & 0x77,
                          rng.integers(110, 125, (E, H, I // 32)).astype(np.uint8))
    elif fp8:
        w13 = O.dequant_block(rng.integers(0, 256, (E, 2 * I, H)).astype(np.uint8) & 0x77,
                              np.abs(rng.standard_normal((E, 2 * I // 128, H // 128))) * 0.01)
        w2 = O.dequant_block(rng.integers(0, 256, (E, H, I)).astype(np.uint8) & 0x77,
                             np.abs(rng.standard_normal((E, H // 128, I // 128))) * 0.01)
    else:
        w13 = _bf16(rng.standard_normal((E, 2 * I, H)) / np.sqrt(H))
        w2 = _bf16(rng.standard_normal((E, H, I)) / np.sqrt(I))
    ids = rng.integers(0, E, (T, k))
    tw = rng.random((T, k))
    return x, w13, w2, ids, tw


def test_E1_k1_pure_is_dense_swiglu_mlp():
    x, w13, w2, _, _ = _layer(9, 1, 64, 48, 1, 0)
    ids = np.zeros((9, 1), dtype=np.int64)
    tw = np.full((9, 1), 0.7)
    got = O.forward(x, w13, w2, ids, tw, mode="pure")
    xt = torch.from_numpy(x)
    gate = torch.from_numpy(w13[0, :48])
    up = torch.from_numpy(w13[0, 48:])
    down = torch.from_numpy(w2[0])
    ref = 0.7 * (torch.nn.functional.silu(xt @ gate.T) * (xt @ up.T)) @ down.T
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)


def _dense_masked(x, w13, w2, ids, tw, method, fp8, group=128):
    """out[t] = sum_e G[t,e] * FFN_e(x_t), G[t,e] = sum of tw[t,j] over j with
    ids[t,j] == e.  Scalar loops over tokens, experts and features."""
    T, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    out = np.zeros((T, H))
    for t in range(T):
        xt = x[t]
        if fp8 and method:
            xt = O.quant_act(xt[None, :], group)[2][0]
        for e in range(E):
            G = sum(tw[t, j] for j in range(ids.shape[1]) if ids[t, j] == e)
            if G == 0:
                continue
            act = np.empty(I)
            for i in range(I):
                g = float(np.dot(w13[e, i], xt))
                u = float(np.dot(w13[e, I + i], xt))
                if method:
                    g, u = _bf16(g)[()], _bf16(u)[()]
                    s = _bf16(g / (1.0 + np.exp(-g)))[()]
                    act[i] = _bf16(s * u)[()]
                else:
                    act[i] = g / (1.0 + np.exp(-g)) * u
            if fp8 and method:
                act = O.quant_act(act[None, :], group)[2][0]
            for h in range(H):
                out[t, h] += G * float(np.dot(w2[e, h], act))
    return out


@pytest.mark.parametrize("mode", ["method", "pure"])
@pytest.mark.parametrize("fp8", [False, True, "mx"])
def test_matches_dense_masked_evaluation(mode, fp8):
    if fp8:
        T, E, H, I, k = 5, 3, 128, 128, 2
    else:
        T, E, H, I, k = 6, 4, 24, 16, 3
    group = 32 if fp8 == "mx" else 128
    x, w13, w2, ids, tw = _layer(T, E, H, I, k, 1 + bool(fp8), fp8)
    ids[0, 1] = ids[0, 0]          # a duplicate id
    ids[1, 0] = -1                 # an id outside [0, E): not routed
    ids[2, 1] = E
    got = O.forward(x, w13, w2, ids, tw, mode=mode, fp8=bool(fp8), group=group)
    ref = _dense_masked(x, w13, w2, ids, tw, mode == "method", bool(fp8), group)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_mx_groups_quantise_the_intermediate_per_32_columns():
    """Hand-derived: one token, one expert, I = 64.  The intermediate's two
    32-column groups get their own scales: a group of 1.5 values quantises
    exactly, a group whose max is 3.0 maps 3.0 to 384 * 2^-7."""
    H, I = 32, 64
    x = np.zeros((1, H)); x[0, 0] = 1.0
    w13 = np.zeros((1, 2 * I, H))
    w13[0, :I, 0] = 30.0           # gate: silu(30) rounds to 30 in bf16
    w13[0, I:I + 32, 0] = 0.05     # up, group 0: a = bf16(30 * 0.05) = 1.5
    w13[0, I + 32:, 0] = 0.1       # up, group 1: a = 3.0
    w2 = np.zeros((1, H, I)); w2[0, 0, :] = 1.0
    out = O.forward(x, w13, w2, np.array([[0]]), np.array([[1.0]]), fp8=True, group=32)
    # group scales: pow2ceil(1.5/448) = 2^-8 (1.5 -> 384 exactly), pow2ceil(3/448) = 2^-7
    assert out[0, 0] == 32 * 1.5 + 32 * 3.0


@pytest.mark.parametrize("case", [c for c in GOLDEN["forward"] if not c["fp8"]])
def test_worked_examples_bf16(case):
    args = [np.array(case[n], dtype=np.float64) for n in ("x", "w13", "w2")]
    ids, tw = np.array(case["ids"]), np.array(case["tw"])
    m = O.forward(*args, ids, tw, mode="method")
    p = O.forward(*args, ids, tw, mode="pure")
    np.testing.assert_array_equal(m, np.array(case["out_method"]))
    np.testing.assert_allclose(p, np.array(case["out_pure"]), rtol=1e-15)


def test_worked_example_fp8_intermediate():
    case = [c for c in GOLDEN["forward"] if c["fp8"]][0]
    H = I = 128
    x = np.zeros((1, H)); x[0, 0] = 1.0
    w13 = np.zeros((1, 2 * I, H)); w13[0, :I, 0] = 1.0; w13[0, I:, 0] = 2.0
    w2 = np.zeros((1, H, I)); w2[0, 0, 0] = 1.0
    out = O.forward(x, w13, w2, np.zeros((1, 1), int), np.ones((1, 1)), fp8=True)
    assert out[0, 0] == case["out0_method"]
    assert np.all(out[0, 1:] == 0)


def test_invariants():
    T, E, H, I, k = 12, 5, 32, 16, 3
    x, w13, w2, ids, tw = _layer(T, E, H, I, k, 7)
    base = O.forward(x, w13, w2, ids, tw)
    # linear in the router weights
    np.testing.assert_allclose(O.forward(x, w13, w2, ids, 2.5 * tw), 2.5 * base, rtol=1e-13, atol=1e-15)
    tw2 = np.random.default_rng(8).random((T, k))
    np.testing.assert_allclose(O.forward(x, w13, w2, ids, tw + tw2),
                               base + O.forward(x, w13, w2, ids, tw2), rtol=1e-12, atol=1e-14)
    # token permutation equivariance
    p = np.random.default_rng(9).permutation(T)
    np.testing.assert_allclose(O.forward(x[p], w13, w2, ids[p], tw[p]), base[p], rtol=1e-13, atol=1e-15)
    # zero weights give zero
    assert np.all(O.forward(x, w13, w2, ids, np.zeros_like(tw)) == 0)
    # a duplicated id behaves as one slot with the summed weight
    ids_d = ids.copy(); ids_d[:, 1] = ids_d[:, 0]
    tw_d = tw.copy()
    merged_ids = ids_d.copy(); merged_ids[:, 1] = -1
    merged_tw = tw.copy(); merged_tw[:, 0] = tw[:, 0] + tw[:, 1]; merged_tw[:, 1] = 0
    np.testing.assert_allclose(O.forward(x, w13, w2, ids_d, tw_d),
                               O.forward(x, w13, w2, merged_ids, merged_tw), rtol=1e-12, atol=1e-14)


def test_expert_rows_sums_to_forward():
    T, E, H, I, k = 10, 4, 128, 128, 2
    for fp8 in (False, True):
        x, w13, w2, ids, tw = _layer(T, E, H, I, k, 11, fp8)
        full = O.forward(x, w13, w2, ids, tw, fp8=fp8)
        acc = np.zeros_like(full)
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                acc[t] += O.expert_rows(x, w13[e], w2[e], [t], [tw[t, j]], fp8=fp8)[0]
        np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-14)


def test_method_differs_from_pure_by_rounding_only():
    """The rounding points move the output by a few bf16 ulps of the
    intermediate, far below the output scale (a sanity bound, not a pin)."""
    x, w13, w2, ids, tw = _layer(16, 4, 64, 64, 2, 12)
    m = O.forward(x, w13, w2, ids, tw)
    p = O.forward(x, w13, w2, ids, tw, mode="pure")
    rms = np.sqrt(np.mean(p ** 2))
    assert 0 < np.max(np.abs(m - p)) < 0.05 * rms


# ---------------------------------------------------------------------------
# layer variants: router weight on the input, SwiGLU clamp limit
# ---------------------------------------------------------------------------

def _per_slot_loops(x, w13, w2, ids, tw, method, fp8, group=128, weight_on_input=False, clamp_limit=None):
    """out[t] = sum_j FFN_{ids[t,j]}(x_t, tw[t,j]) slot by slot with scalar
    loops over features (a different algorithm from the oracle's per-expert
    gather).  The variants are written out inline."""
    T, H = x.shape
    E, twoI, _ = w13.shape
    I = twoI // 2
    out = np.zeros((T, H))
    for t in range(T):
        xq = x[t]
        if fp8 and method:
            xq = O.quant_act(xq[None, :], group)[2][0]
        for j in range(ids.shape[1]):
            e = ids[t, j]
            if not 0 <= e < E:
                continue
            xin = xq * tw[t, j] if weight_on_input else xq
            act = np.empty(I)
            for i in range(I):
                g = float(np.dot(w13[e, i], xin))
                u = float(np.dot(w13[e, I + i], xin))
                if method:
                    g, u = _bf16(g)[()], _bf16(u)[()]
                if clamp_limit is not None:
                    g = min(g, clamp_limit)
                    u = max(-clamp_limit, min(u, clamp_limit))
                s = g / (1.0 + np.exp(-g))
                act[i] = _bf16(_bf16(s)[()] * u)[()] if method else s * u
            if fp8 and method:
                act = O.quant_act(act[None, :], group)[2][0]
            scale = 1.0 if weight_on_input else tw[t, j]
            for h in range(H):
                out[t, h] += scale * float(np.dot(w2[e, h], act))
    return out


@pytest.mark.parametrize("mode", ["method", "pure"])
@pytest.mark.parametrize("fp8", [False, True, "mx"])
@pytest.mark.parametrize("variant", ["on_input", "clamp", "both"])
def test_variants_match_per_slot_loops(mode, fp8, variant):
    if fp8:
        T, E, H, I, k = 4, 3, 128, 128, 2
    else:
        T, E, H, I, k = 6, 4, 24, 16, 3
    group = 32 if fp8 == "mx" else 128
    x, w13, w2, ids, tw = _layer(T, E, H, I, k, 21 + bool(fp8), fp8)
    x = x * 30.0                   # gate/up values well past the clamp limit
    ids[0, 1] = ids[0, 0]          # a duplicate id
    ids[1, 0] = -1                 # not routed
    on_input = variant in ("on_input", "both")
    limit = 0.7 if variant in ("clamp", "both") else None   # not a bf16 value: rounding comes first
    got = O.forward(x, w13, w2, ids, tw, mode=mode, fp8=bool(fp8), group=group,
                    weight_on_input=on_input, clamp_limit=limit)
    ref = _per_slot_loops(x, w13, w2, ids, tw, mode == "method", bool(fp8), group, on_input, limit)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)
    if limit is not None:          # the clamp is active in this draw
        assert not np.allclose(got, O.forward(x, w13, w2, ids, tw, mode=mode, fp8=bool(fp8), group=group,
                                              weight_on_input=on_input))


def test_weight_on_input_E1_k1_pure_is_dense_mlp_of_scaled_input():
    x, w13, w2, _, _ = _layer(7, 1, 64, 48, 1, 3)
    ids = np.zeros((7, 1), dtype=np.int64)
    tw = np.random.default_rng(4).random((7, 1))
    got = O.forward(x, w13, w2, ids, tw, mode="pure", weight_on_input=True)
    xt = torch.from_numpy(x * tw)
    gate, up, down = (torch.from_numpy(a) for a in (w13[0, :48], w13[0, 48:], w2[0]))
    ref = (torch.nn.functional.silu(xt @ gate.T) * (xt @ up.T)) @ down.T
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_weight_on_input_worked_example():
    """Hand-derived: x = 1, gate weight 2, up weight 3, router weight 0.5.
    On the input: g = 1, u = 1.5; silu(1) = 0.7310586 -> bf16 0.73046875;
    0.73046875 * 1.5 = 1.095703125 -> bf16 (step 2^-7) 1.09375; no weight after
    the down GEMM.  After the down GEMM instead: g = 2, u = 3; silu(2) =
    1.7615942 -> 1.7578125; * 3 = 5.2734375 -> (step 2^-5) 5.28125; * 0.5."""
    x = np.array([[1.0]])
    w13 = np.array([[[2.0], [3.0]]])
    w2 = np.array([[[1.0]]])
    ids, tw = np.array([[0]]), np.array([[0.5]])
    assert O.forward(x, w13, w2, ids, tw, weight_on_input=True)[0, 0] == 1.09375
    assert O.forward(x, w13, w2, ids, tw)[0, 0] == 0.5 * 5.28125


def test_clamp_worked_examples():
    """Hand-derived, L = 7, x = 1, one expert, down weight 1.
    gate 10, up 20: both clamp to 7; silu(7) = 6.99363 -> bf16 (step 2^-5)
    7.0; a = 49.  Without the limit: silu(10) = 9.99955 -> (step 2^-4) 10.0,
    a = 200.  gate 10, up -20: a = -49.  gate -10 stays -10 (the gate is capped
    from above only): silu(-10) = -4.5397869e-4 -> bf16 (step 2^-19)
    -238 * 2^-19; times up 2 -> -238 * 2^-18, exact in bf16."""
    def one(gv, uv, limit):
        w13 = np.array([[[gv], [uv]]])
        return O.forward(np.array([[1.0]]), w13, np.array([[[1.0]]]), np.array([[0]]),
                         np.array([[1.0]]), clamp_limit=limit)[0, 0]
    assert one(10.0, 20.0, 7.0) == 49.0
    assert one(10.0, 20.0, None) == 200.0
    assert one(10.0, -20.0, 7.0) == -49.0
    assert one(-10.0, 2.0, 7.0) == -238 * 2.0 ** -18


def test_variant_special_cases():
    T, E, H, I, k = 8, 4, 32, 16, 2
    x, w13, w2, ids, tw = _layer(T, E, H, I, k, 31)
    base = O.forward(x, w13, w2, ids, tw)
    # unit router weights: the weight's position does not matter
    ones = np.ones_like(tw)
    np.testing.assert_array_equal(O.forward(x, w13, w2, ids, ones, weight_on_input=True),
                                  O.forward(x, w13, w2, ids, ones))
    # a limit beyond every gate/up value changes nothing
    np.testing.assert_array_equal(O.forward(x, w13, w2, ids, tw, clamp_limit=1e30), base)
    # with the weight on the input the layer is no longer linear in the weights
    assert not np.allclose(O.forward(x, w13, w2, ids, 2 * tw, weight_on_input=True),
                           2 * O.forward(x, w13, w2, ids, tw, weight_on_input=True))
    # expert_rows follows the same options
    for on_input, limit in ((True, None), (False, 0.05), (True, 0.05)):
        full = O.forward(x, w13, w2, ids, tw, weight_on_input=on_input, clamp_limit=limit)
        acc = np.zeros_like(full)
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                acc[t] += O.expert_rows(x, w13[e], w2[e], [t], [tw[t, j]], weight_on_input=on_input,
                                        clamp_limit=limit)[0]
        np.testing.assert_allclose(acc, full, rtol=1e-12, atol=1e-14)
