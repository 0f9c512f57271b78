"""Pins of the oracle's layer forward.

* E=1, k=1 in pure mode equals the dense SwiGLU MLP computed with torch's
  fp64 CPU ops (silu, matmul);
* a dense masked evaluation sum_e G[t,e] FFN_e(x_t), evaluated token by token
  with scalar loops (a different algorithm from the oracle's per-expert
  gather), agrees in both modes, bf16 and fp8, with duplicate and invalid ids;
* hand-derived worked examples pin the rounding points;
* invariants: linear in the router weights, token-permutation equivariant,
  zero weights give zero, a duplicated id equals the summed weight.
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
