"""Pins of the oracle's number formats and the fp8 group scale.

bf16 and OCP E4M3FN rounding are pinned against exhaustive enumeration of the
formats, their tie rule, and torch's CPU casts (library routines); the
power-of-two scale against the hand-derived worked examples and a brute-force
search over powers of two.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _all_finite_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_bits_to_f64(bits)
    return bits, v[np.isfinite(v)]


def test_bf16_identity_on_every_finite_value():
    _, v = _all_finite_bf16()
    np.testing.assert_array_equal(O.round_bf16(v), v)


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])


def test_bf16_ties_go_to_even():
    _, v = _all_finite_bf16()
    pos = np.unique(v[v > 0])
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2.0                      # exact in fp64
    r = O.round_bf16(mid)
    lo_bits = (lo.astype(np.float32).view(np.uint32) >> 16)
    expect = np.where(lo_bits % 2 == 0, lo, hi)
    np.testing.assert_array_equal(r, expect)
    # just off the tie goes to the nearer neighbour
    np.testing.assert_array_equal(O.round_bf16(np.nextafter(mid, lo)), lo)
    np.testing.assert_array_equal(O.round_bf16(np.nextafter(mid, hi)), hi)


def test_bf16_matches_torch_cast_from_fp32():
    rng = np.random.default_rng(7)
    v = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_bf16(v.astype(np.float64)), ref)


def test_bf16_overflow_and_negative():
    assert O.round_bf16(np.array([3.5e38]))[0] == np.inf
    assert O.round_bf16(np.array([-1.0 - 2 ** -9]))[0] == -1.0


def _all_e4m3_codes():
    codes = np.arange(256).astype(np.uint8)
    v = O.e4m3_decode(codes)
    fin = np.isfinite(v)
    return codes[fin], v[fin]


def test_e4m3_has_254_finite_codes_and_max_448():
    codes, v = _all_e4m3_codes()
    assert len(codes) == 254
    assert v.max() == 448.0 and v.min() == -448.0
    assert np.isnan(O.e4m3_decode(np.array([0x7F, 0xFF], dtype=np.uint8))).all()


def test_e4m3_decode_matches_torch():
    codes = np.arange(256).astype(np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = O.e4m3_decode(codes)
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[fin], ref[fin])


def test_e4m3_encode_decode_roundtrip_every_code():
    codes, v = _all_e4m3_codes()
    np.testing.assert_array_equal(O.round_e4m3(v), v)
    np.testing.assert_array_equal(O.e4m3_encode(v), codes)


def test_e4m3_ties_go_to_even():
    _, v = _all_e4m3_codes()
    pos = np.unique(v[v >= 0])
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2.0
    lo_code = O.e4m3_encode(lo)
    expect = np.where(lo_code % 2 == 0, lo, hi)
    np.testing.assert_array_equal(O.round_e4m3(mid), expect)
    np.testing.assert_array_equal(O.round_e4m3(-mid), -expect)


def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(11)
    v = rng.uniform(-448, 448, 100000).astype(np.float32)
    v[:2000] *= np.float32(2.0 ** -12)         # subnormal range of e4m3
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_e4m3(v.astype(np.float64)), ref)
    ref_codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # every code, values that round to a signed zero included
    np.testing.assert_array_equal(O.e4m3_encode(O.round_e4m3(v.astype(np.float64))), ref_codes)


def test_signed_zeros_keep_their_sign():
    """A cast keeps the sign of zero, also for values that round to zero:
    -0.0 and -2^-11 give the negative-zero codes (e4m3 0x80, bf16 0x8000), as
    torch's casts do."""
    v = np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), -(2.0 ** -10)], np.float32)
    ref_e4m3 = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(O.round_e4m3(v.astype(np.float64))), ref_e4m3)
    assert list(ref_e4m3[:4]) == [0x00, 0x80, 0x00, 0x80]
    tiny = np.array([0.0, -0.0, -(2.0 ** -140)], np.float32)
    ref_bf16 = torch.from_numpy(tiny).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = O.round_bf16(tiny.astype(np.float64))
    np.testing.assert_array_equal(np.signbit(ours), (ref_bf16 & 0x8000) != 0)
    np.testing.assert_array_equal(ours, O.bf16_bits_to_f64(ref_bf16))


def test_fl32_is_correctly_rounded_multiply():
    rng = np.random.default_rng(3)
    a = rng.standard_normal(10000).astype(np.float32)
    b = rng.standard_normal(10000).astype(np.float32)
    np.testing.assert_array_equal(O.fl32(a.astype(np.float64) * b.astype(np.float64)),
                                  (a * b).astype(np.float64))


def test_pow2_ceil_brute_force():
    rng = np.random.default_rng(5)
    v = np.exp(rng.uniform(-60, 60, 5000))
    v = np.concatenate([v, 2.0 ** np.arange(-60, 60)])
    got = O.pow2_ceil(v)
    for x, g in zip(v, got):
        n = -200
        while 2.0 ** n < x:
            n += 1
        assert g == 2.0 ** n


@pytest.mark.parametrize("case", GOLDEN["quant"])
def test_group_scale_worked_examples(case):
    s = O.fp8_group_scale(np.array([case["amax"]]))[0]
    assert s == case["scale"]
    if "value" in case:
        q = O.round_e4m3(np.clip(np.array([case["value"]]) / s, -448, 448))
        assert O.e4m3_encode(q)[0] == case["code"]
        assert q[0] * s == case["dequant"]


def test_quant_act_bound_and_scale_range():
    """|x - s q| <= max(2^-4 |x|, 2^-10 s) elementwise; for normal amax the
    group maximum lands in (224, 448] after scaling."""
    rng = np.random.default_rng(9)
    x = O.round_bf16(rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1))))
    codes, s, deq = O.quant_act(x)
    sf = np.repeat(s, 128, axis=1)
    err = np.abs(x - deq)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sf))
    amax = np.abs(x).reshape(64, 4, 128).max(axis=2)
    ratio = amax / s
    assert np.all(ratio > 224) and np.all(ratio <= 448)
    # codes decode back to the dequantised values
    np.testing.assert_array_equal(O.e4m3_decode(codes) * sf, deq)


def test_quant_act_zero_group():
    codes, s, deq = O.quant_act(np.zeros((1, 128)))
    assert np.all(codes == 0) and np.all(deq == 0)
    assert s[0, 0] == O.pow2_ceil(O.fl32(np.float32(1e-10) * np.float64(np.float32(1 / 448))))


def test_dequant_block_layout():
    codes = np.zeros((256, 384), dtype=np.uint8)
    codes[:, :] = 0x38                       # e4m3 1.0
    scales = np.arange(6, dtype=np.float64).reshape(2, 3) + 1
    w = O.dequant_block(codes, scales)
    assert w[0, 0] == 1 and w[127, 127] == 1 and w[128, 0] == 4 and w[255, 383] == 6 and w[0, 200] == 2


# ------------------------------------------------------------------- MXFP8 ---

def test_e8m0_spec_values():
    """E8M0 is a bare biased exponent: 0x7F is 1.0, 0x00 is 2^-127, 0xFE is
    2^127, 0xFF is NaN (OCP microscaling formats)."""
    d = O.e8m0_decode(np.array([0x7F, 0x00, 0xFE, 0x80, 0x7E, 0xFF]))
    assert d[0] == 1.0 and d[1] == 2.0 ** -127 and d[2] == 2.0 ** 127
    assert d[3] == 2.0 and d[4] == 0.5 and np.isnan(d[5])
    e = np.arange(-127, 128)
    codes = O.e8m0_encode(np.ldexp(1.0, e))
    np.testing.assert_array_equal(codes.astype(np.int64), e + 127)
    with pytest.raises(ValueError):
        O.e8m0_encode(np.array([3.0]))


def test_dequant_mx_matches_element_loop():
    rng = np.random.default_rng(4)
    codes = (rng.integers(0, 256, (6, 96)) & 0x7E).astype(np.uint8)   # finite codes
    scales = rng.integers(100, 150, (6, 3)).astype(np.uint8)
    got = O.dequant_mx(codes, scales)
    for r in range(6):
        for c in range(96):
            v = O.e4m3_decode(np.array([codes[r, c]]))[0]
            assert got[r, c] == v * 2.0 ** (int(scales[r, c // 32]) - 127)


def test_quant_act_group32_bound_and_e8m0_scales():
    """MXFP8 activation groups of 32: the same error bound and scale range as
    the 128 groups, every scale an E8M0-representable power of two."""
    rng = np.random.default_rng(10)
    x = O.round_bf16(rng.standard_normal((32, 256)) * np.exp(rng.uniform(-20, 20, (32, 8)).repeat(32, axis=1)))
    codes, s, deq = O.quant_act(x, 32)
    assert s.shape == (32, 8)
    sf = np.repeat(s, 32, axis=1)
    err = np.abs(x - deq)
    assert np.all(err <= np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * sf))
    amax = np.abs(x).reshape(32, 8, 32).max(axis=2)
    assert np.all(amax / s > 224) and np.all(amax / s <= 448)
    np.testing.assert_array_equal(O.e8m0_decode(O.e8m0_encode(s)), s)
    # finer groups never raise the error of a group of 128 that contains them
    _, _, deq128 = O.quant_act(x, 128)
    assert np.abs(x - deq).max() <= np.abs(x - deq128).max()
