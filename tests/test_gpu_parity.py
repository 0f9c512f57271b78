"""GPU parity of the HIP path against the oracle, through the C ABI.

Routing ids, alignment buffers and fp8 activation codes/scales are compared
bit-exactly; layer outputs with the rule in tests/gpu_util.py.  Workloads are
the seeded configurations of moe_layer_amd.workloads (full sizes, with sampled
oracle rows where the whole layer would take the oracle minutes), plus edge
cases: ragged and tiny shapes, invalid and duplicate ids, empty experts.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle as O
from moe_layer_amd import ops
from moe_layer_amd.workloads import CONFIGS, Workload

from gpu_util import (TAU, bits_to_bf16, compare_output, dev, layer_for, log, oracle_tokens,
                      route_weight_tol, routing, run_forward)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------- routing ---

def _check_route(lg: np.ndarray, k: int, renormalize=True):
    lg_t = torch.from_numpy(lg).to(dev())
    ids, w = ops.moe_route(lg_t, k, renormalize)
    ids, w = ids.cpu().numpy(), w.cpu().numpy().astype(np.float64)
    ids_o, w_o = O.route(lg, k, renormalize)
    np.testing.assert_array_equal(ids, ids_o)
    assert np.all(np.abs(w - w_o) <= route_weight_tol(lg, ids_o, w_o)), np.max(np.abs(w - w_o) / w_o)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "skew"])
def test_route_workloads(name):
    cfg = CONFIGS[name]
    log(f"route {name}")
    _check_route(Workload(cfg).logits(), cfg.topk)


# E across the router's experts-per-lane instances (64, 128, 256, 512, 1024) and their edges
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (3, 7, 2), (257, 64, 8), (100, 65, 64), (9, 128, 8), (9, 129, 8),
                                   (33, 256, 8), (6, 257, 8), (4, 512, 8), (4, 513, 16), (17, 1024, 64),
                                   (5, 1000, 3)])
@pytest.mark.parametrize("renormalize", [True, False])
def test_route_ties_and_shapes(T, E, k, renormalize):
    rng = np.random.default_rng(T * E + k)
    lg = rng.integers(-4, 5, size=(T, E)).astype(np.float32)          # heavy ties
    _check_route(lg, k, renormalize)
    lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    _check_route(lg, k, renormalize)


# --------------------------------------------------------------- alignment ---

def _check_align(ids: np.ndarray, E: int, B: int):
    a = ops.moe_align(torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev()), E, B)
    o = O.align(ids, E, B)
    np.testing.assert_array_equal(a["sorted_token_ids"].cpu().numpy(), o["sorted_token_ids"])
    np.testing.assert_array_equal(a["expert_ids"].cpu().numpy(), o["expert_ids"])
    assert int(a["num_tokens_post_padded"].item()) == o["num_tokens_post_padded"]
    np.testing.assert_array_equal(a["inv"].cpu().numpy(), o["inv"])


# slot counts across the one-wave alignment's batch instances (64, 128, 256 slots) and their edges
@pytest.mark.parametrize("T,k,E,B", [(1, 1, 1, 1), (3, 2, 3, 4), (8, 8, 32, 16), (13, 5, 32, 16), (16, 8, 128, 16),
                                     (43, 3, 20, 8), (32, 8, 64, 16), (257, 1, 16, 4), (7, 3, 5, 64),
                                     (1024, 8, 256, 32), (4096, 8, 128, 64), (999, 5, 1024, 16),
                                     (50, 4, 9, 1024), (2000, 64, 40, 7)])
def test_align_random_ids(T, k, E, B):
    rng = np.random.default_rng(T + E + B)
    ids = rng.integers(-2, E + 2, size=(T, k))      # invalid ids and duplicates included
    _check_align(ids, E, B)


@pytest.mark.parametrize("name,B", [("decode", 16), ("prefill", 64), ("fp8", 32), ("skew", 64), ("skew", 16)])
def test_align_workloads(name, B):
    cfg = CONFIGS[name]
    ids, _, _ = routing(cfg)
    _check_align(ids, cfg.E, B)


@pytest.mark.parametrize("T,k,E,B", [(100, 8, 64, 16), (256, 8, 64, 16), (4096, 8, 128, 64), (4096, 8, 128, 256),
                                     (8192, 8, 256, 16), (3000, 3, 5, 16), (2000, 64, 40, 7), (999, 5, 1024, 16)])
def test_align_ws_multi_workgroup(T, k, E, B):
    """moe_align_ws (many workgroups above 8192 slots, one up to it) gives the
    oracle's alignment bit for bit, inverse permutation included, also on a
    scratch buffer poisoned with 0xFF bytes."""
    rng = np.random.default_rng(T * 7 + E + B)
    ids = rng.integers(-2, E + 2, size=(T, k))
    ids[: T // 4, 0] = rng.integers(0, max(1, E // 16), size=T // 4)   # skewed load
    ids_t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev())
    need = ops.moe_align_scratch_bytes(T, k, E)
    scratch = torch.full((max(need, 256),), 0xFF, dtype=torch.uint8, device=dev())
    a = ops.moe_align_ws(ids_t, E, B, scratch=scratch)
    o = O.align(ids, E, B)
    np.testing.assert_array_equal(a["sorted_token_ids"].cpu().numpy(), o["sorted_token_ids"])
    np.testing.assert_array_equal(a["expert_ids"].cpu().numpy(), o["expert_ids"])
    assert int(a["num_tokens_post_padded"].item()) == o["num_tokens_post_padded"]
    np.testing.assert_array_equal(a["inv"].cpu().numpy(), o["inv"])


def test_align_empty_experts_worked_example():
    _check_align(np.array([[3, 1], [1, 3]]), 4, 2)


@pytest.mark.parametrize("T,k,E,B", [(16, 8, 128, 16), (255, 8, 64, 32), (256, 8, 64, 32), (1024, 8, 256, 32),
                                     (1000, 7, 1024, 64), (4096, 8, 128, 256), (8192, 8, 256, 256),
                                     (3000, 3, 5, 16)])
def test_forward_alignment_buffers(T, k, E, B):
    """The alignment moe_forward leaves in its workspace (one workgroup up to
    8192 slots, several above) equals the oracle's, bit for bit."""
    from moe_layer_amd.workloads import Config
    cfg = Config("align", T, E, 256, 128, k, "bf16", "given")
    layer = layer_for(cfg)
    rng = np.random.default_rng(T * k + E)
    ids = rng.integers(-1, E + 1, size=(T, k)).astype(np.int32)     # invalid and duplicate ids
    ids[: T // 3] = rng.integers(0, max(1, E // 8), size=(T // 3, k))  # skewed load
    tw = np.ones((T, k), np.float32)
    x = np.zeros((T, 256), np.uint16)
    out, ws, (xt, ids_t, tw_t) = run_forward(layer, x, ids, tw, block_m=B,
                                             path=ops.MOE_PATH_LARGE_M if B == 256 else ops.MOE_PATH_SMALL_M)
    p = ops.moe_plan(ops.forward_args(xt, layer.w13, layer.w2, ids_t, tw_t, None, None, out,
                                      ops.MOE_PATH_LARGE_M if B == 256 else ops.MOE_PATH_SMALL_M, B))
    o = O.align(ids, E, B)
    w = ws.cpu().numpy()

    def buf(off, n):
        return w[off: off + 4 * n].view(np.int32)

    np.testing.assert_array_equal(buf(p["off_sorted_ids"], p["capacity"]), o["sorted_token_ids"])
    np.testing.assert_array_equal(buf(p["off_expert_ids"], p["num_blocks"]), o["expert_ids"])
    assert int(buf(p["off_num_post_padded"], 1)[0]) == o["num_tokens_post_padded"]


# ------------------------------------------------------ fp8 activation quant ---

def test_quant_act_bit_exact():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((300, 1024)) * 0.1).astype(np.float32)
    x[0] = 0.0                                   # all-zero rows: scale from the 1e-10 floor
    x[1] *= 1e-6                                 # e4m3 subnormal codes
    x[2] *= 1e4
    x[3, :128] = 1.75                            # the amax=1.75 boundary case
    x[4, ::2] = -x[4, ::2]
    x = np.concatenate([x, Workload(CONFIGS["fp8"]).x_f32()[:64, :1024]])
    bits = torch.from_numpy(x).to(torch.bfloat16)
    codes, scales = ops.moe_quant_act(bits.to(dev()))
    xo = bits.to(torch.float64).numpy()
    c_o, s_o, _ = O.quant_act(xo)
    np.testing.assert_array_equal(scales.cpu().numpy().astype(np.float64), s_o)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_o)


def test_quant_act_mx_bit_exact():
    """MXFP8 activation quantisation: e4m3 codes and E8M0 scale bytes of every
    32-column group equal the oracle's, bit for bit."""
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((200, 512)) * 0.1).astype(np.float32)
    x[0] = 0.0
    x[1, :32] *= 1e-6
    x[2, 32:64] *= 1e4
    x[3, :32] = 1.75
    x[5] *= np.repeat(np.exp(rng.uniform(-10, 10, 16)), 32).astype(np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16)
    codes, scales = ops.moe_quant_act_mx(bits.to(dev()))
    c_o, s_o, _ = O.quant_act(bits.to(torch.float64).numpy(), 32)
    np.testing.assert_array_equal(scales.cpu().numpy(), O.e8m0_encode(s_o))
    np.testing.assert_array_equal(codes.cpu().numpy(), c_o)


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
@pytest.mark.parametrize("T", [16, 300, 1100])
def test_forward_input_quant_in_workspace(wdtype, T):
    """The layer input's e4m3 codes and scales that moe_forward leaves in its
    workspace equal the oracle's bit for bit: quantised by the other
    workgroups of the alignment's launch up to 8192 slots (16 tokens: the
    one-wave alignment, 300: the one-workgroup form), by their own kernel
    above (1100 tokens x 8 slots)."""
    from moe_layer_amd.workloads import Config
    k, H = 8, 512
    cfg = Config("xq_" + wdtype, T, 8, H, 256, k, wdtype, "given")
    layer = layer_for(cfg)
    layer.ensure(range(8))
    rng = np.random.default_rng(T)
    x = (rng.standard_normal((T, H)) * 0.1).astype(np.float32)
    x[0] = 0.0                                   # all-zero groups: the 1e-10 floor
    x[1, :64] *= 1e-6                            # e4m3 subnormal codes
    x[2, 128:256] *= 1e4
    x[3, :128] = 1.75                            # the amax = 1.75 boundary
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids = rng.integers(0, 8, size=(T, k)).astype(np.int32)
    tw = np.full((T, k), 1.0 / k, np.float32)
    out, ws, (xt, ids_t, tw_t) = run_forward(layer, bits, ids, tw)
    p = ops.moe_plan(ops.forward_args(xt, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2, out))
    assert (T * k <= 8192) == (ops.moe_align_scratch_bytes(T, k, 8) == 0)
    w = ws.cpu().numpy()
    group = 32 if wdtype == "mxfp8" else 128
    c_o, s_o, _ = O.quant_act(bits_to_bf16(bits).to(torch.float64).numpy(), group)
    np.testing.assert_array_equal(w[p["off_xq"]: p["off_xq"] + T * H].reshape(T, H), c_o)
    if wdtype == "mxfp8":
        xs = w[p["off_xs"]: p["off_xs"] + T * (H // 32)].reshape(T, H // 32)
        np.testing.assert_array_equal(xs, O.e8m0_encode(s_o))
    else:
        xs = w[p["off_xs"]: p["off_xs"] + 4 * T * (H // 128)].view(np.float32).reshape(T, H // 128)
        np.testing.assert_array_equal(xs.astype(np.float64), s_o)


# ----------------------------------------------------------------- forward ---

def _forward_case(cfg, tokens=None, **kw):
    """Run route (if the workload routes from logits) + forward on the GPU and
    compare with the oracle on ``tokens`` (all when None)."""
    wl = Workload(cfg)
    ids_o, tw_o, lg = routing(cfg)
    if lg is not None:
        ids_t, tw_t = ops.moe_route(torch.from_numpy(lg).to(dev()), cfg.topk)
        ids = ids_t.cpu().numpy()
        np.testing.assert_array_equal(ids, ids_o)
        tw32 = tw_t.cpu().numpy()
    else:
        ids, tw32 = ids_o, tw_o.astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(np.unique(ids))
    log(f"forward {cfg.name} T={cfg.T} {cfg.wdtype} {kw}")
    out, ws, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw32, **kw)
    gpu = out.to(torch.float64).cpu().numpy()
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    o = oracle_tokens(layer, wl.x_exact(), ids_o, tw_o, tokens, kw.get("weight_on_input", False),
                      kw.get("clamp_limit", 0.0))
    excess, raw, floor = compare_output(gpu[tokens], o)
    log(f"  excess/RMS={excess:.3e} raw max/RMS={raw:.3e} bf16 floor/RMS={floor:.3e}")
    assert np.all(np.isfinite(gpu))
    assert excess <= TAU[cfg.wdtype], (excess, raw)
    return out, ws


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("block_m", [0, 16, 32, 64])
def test_forward_tiny(wdtype, block_m):
    _forward_case(replace(CONFIGS["tiny"], wdtype=wdtype), block_m=block_m)


def test_forward_decode():
    _forward_case(CONFIGS["decode"])


def test_forward_fp8_workload():
    _forward_case(CONFIGS["fp8"])


def test_forward_mxfp8_workload():
    _forward_case(CONFIGS["mxfp8"])


def test_forward_prefill_sampled():
    rng = np.random.default_rng(1)
    _forward_case(CONFIGS["prefill"], tokens=np.sort(rng.choice(4096, 192, replace=False)))


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_forward_skew_small_batches(T):
    _forward_case(CONFIGS["skew"].with_tokens(T))


def test_forward_skew_full_sampled():
    rng = np.random.default_rng(2)
    _forward_case(CONFIGS["skew"], tokens=np.sort(rng.choice(8192, 64, replace=False)))


def test_forward_tiny_large_path():
    _forward_case(CONFIGS["tiny"], path=ops.MOE_PATH_LARGE_M)


def test_forward_ragged_large_path():
    """The LDS-tiled path on an odd token count, E not a power of two, blocks
    whose last 32-row sub-tiles are partly or wholly padding, invalid and
    duplicate ids."""
    from moe_layer_amd.workloads import Config
    cfg = Config("ragged_large", 301, 5, 512, 384, 3, "bf16", "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(6)
    ids = rng.integers(0, 5, size=(301, 3)).astype(np.int32)
    ids[0, 1] = ids[0, 0]
    ids[1, 2] = -1
    ids[2, 0] = 5
    ids[10:200, 0] = 3                      # one hot expert with several full blocks
    tw = rng.random((301, 3)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(range(5))
    out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, path=ops.MOE_PATH_LARGE_M)
    gpu = out.to(torch.float64).cpu().numpy()
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(301))
    excess, raw, _ = compare_output(gpu, o)
    log(f"ragged large: excess/RMS={excess:.3e} raw={raw:.3e}")
    assert excess <= TAU["bf16"]


@pytest.mark.parametrize("variant", ["plain", "on_input", "clamp"])
def test_forward_large_path_short_tail_blocks(variant):
    """The LDS-tiled path where an expert's last 256-row block holds 1, 32, 33
    or 64 rows (taken by the workgroup of the expert's previous block as token
    rows 256..319), 65 rows (a block of its own), a three-block expert whose
    third block is short, an expert of exactly one full block and a small one;
    every token compared with the oracle, for the plain layer and the layer
    variants (their epilogues run on the taken rows too)."""
    kw = {} if variant == "plain" else _VARIANTS[variant]
    from moe_layer_amd.workloads import Config
    counts = [257, 288, 289, 320, 321, 576, 256, 5]
    k = 2
    T = sum(counts) // k
    cfg = Config("short_tails", T, len(counts), 512, 384, k, "bf16", "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(8)
    slots = np.repeat(np.arange(len(counts), dtype=np.int32), counts)
    ids = rng.permutation(slots).reshape(T, k)
    tw = rng.random((T, k)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(range(len(counts)))
    plan = ops.moe_plan(ops.forward_args(None, None, None, None, None, path=ops.MOE_PATH_LARGE_M,
                                         shape=(T, len(counts), 512, 384, k, 0)))
    assert plan["block_m"] == 256
    out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, path=ops.MOE_PATH_LARGE_M, **kw)
    gpu = out.to(torch.float64).cpu().numpy()
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(T),
                      kw.get("weight_on_input", False), kw.get("clamp_limit", 0.0))
    excess, raw, _ = compare_output(gpu, o)
    log(f"short tails {variant}: excess/RMS={excess:.3e} raw={raw:.3e}")
    assert np.all(np.isfinite(gpu))
    assert excess <= TAU["bf16"]


def test_prefill_takes_the_large_path():
    cfg = CONFIGS["prefill"]
    a = ops.forward_args(None, None, None, None, None, shape=(cfg.T, cfg.E, cfg.H, cfg.I, cfg.topk, 0))
    p = ops.moe_plan(a)
    assert p["path"] == ops.MOE_PATH_LARGE_M and p["block_m"] == 256


@pytest.mark.parametrize("path,block_m", [(ops.MOE_PATH_AUTO, 0), (ops.MOE_PATH_AUTO, 32), (ops.MOE_PATH_SMALL_M, 64)])
def test_forward_mid_batch(path, block_m):
    """32 rows per expert: AUTO takes the LDS-tiled path (256-row blocks, most
    32-token sub-tiles padding-only), an explicit 32-row block keeps AUTO on the
    weight-streaming path; every form matches the oracle."""
    from moe_layer_amd.workloads import Config
    cfg = Config("midbatch", 256, 64, 512, 512, 8, "bf16", "logits")
    a = ops.forward_args(None, None, None, None, None, shape=(cfg.T, cfg.E, cfg.H, cfg.I, cfg.topk, 0),
                         path=path, block_m=block_m)
    want = ops.MOE_PATH_LARGE_M if (path, block_m) == (ops.MOE_PATH_AUTO, 0) else ops.MOE_PATH_SMALL_M
    assert ops.moe_plan(a)["path"] == want
    _forward_case(cfg, path=path, block_m=block_m)


def test_forward_prefill_small_path_sampled():
    rng = np.random.default_rng(7)
    _forward_case(CONFIGS["prefill"], tokens=np.sort(rng.choice(4096, 64, replace=False)),
                  path=ops.MOE_PATH_SMALL_M)


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
def test_forward_ragged_shapes(wdtype):
    """Odd token counts, an expert count that is not a power of two, H/I at the
    smallest supported multiples, invalid and duplicate ids."""
    from moe_layer_amd.workloads import Config
    q = 64 if wdtype == "bf16" else 128
    cfg = Config("ragged", 37, 13, 3 * q, 5 * q if wdtype == "bf16" else 2 * q, 3, wdtype, "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(5)
    ids = rng.integers(0, 13, size=(37, 3)).astype(np.int32)
    ids[0, 1] = ids[0, 0]        # duplicate
    ids[1, 2] = -1               # not routed
    ids[2, 0] = 13               # not routed
    ids[3:6] = 4                 # three duplicates
    tw = rng.random((37, 3)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(range(13))
    for bm in (16, 32, 64):
        out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=bm)
        gpu = out.to(torch.float64).cpu().numpy()
        o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(37))
        excess, raw, _ = compare_output(gpu, o)
        log(f"ragged {wdtype} bm={bm}: excess/RMS={excess:.3e} raw={raw:.3e}")
        assert excess <= TAU[wdtype]


@pytest.mark.parametrize("wdtype,H,I", [("bf16", 128, 64), ("bf16", 192, 128), ("fp8", 512, 128), ("fp8", 1024, 256)])
def test_forward_short_k_16_row_blocks(wdtype, H, I):
    """Down GEMMs of 16-row blocks whose K walk is shorter than their LDS ring
    (bf16: one or two stages of 64; block fp8: one or two scale blocks):
    oracle parity, and the same bits as the 32-row register-streaming form."""
    from moe_layer_amd.workloads import Config
    cfg = Config("short_k", 40, 8, H, I, 2, wdtype, "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(11)
    ids = np.stack([rng.permutation(8)[:2] for _ in range(40)]).astype(np.int32)
    ids[:20, 0] = 3                      # one expert with a full 16-row block and more
    ids[:20, 1] = np.where(ids[:20, 1] == 3, 4, ids[:20, 1])
    tw = rng.random((40, 2)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(range(8))
    a, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=16)
    b, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=32)
    assert torch.equal(a, b)
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(40))
    excess, raw, _ = compare_output(a.to(torch.float64).cpu().numpy(), o)
    log(f"short K {wdtype} H={H} I={I}: excess/RMS={excess:.3e} raw={raw:.3e}")
    assert excess <= TAU[wdtype]


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
@pytest.mark.parametrize("H,I", [(8448, 384), (8320, 256)])
def test_forward_fp8_long_k(H, I, wdtype):
    """fp8 with more than 64 K-blocks of 128 (the activation-scale table is
    staged in two chunks), an odd K-block count in GEMM2, and H not a
    multiple of 256 (the narrower GEMM2 tile)."""
    from moe_layer_amd.workloads import Config
    cfg = Config("fp8_longk", 20, 6, H, I, 2, wdtype, "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(H + I)
    ids = np.stack([rng.permutation(6)[:2] for _ in range(20)]).astype(np.int32)
    tw = rng.random((20, 2)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(range(6))
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(20))
    for bm in (16, 32, 64):
        out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=bm)
        gpu = out.to(torch.float64).cpu().numpy()
        excess, raw, _ = compare_output(gpu, o)
        log(f"{wdtype} H={H} I={I} bm={bm}: excess/RMS={excess:.3e} raw={raw:.3e}")
        assert excess <= TAU[wdtype]


# ------------------------------------------------------ self-consistency ---

def _layer_inputs(cfg):
    wl = Workload(cfg)
    ids, tw, lg = routing(cfg)
    layer = layer_for(cfg)
    layer.ensure(np.unique(ids))
    return wl, layer, ids.astype(np.int32), tw.astype(np.float32)


@pytest.mark.parametrize("name,wdtype", [("tiny", "bf16"), ("tiny", "fp8"), ("tiny", "mxfp8"), ("decode", "bf16"),
                                         ("fp8", "fp8"), ("mxfp8", "mxfp8")])
def test_block_m_invariance_bitwise(name, wdtype):
    """Every output element is accumulated over K in the same order whatever the
    block size, so the output is bit-identical across block_m."""
    cfg = replace(CONFIGS[name], wdtype=wdtype)
    wl, layer, ids, tw = _layer_inputs(cfg)
    ref = None
    for bm in (16, 32, 64):
        out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=bm)
        if ref is None:
            ref = out.clone()
        else:
            assert torch.equal(out, ref), f"block_m={bm}"


def test_block_m_invariance_skew_full_blocks():
    """64 tokens of the skewed layer: its hot experts fill whole 16-row blocks,
    so the down GEMM of 16-row blocks (weights through LDS) also loads the
    blocks' second 8-row token group; the output is bit-identical to that of
    the 32- and 64-row blocks (register-streaming down GEMM)."""
    cfg = CONFIGS["skew"].with_tokens(64)
    wl, layer, ids, tw = _layer_inputs(cfg)
    assert np.bincount(ids.ravel(), minlength=cfg.E).max() > 8
    ref = None
    for bm in (16, 32, 64):
        out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=bm)
        if ref is None:
            ref = out.clone()
        else:
            assert torch.equal(out, ref), f"block_m={bm}"


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
def test_rotated_k_walk_parity_and_block_m_invariance(wdtype):
    """64 tokens of the fp8 / MXFP8 layer (2 routed rows per expert: GEMM1's
    rotated K walk is on, 32 K-steps): oracle parity, and the same bits for
    block sizes 16, 32 and 64 (the walk's start depends on the expert and the
    column tile only)."""
    cfg = CONFIGS[wdtype].with_tokens(64)
    _forward_case(cfg, tokens=np.arange(0, 64, 3))
    wl, layer, ids, tw = _layer_inputs(cfg)
    ref = None
    for bm in (16, 32, 64):
        out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=bm)
        if ref is None:
            ref = out.clone()
        else:
            assert torch.equal(out, ref), f"block_m={bm}"


@pytest.mark.parametrize("T", [256, 512])
def test_fp8_16_row_blocks_lds_down_gemm(T):
    """256 and 512 tokens of the fp8 layer on 16-row blocks (the down GEMM
    streams W2 through LDS, 512 output rows per workgroup): oracle parity on
    sampled tokens, and the same bits as the register-streaming down GEMM of
    32-row blocks."""
    cfg = CONFIGS["fp8"].with_tokens(T)
    _forward_case(cfg, tokens=np.arange(0, T, 37))
    wl, layer, ids, tw = _layer_inputs(cfg)
    a, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=16)
    b, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=32)
    assert torch.equal(a, b)


def test_pack_mx_scales_layout():
    """moe_pack_mx_scales against its definition written as a numpy reshape:
    packed[((e*rows/16 + t)*K/128 + s)*64 + g*16 + r] = scales[e, 16t + r, 4s + g]."""
    rng = np.random.default_rng(9)
    for E, rows, K in [(1, 16, 128), (3, 48, 384), (2, 512, 4096)]:
        sc = rng.integers(0, 256, size=(E, rows, K // 32), dtype=np.uint8)
        want = sc.reshape(E, rows // 16, 16, K // 128, 4).transpose(0, 1, 3, 4, 2).reshape(E, rows, K // 32)
        got = ops.moe_pack_mx_scales(torch.from_numpy(sc).to(dev()))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("name,block_m,variant", [("tiny", 16, "plain"), ("tiny", 32, "plain"), ("tiny", 64, "plain"),
                                                  ("tiny", 16, "both"), ("mxfp8", 0, "plain"), ("mxfp8", 0, "clamp")])
def test_mx_packed_scales_bitwise(name, block_m, variant):
    """The MXFP8 layer with its weight scales in the packed layout gives the
    same bits as with the row-major scales (same values, same arithmetic)."""
    kw = {} if variant == "plain" else _VARIANTS[variant]
    cfg = replace(CONFIGS[name], wdtype="mxfp8")
    wl, layer, ids, tw = _layer_inputs(cfg)
    ref, _, (x, ids_t, tw_t) = run_forward(layer, wl.x_bf16_bits(), ids, tw, block_m=block_m, **kw)
    s13p, s2p = ops.moe_pack_mx_scales(layer.s13), ops.moe_pack_mx_scales(layer.s2)
    out, _ = ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, s13p, s2p, block_m=block_m,
                             mx_packed_scales=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    if name == "tiny":   # the single-launch layer reads the packed scales too
        sync = torch.zeros(ops.MOE_SYNC_WORDS, dtype=torch.int32, device=dev())
        ref16, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, path=ops.MOE_PATH_SMALL_M, block_m=16, **kw)
        dl, _, _, _ = ops.moe_decode_layer(x, layer.w13, layer.w2, ids_t, tw_t, s13p, s2p, sync=sync,
                                           mx_packed_scales=True, **kw)
        torch.cuda.synchronize()
        assert torch.equal(dl, ref16)


@pytest.mark.parametrize("name", ["tiny", "fp8", "mxfp8"])
def test_token_permutation_equivariance(name):
    cfg = CONFIGS[name]
    wl, layer, ids, tw = _layer_inputs(cfg)
    x = wl.x_bf16_bits()
    p = np.random.default_rng(3).permutation(cfg.T)
    out, _, _ = run_forward(layer, x, ids, tw)
    outp, _, _ = run_forward(layer, x[p], ids[p], tw[p])
    assert torch.equal(outp, out[torch.from_numpy(p).to(out.device)])


@pytest.mark.parametrize("name", ["tiny", "decode", "fp8", "mxfp8", "prefill"])
def test_determinism_and_poisoned_workspace(name):
    """Two runs agree bitwise, also when the workspace starts as all-NaN bytes:
    no padding row or unwritten workspace value reaches the output."""
    cfg = CONFIGS[name]
    wl, layer, ids, tw = _layer_inputs(cfg)
    out1, ws, (x, ids_t, tw_t) = run_forward(layer, wl.x_bf16_bits(), ids, tw)
    ws.fill_(0xFF)
    out2, _ = ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


def test_output_guard_bands():
    cfg = CONFIGS["tiny"]
    wl, layer, ids, tw = _layer_inputs(cfg)
    T, H = cfg.T, cfg.H
    buf = torch.full((T + 8, H), 7.0, dtype=torch.bfloat16, device=dev())
    x = bits_to_bf16(wl.x_bf16_bits()).to(dev())
    ids_t = torch.from_numpy(ids).to(dev())
    tw_t = torch.from_numpy(tw).to(dev())
    ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, out=buf[4:4 + T])
    torch.cuda.synchronize()
    assert torch.all(buf[:4] == 7.0) and torch.all(buf[4 + T:] == 7.0)
    ref, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw)
    assert torch.equal(buf[4:4 + T], ref)


def test_plan_reports_the_path_taken():
    cfg = CONFIGS["decode"]
    a = ops.forward_args(None, None, None, None, None, shape=(cfg.T, cfg.E, cfg.H, cfg.I, cfg.topk, 0))
    p = ops.moe_plan(a)
    assert p["path"] == ops.MOE_PATH_SMALL_M and p["block_m"] == 16


# ------------------------------------------------------------ layer variants ---

# A clamp limit that is not a bf16 value (the clamp acts after the bf16
# rounding of gate/up) and that the tiny layer's gate/up values often exceed.
_LIMIT = float(np.float32(0.07))
_VARIANTS = {"on_input": dict(weight_on_input=True), "clamp": dict(clamp_limit=_LIMIT),
             "both": dict(weight_on_input=True, clamp_limit=_LIMIT)}


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("variant", sorted(_VARIANTS))
@pytest.mark.parametrize("block_m", [16, 64])
def test_forward_variants_tiny(wdtype, variant, block_m):
    _forward_case(replace(CONFIGS["tiny"], wdtype=wdtype), block_m=block_m, **_VARIANTS[variant])


@pytest.mark.parametrize("variant", sorted(_VARIANTS))
def test_forward_variants_large_path(variant):
    _forward_case(CONFIGS["tiny"], path=ops.MOE_PATH_LARGE_M, **_VARIANTS[variant])


@pytest.mark.parametrize("name,variant", [("decode", "both"), ("fp8", "clamp"), ("mxfp8", "clamp")])
def test_forward_variants_workloads(name, variant):
    _forward_case(CONFIGS[name], **_VARIANTS[variant])


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
@pytest.mark.parametrize("variant", ["on_input", "both"])
def test_forward_weight_on_input_top1_workload(wdtype, variant):
    """The router weight on the input at the fp8 layer's shape with top-1
    routing (one slot per token carries the weight) and weights spread over
    [0.1, 1)."""
    from moe_layer_amd.workloads import Config
    cfg = Config(f"{wdtype}_top1", 1024, 256, 4096, 256, 1, wdtype, "given")
    wl = Workload(cfg)
    ids, _ = wl.given_routing()
    tw = np.random.default_rng(17).uniform(0.1, 1.0, size=(cfg.T, 1)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(np.unique(ids))
    kw = _VARIANTS[variant]
    out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, **kw)
    gpu = out.to(torch.float64).cpu().numpy()
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(cfg.T),
                      kw.get("weight_on_input", False), kw.get("clamp_limit", 0.0))
    excess, raw, _ = compare_output(gpu, o)
    log(f"{wdtype} top-1 {variant}: excess/RMS={excess:.3e} raw={raw:.3e}")
    assert excess <= TAU[wdtype]


def test_forward_variants_change_the_output():
    """The variants are live on the GPU: each moves the tiny layer's output."""
    cfg = replace(CONFIGS["tiny"], wdtype="bf16")
    base, _ = _forward_case(cfg)
    for v in ("on_input", "clamp"):
        out, _ = _forward_case(cfg, **_VARIANTS[v])
        assert not torch.equal(out, base), v


# ------------------------------------------------- single-launch decode layer ---

def _decode_layer_case(cfg, tokens=None, **kw):
    """moe_decode_layer (routing inside the kernel when the workload routes
    from logits) against moe_route + moe_forward on the GPU (bitwise: the same
    device code) and against the oracle; the barrier buffer must come back
    zero."""
    wl = Workload(cfg)
    ids_o, tw_o, lg = routing(cfg)
    layer = layer_for(cfg)
    layer.ensure(np.unique(ids_o))
    d = dev()
    x = bits_to_bf16(wl.x_bf16_bits()).to(d)
    sync = torch.zeros(ops.MOE_SYNC_WORDS, dtype=torch.int32, device=d)
    log(f"decode layer {cfg.name} T={cfg.T} {cfg.wdtype} {kw}")
    if lg is not None:
        lg_t = torch.from_numpy(lg).to(d)
        out, ids_t, tw_t, _ = ops.moe_decode_layer(x, layer.w13, layer.w2, None, None, layer.s13, layer.s2,
                                                   router_logits=lg_t, topk=cfg.topk, sync=sync, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ids_t.cpu().numpy(), ids_o)
        w = tw_t.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(w - tw_o) <= route_weight_tol(lg, ids_o, tw_o))
        ref_ids, ref_tw = ops.moe_route(lg_t, cfg.topk)
    else:
        ids_t = torch.from_numpy(np.ascontiguousarray(ids_o, dtype=np.int32)).to(d)
        tw_t = torch.from_numpy(tw_o.astype(np.float32)).to(d)
        out, _, _, _ = ops.moe_decode_layer(x, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2, sync=sync,
                                            **kw)
        ref_ids, ref_tw = ids_t, tw_t
    ref, _ = ops.moe_forward(x, layer.w13, layer.w2, ref_ids, ref_tw, layer.s13, layer.s2,
                             path=ops.MOE_PATH_SMALL_M, block_m=16, **kw)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), "decode layer differs from moe_forward"
    assert int(sync.abs().sum()) == 0, sync.cpu().numpy()
    tokens = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    o = oracle_tokens(layer, wl.x_exact(), ids_o, tw_o, tokens, kw.get("weight_on_input", False),
                      kw.get("clamp_limit", 0.0))
    excess, raw, _ = compare_output(out.to(torch.float64).cpu().numpy()[tokens], o)
    log(f"  excess/RMS={excess:.3e} raw max/RMS={raw:.3e}")
    assert excess <= TAU[cfg.wdtype], (excess, raw)
    return out


@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
def test_decode_layer_tiny(wdtype):
    _decode_layer_case(replace(CONFIGS["tiny"], wdtype=wdtype))


def test_decode_layer_decode_workload():
    _decode_layer_case(CONFIGS["decode"])


@pytest.mark.parametrize("T", [1, 4, 16, 32])
def test_decode_layer_skew(T):
    _decode_layer_case(CONFIGS["skew"].with_tokens(T))


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
def test_decode_layer_given_routing(wdtype):
    """fp8 layers at the decode shape with routing handed in (no route phase)."""
    _decode_layer_case(replace(CONFIGS[wdtype], T=16))


@pytest.mark.parametrize("wdtype", ["bf16", "fp8"])
def test_decode_layer_variants(wdtype):
    _decode_layer_case(replace(CONFIGS["tiny"], wdtype=wdtype), **_VARIANTS["both"])


def test_decode_layer_repeated_calls_and_plan():
    """Back-to-back calls on one barrier buffer give the same output and leave
    it zero; the plan reports where the decode layer applies."""
    cfg = CONFIGS["decode"]
    a = ops.forward_args(None, None, None, None, None, shape=(cfg.T, cfg.E, cfg.H, cfg.I, cfg.topk, 0))
    assert ops.moe_plan(a)["decode_layer"] == 1
    a = ops.forward_args(None, None, None, None, None, shape=(64, cfg.E, cfg.H, cfg.I, cfg.topk, 0))
    assert ops.moe_plan(a)["decode_layer"] == 0          # 512 slots: beyond the one-wave alignment
    wl = Workload(cfg)
    _, _, lg = routing(cfg)
    layer = layer_for(cfg)
    layer.ensure(np.unique(routing(cfg)[0]))
    d = dev()
    x = bits_to_bf16(wl.x_bf16_bits()).to(d)
    lg_t = torch.from_numpy(lg).to(d)
    sync = torch.zeros(ops.MOE_SYNC_WORDS, dtype=torch.int32, device=d)
    outs = []
    for _ in range(3):
        out, _, _, _ = ops.moe_decode_layer(x, layer.w13, layer.w2, router_logits=lg_t, topk=cfg.topk, sync=sync)
        outs.append(out)
    torch.cuda.synchronize()
    assert all(torch.equal(o.view(torch.int16), outs[0].view(torch.int16)) for o in outs)
    assert int(sync.abs().sum()) == 0


# ---------------------------------------------------------- extreme shapes ---

@pytest.mark.parametrize("wdtype", ["bf16", "fp8", "mxfp8"])
def test_forward_max_experts_and_topk(wdtype):
    """E = 1024 experts and topk = 64 (the ABI limits) with duplicate and
    unrouted ids; 1280 routed slots take the one-workgroup alignment."""
    from moe_layer_amd.workloads import Config
    cfg = Config("maxek", 20, 1024, 256, 128, 64, wdtype, "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(23)
    ids = rng.integers(0, 1024, size=(20, 64)).astype(np.int32)
    ids[0, :8] = 7                      # one expert taking 8 slots of a token
    ids[1, 5] = -1
    ids[2, 9] = 1024
    tw = rng.random((20, 64)).astype(np.float32) / 64
    layer = layer_for(cfg)
    layer.ensure(np.unique(ids[(ids >= 0) & (ids < 1024)]))
    out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw)
    gpu = out.to(torch.float64).cpu().numpy()
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(20))
    excess, raw, _ = compare_output(gpu, o)
    log(f"E=1024 topk=64 {wdtype}: excess/RMS={excess:.3e} raw={raw:.3e}")
    assert excess <= TAU[wdtype]


def test_forward_single_expert_single_token_and_empty_batch():
    """E = 1, topk = 1, T = 1 (the dense-MLP special case), and T = 0, which
    must leave the output untouched."""
    from moe_layer_amd.workloads import Config
    cfg = Config("e1", 1, 1, 256, 128, 1, "bf16", "given")
    wl = Workload(cfg)
    layer = layer_for(cfg)
    layer.ensure([0])
    ids = np.zeros((1, 1), np.int32)
    tw = np.full((1, 1), 0.75, np.float32)
    out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw)
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(1))
    excess, _, _ = compare_output(out.to(torch.float64).cpu().numpy(), o)
    assert excess <= TAU["bf16"]
    d = dev()
    x0 = torch.empty((0, 256), dtype=torch.bfloat16, device=d)
    sentinel = torch.full((1, 256), 7.0, dtype=torch.bfloat16, device=d)
    out0, _ = ops.moe_forward(x0, layer.w13, layer.w2, torch.empty((0, 1), dtype=torch.int32, device=d),
                              torch.empty((0, 1), dtype=torch.float32, device=d), out=sentinel[:0])
    torch.cuda.synchronize()
    assert out0.shape == (0, 256) and bool((sentinel == 7.0).all())


def test_decode_layer_max_experts_and_topk():
    """The single-launch layer at E = 1024, topk = 64 (256 slots, the one-wave
    alignment's limit), from logits."""
    from moe_layer_amd.workloads import Config
    _decode_layer_case(Config("dl_maxek", 4, 1024, 256, 128, 64, "bf16", "logits"))


# ------------------------------------------- LDS-tiled fp8 / MXFP8 path ---

@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
@pytest.mark.parametrize("variant", ["plain", "on_input", "clamp", "both"])
def test_forward_q_large_path_tiny(wdtype, variant):
    """The fp8 and MXFP8 LDS-tiled kernels (128-row blocks) on the tiny layer,
    plain and with the layer variants."""
    kw = {} if variant == "plain" else _VARIANTS[variant]
    cfg = replace(CONFIGS["tiny"], wdtype=wdtype)
    a = ops.forward_args(None, None, None, None, None, shape=(cfg.T, cfg.E, cfg.H, cfg.I, cfg.topk,
                                                               1 if wdtype == "fp8" else 2),
                         path=ops.MOE_PATH_LARGE_M)
    assert ops.moe_plan(a)["block_m"] == 128
    _forward_case(cfg, path=ops.MOE_PATH_LARGE_M, **kw)


@pytest.mark.parametrize("wdtype", ["fp8", "mxfp8"])
@pytest.mark.parametrize("H,I,variant", [(512, 384, "plain"), (512, 256, "plain"), (768, 128, "plain"),
                                         (512, 256, "both"), (768, 256, "clamp"), (768, 128, "on_input"),
                                         (4352, 256, "plain")])
def test_forward_q_large_path_ragged(wdtype, H, I, variant):
    """Odd token count, E not a power of two, a hot expert with several
    128-row blocks, partly filled 32-row sub-tiles, invalid and duplicate ids,
    K = H = 512 (4 stages) and I = 384 (3 stages: an odd stage count).  With
    I <= 256 the down GEMM keeps the token tile in LDS and walks several
    column tiles per workgroup: H = 512 gives two tiles per workgroup, H = 768
    (three tiles) one, H = 4352 (17 tiles) one, and I = 128 a single K stage
    per tile."""
    from moe_layer_amd.workloads import Config
    kw = {} if variant == "plain" else _VARIANTS[variant]
    cfg = Config("ragged_q", 301, 5, H, I, 3, wdtype, "given")
    wl = Workload(cfg)
    rng = np.random.default_rng(16)
    ids = rng.integers(0, 5, size=(301, 3)).astype(np.int32)
    ids[0, 1] = ids[0, 0]
    ids[1, 2] = -1
    ids[2, 0] = 5
    ids[10:250, 0] = 3
    tw = rng.random((301, 3)).astype(np.float32)
    layer = layer_for(cfg)
    layer.ensure(range(5))
    out, _, _ = run_forward(layer, wl.x_bf16_bits(), ids, tw, path=ops.MOE_PATH_LARGE_M, **kw)
    gpu = out.to(torch.float64).cpu().numpy()
    o = oracle_tokens(layer, wl.x_exact(), ids, tw.astype(np.float64), np.arange(301),
                      weight_on_input=kw.get("weight_on_input", False),
                      clamp_limit=kw.get("clamp_limit", 0.0))
    excess, raw, _ = compare_output(gpu, o)
    log(f"ragged large {wdtype} H={H} I={I} {variant}: excess/RMS={excess:.3e} raw={raw:.3e}")
    assert np.all(np.isfinite(gpu))
    assert excess <= TAU[wdtype]


@pytest.mark.parametrize("name", ["fp8", "mxfp8"])
def test_forward_q_large_path_workload(name):
    """The 1024-token fp8 / MXFP8 layer (32 rows per expert) on the tiled path,
    every token against the oracle."""
    _forward_case(CONFIGS[name], path=ops.MOE_PATH_LARGE_M)


@pytest.mark.parametrize("name", ["fp8", "mxfp8"])
def test_forward_q_large_path_8192_tokens_sampled(name):
    """8192 tokens of the fp8 / MXFP8 layer (256 rows per expert: two 128-row
    blocks each) on the tiled path, sampled tokens against the oracle."""
    rng = np.random.default_rng(21)
    _forward_case(CONFIGS[name].with_tokens(8192), tokens=np.sort(rng.choice(8192, 96, replace=False)),
                  path=ops.MOE_PATH_LARGE_M)


def test_forward_q_large_path_mx_packed_scales_bitwise():
    """The MXFP8 tiled kernels read packed weight scales to the same bits as
    row-major ones."""
    cfg = CONFIGS["mxfp8"].with_tokens(256)
    wl, layer, ids, tw = _layer_inputs(cfg)
    ref, _, (x, ids_t, tw_t) = run_forward(layer, wl.x_bf16_bits(), ids, tw, path=ops.MOE_PATH_LARGE_M)
    s13p, s2p = ops.moe_pack_mx_scales(layer.s13), ops.moe_pack_mx_scales(layer.s2)
    out, _ = ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, s13p, s2p, path=ops.MOE_PATH_LARGE_M,
                             mx_packed_scales=True)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("name", ["fp8", "mxfp8"])
def test_q_large_path_determinism_and_permutation(name):
    """Two runs agree bitwise (the second on an 0xFF-poisoned workspace), and a
    token permutation permutes the output."""
    cfg = CONFIGS[name].with_tokens(512)
    wl, layer, ids, tw = _layer_inputs(cfg)
    x = wl.x_bf16_bits()
    out1, ws, (xt, ids_t, tw_t) = run_forward(layer, x, ids, tw, path=ops.MOE_PATH_LARGE_M)
    ws.fill_(0xFF)
    out2, _ = ops.moe_forward(xt, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2, workspace=ws,
                              path=ops.MOE_PATH_LARGE_M)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)
    p = np.random.default_rng(4).permutation(cfg.T)
    outp, _, _ = run_forward(layer, x[p], ids[p], tw[p], path=ops.MOE_PATH_LARGE_M)
    assert torch.equal(outp, out1[torch.from_numpy(p).to(out1.device)])
