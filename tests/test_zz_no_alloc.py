"""moe_forward_noalloc (the library's static per-GPU workspace, for callers
that cannot allocate) against moe_forward through the C ABI: the same kernels,
so the outputs must be equal bit for bit, on two calls in a row, the second
with a smaller input (the array keeps the first call's contents)."""
from dataclasses import replace

import numpy as np
import pytest
import torch

from moe_layer_amd import ops
from moe_layer_amd.workloads import CONFIGS, Workload

from gpu_util import bits_to_bf16, dev, layer_for, log, routing

pytestmark = pytest.mark.gpu


def _inputs(cfg, T):
    wl = Workload(cfg)
    ids, tw, _ = routing(cfg)
    layer = layer_for(cfg)
    layer.ensure(np.unique(ids[:T]))
    d = dev()
    x = bits_to_bf16(wl.x_bf16_bits()[:T]).to(d)
    ids_t = torch.from_numpy(np.ascontiguousarray(ids[:T], dtype=np.int32)).to(d)
    tw_t = torch.from_numpy(np.ascontiguousarray(tw[:T], dtype=np.float32)).to(d)
    return layer, x, ids_t, tw_t


@pytest.mark.parametrize("name,wdtype,sizes", [("tiny", "bf16", (64, 5)), ("tiny", "fp8", (64, 7)),
                                               ("tiny", "mxfp8", (64, 3)), ("decode", "bf16", (16, 4))])
def test_noalloc_equals_moe_forward(name, wdtype, sizes):
    cfg = replace(CONFIGS[name], wdtype=wdtype)
    for T in sizes:
        layer, x, ids_t, tw_t = _inputs(cfg, T)
        a = ops.forward_args(x, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2)
        assert ops.moe_forward_workspace(a) <= ops.MOE_NOALLOC_MAX_BYTES
        ref, _ = ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2)
        out = torch.full_like(ref, 7.0)
        a.out = ops._ptr(out)
        st = ops.lib().moe_forward_noalloc(ops.C.byref(a), ops._stream(x.device))
        assert st == ops.MOE_OK, ops.status_string(st)
        torch.cuda.synchronize()
        log(f"noalloc {name} {wdtype} T={T}: workspace {ops.moe_forward_workspace(a)} bytes")
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), (name, wdtype, T)


def test_noalloc_binding_and_variants():
    cfg = CONFIGS["tiny"]
    layer, x, ids_t, tw_t = _inputs(cfg, 64)
    for kw in ({}, dict(weight_on_input=True, clamp_limit=0.07), dict(block_m=64)):
        ref, _ = ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, **kw)
        out = ops.moe_forward_noalloc(x, layer.w13, layer.w2, ids_t, tw_t, **kw)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), kw
