"""The C ABI on the host: every symbol include/moe.h declares is exported, and
the host-only functions (capacity, planning, workspace, validation) behave as
documented.  Every call here either is host-only or fails validation before
any device work, so no GPU is needed."""
import ctypes as C
import os
import re
import subprocess

import pytest

from moe_layer_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

FAKE = 0x7f0000000000          # 256-byte aligned address that is never dereferenced
ODD = FAKE + 2                 # misaligned


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", text)


def test_header_declares_the_binding_exports():
    assert sorted(declared_functions()) == sorted(ops.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ops.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", ops._LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (moe_\w+)$", out, re.M))
    assert set(declared_functions()) == exported


def test_version_and_status_strings():
    assert ops.moe_version() >> 16 == 1
    assert ops.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert ops.status_string(s) != "unknown status"
    assert ops.status_string(123) == "unknown status"


@pytest.mark.parametrize("T,k,E,B", [(3, 2, 3, 4), (16, 8, 128, 16), (4096, 8, 128, 64), (0, 8, 256, 16)])
def test_align_capacity(T, k, E, B):
    assert ops.moe_align_capacity(T, k, E, B) == T * k + E * (B - 1)


def test_align_capacity_errors():
    L = ops.lib()
    assert L.moe_align_capacity(-1, 2, 3, 4) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_capacity(3, 0, 3, 4) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_capacity(3, 2, 0, 4) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_capacity(3, 2, 1025, 4) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_capacity(3, 2, 3, 0) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_capacity(2 ** 28, 64, 1024, 1024) == ops.MOE_ERR_UNSUPPORTED


def _args(T=16, E=128, H=4096, I=1536, k=8, wdtype=0, path=0, block_m=0, ptr=FAKE, scales=True, flags=0,
          clamp_limit=0.0):
    a = ops.forward_args(None, None, None, None, None, shape=(T, E, H, I, k, wdtype), path=path, block_m=block_m,
                         clamp_limit=clamp_limit)
    a.flags = flags
    for f in ("x", "w13", "w2", "topk_ids", "topk_weights", "out"):
        setattr(a, f, ptr)
    if wdtype in (ops.MOE_WDTYPE_FP8_E4M3, ops.MOE_WDTYPE_MXFP8) and scales:
        a.w13_scale = a.w2_scale = FAKE
    return a


@pytest.mark.parametrize("T,E,k,wdtype,expect_bm,expect_path", [
    (16, 128, 8, 0, 16, ops.MOE_PATH_SMALL_M),      # decode: 1 row per expert
    (1024, 256, 8, 1, 128, ops.MOE_PATH_LARGE_M),   # fp8: 32 rows per expert take the tiled path
    (512, 256, 8, 1, 16, ops.MOE_PATH_SMALL_M),     # fp8: 16 rows per expert stream the weights
    (640, 256, 8, 1, 128, ops.MOE_PATH_LARGE_M),    # fp8: 20 rows per expert
    (128, 128, 8, 0, 16, ops.MOE_PATH_SMALL_M),     # 8 rows per expert: weight streaming
    (176, 128, 8, 0, 16, ops.MOE_PATH_SMALL_M),     # 11 rows per expert
    (192, 128, 8, 0, 256, ops.MOE_PATH_LARGE_M),    # 12 rows per expert: LDS-tiled from here on
    (64, 8, 2, 0, 16, ops.MOE_PATH_SMALL_M),        # tiny: 16 rows per expert, too few tiles for the LDS path
    (512, 64, 8, 0, 256, ops.MOE_PATH_LARGE_M),     # 64 rows per expert
    (4096, 128, 8, 0, 256, ops.MOE_PATH_LARGE_M),   # prefill: 256 rows per expert
    (1024, 256, 8, 2, 128, ops.MOE_PATH_LARGE_M),   # MXFP8: 32 rows per expert
    (8192, 256, 8, 2, 128, ops.MOE_PATH_LARGE_M),   # MXFP8: 256 rows per expert
    (2048, 256, 8, 1, 128, ops.MOE_PATH_LARGE_M),   # fp8: 64 rows per expert
    (768, 256, 8, 2, 32, ops.MOE_PATH_SMALL_M),     # MXFP8: 24 rows per expert stream the weights
    (896, 256, 8, 2, 128, ops.MOE_PATH_LARGE_M),    # MXFP8: 28 rows per expert
])
def test_plan_block_size(T, E, k, wdtype, expect_bm, expect_path):
    H, I = (4096, 256) if wdtype else (4096, 1536)
    p = ops.moe_plan(_args(T, E, H, I, k, wdtype))
    assert p["block_m"] == expect_bm
    assert p["path"] == expect_path
    assert p["capacity"] == T * k + E * (expect_bm - 1)
    assert p["num_blocks"] == -(-p["capacity"] // expect_bm)
    assert p["workspace_bytes"] == ops.moe_forward_workspace(_args(T, E, H, I, k, wdtype))
    offs = [p[n] for n in ("off_sorted_ids", "off_expert_ids", "off_num_post_padded", "off_xq", "off_xs",
                           "off_inter", "off_inter_scale", "off_y") if p[n] >= 0]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    y_bytes = T * k * H * (2 if wdtype else 4)     # y: bf16 for fp8 and MXFP8 weights, else fp32
    assert p["off_y"] + y_bytes <= p["workspace_bytes"]
    assert p["workspace_bytes"] - p["off_y"] < y_bytes + 256 or p["workspace_bytes"] - p["off_y"] < 2 ** 20
    if wdtype:
        assert p["off_xq"] >= 0 and p["off_inter_scale"] >= 0
    else:
        assert p["off_xq"] == -1 and p["off_inter_scale"] == -1
    if wdtype == ops.MOE_WDTYPE_MXFP8:   # one E8M0 byte per 32 elements
        assert p["off_inter"] - p["off_xs"] >= T * H // 32
        assert p["off_xs"] - p["off_xq"] >= T * H


def test_plan_block_override_and_path():
    assert ops.moe_plan(_args(block_m=64))["block_m"] == 64
    assert ops.moe_plan(_args(path=ops.MOE_PATH_SMALL_M))["path"] == ops.MOE_PATH_SMALL_M
    p = ops.moe_plan(_args(path=ops.MOE_PATH_LARGE_M))
    assert p["path"] == ops.MOE_PATH_LARGE_M and p["block_m"] == 256
    # prefill-sized layer forced onto the weight-streaming path
    p = ops.moe_plan(_args(T=4096, path=ops.MOE_PATH_SMALL_M))
    assert p["path"] == ops.MOE_PATH_SMALL_M and p["block_m"] == 64


def test_plan_column_tiles():
    """GEMM2 column-tile widths the planner reports for the weight-streaming
    path: 16-row blocks stream W2 through LDS in 64-row tiles (every bf16
    shape, whose H and I are multiples of 64; block fp8 and MXFP8 for I <= 256
    and H a multiple of 512); other blocks and fp8 shapes keep the
    register-streaming tiles."""
    assert ops.moe_plan(_args())["gemm2_cols"] == 64                        # decode, bf16, 16-row blocks
    assert ops.moe_plan(_args(block_m=32))["gemm2_cols"] == 128
    assert ops.moe_plan(_args(T=1, E=256, H=7168, I=2048))["gemm2_cols"] == 64
    fp8 = dict(T=64, E=256, H=4096, I=256, k=8)
    assert ops.moe_plan(_args(**fp8, wdtype=1))["block_m"] == 16
    assert ops.moe_plan(_args(**fp8, wdtype=1))["gemm2_cols"] == 64
    assert ops.moe_plan(_args(**dict(fp8, I=512), wdtype=1))["gemm2_cols"] == 256
    assert ops.moe_plan(_args(**dict(fp8, H=4352), wdtype=1))["gemm2_cols"] == 256   # H % 512 != 0
    assert ops.moe_plan(_args(**fp8, wdtype=2))["gemm2_cols"] == 64         # MXFP8
    assert ops.moe_plan(_args(**dict(fp8, I=512), wdtype=2))["gemm2_cols"] == 256
    assert ops.moe_plan(_args())["gemm1_cols"] == 128
    assert ops.moe_plan(_args(**fp8, wdtype=1))["gemm1_cols"] == 256


def test_plan_large_path_limits():
    L = ops.lib()
    info = ops.PlanInfo()
    # fp8 and MXFP8 weights take their own LDS-tiled kernels, on 128-row blocks
    for wd in (1, 2):
        p = ops.moe_plan(_args(T=4096, wdtype=wd, I=256, path=ops.MOE_PATH_LARGE_M))
        assert p["path"] == ops.MOE_PATH_LARGE_M and p["block_m"] == 128
        assert L.moe_plan(C.byref(_args(T=4096, wdtype=wd, I=256, path=ops.MOE_PATH_LARGE_M, block_m=256)),
                          C.byref(info)) == ops.MOE_ERR_UNSUPPORTED
        assert L.moe_plan(C.byref(_args(T=4096, wdtype=wd, H=4224, I=256, path=ops.MOE_PATH_LARGE_M)),
                          C.byref(info)) == ops.MOE_ERR_UNSUPPORTED      # H % 256 != 0
        assert L.moe_plan(C.byref(_args(T=4096, wdtype=wd, H=8448, I=256, path=ops.MOE_PATH_LARGE_M)),
                          C.byref(info)) == ops.MOE_ERR_UNSUPPORTED      # K beyond the scale table
    # H not a multiple of 256 has no bf16 large-M kernel
    assert L.moe_plan(C.byref(_args(T=4096, H=4160, path=ops.MOE_PATH_LARGE_M)), C.byref(info)) \
        == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_plan(C.byref(_args(path=ops.MOE_PATH_LARGE_M, block_m=64)), C.byref(info)) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_plan(C.byref(_args(path=ops.MOE_PATH_SMALL_M, block_m=256)), C.byref(info)) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_plan(C.byref(_args(block_m=128)), C.byref(info)) == ops.MOE_ERR_UNSUPPORTED
    # AUTO with a weight-streaming block size stays on that path
    p = ops.moe_plan(_args(T=4096, block_m=32))
    assert p["path"] == ops.MOE_PATH_SMALL_M and p["block_m"] == 32
    # AUTO falls back to the weight-streaming path where the large one cannot run
    assert ops.moe_plan(_args(T=4096, H=4160))["path"] == ops.MOE_PATH_SMALL_M
    assert ops.moe_plan(_args(T=8192, wdtype=1, I=256, H=4224))["path"] == ops.MOE_PATH_SMALL_M


@pytest.mark.parametrize("kw,status", [
    (dict(T=-1), ops.MOE_ERR_INVALID_ARG),
    (dict(E=0), ops.MOE_ERR_INVALID_ARG),
    (dict(E=1025), ops.MOE_ERR_INVALID_ARG),
    (dict(k=0), ops.MOE_ERR_INVALID_ARG),
    (dict(k=65), ops.MOE_ERR_INVALID_ARG),
    (dict(H=0), ops.MOE_ERR_INVALID_ARG),
    (dict(wdtype=7), ops.MOE_ERR_INVALID_ARG),
    (dict(path=9), ops.MOE_ERR_INVALID_ARG),
    (dict(block_m=48), ops.MOE_ERR_UNSUPPORTED),
    (dict(H=4000), ops.MOE_ERR_UNSUPPORTED),                # bf16 needs H % 64 == 0
    (dict(I=1500), ops.MOE_ERR_UNSUPPORTED),
    (dict(H=4032, wdtype=1, I=256), ops.MOE_ERR_UNSUPPORTED),  # fp8 needs H % 128 == 0
    (dict(I=192, wdtype=1), ops.MOE_ERR_UNSUPPORTED),
    (dict(ptr=None), ops.MOE_ERR_INVALID_ARG),
    (dict(ptr=ODD), ops.MOE_ERR_INVALID_ARG),
    (dict(wdtype=1, I=256, scales=False), ops.MOE_ERR_INVALID_ARG),
    (dict(wdtype=2, I=256, scales=False), ops.MOE_ERR_INVALID_ARG),
    (dict(H=4032, wdtype=2, I=256), ops.MOE_ERR_UNSUPPORTED),   # MXFP8 needs H % 128 == 0
    (dict(wdtype=3), ops.MOE_ERR_INVALID_ARG),
    (dict(T=1 << 20, H=4096, I=256, wdtype=2), ops.MOE_ERR_UNSUPPORTED),   # MXFP8: T * H < 2^32
    (dict(flags=4), ops.MOE_ERR_INVALID_ARG),               # unknown flag bit
    (dict(flags=ops.MOE_FLAG_MX_PACKED_SCALES), ops.MOE_ERR_INVALID_ARG),               # packed scales: MXFP8 only
    (dict(flags=ops.MOE_FLAG_MX_PACKED_SCALES, wdtype=1, I=256), ops.MOE_ERR_INVALID_ARG),
    (dict(flags=-1), ops.MOE_ERR_INVALID_ARG),
    (dict(clamp_limit=-1.0), ops.MOE_ERR_INVALID_ARG),
    (dict(clamp_limit=float("nan")), ops.MOE_ERR_INVALID_ARG),
    (dict(clamp_limit=-0.0, ptr=None), ops.MOE_ERR_INVALID_ARG),   # -0 is "no clamp": the null pointer decides
])
def test_forward_validation(kw, status):
    a = _args(**kw)
    assert ops.lib().moe_forward(C.byref(a), C.c_void_p(FAKE), 1 << 40, None) == status


def test_forward_variants_plan_like_the_plain_layer():
    """The variants change only the epilogues: same plan, same workspace."""
    base = ops.moe_plan(_args())
    for kw in (dict(flags=ops.MOE_FLAG_WEIGHT_ON_INPUT), dict(clamp_limit=7.0), dict(clamp_limit=float("inf")),
               dict(flags=ops.MOE_FLAG_WEIGHT_ON_INPUT, clamp_limit=0.5, wdtype=1, I=256)):
        p = ops.moe_plan(_args(**kw))
        ref = base if "wdtype" not in kw else ops.moe_plan(_args(wdtype=1, I=256))
        assert p == ref


def test_mx_packed_scales_plan_like_row_major():
    """The packed MXFP8 scale layout changes only where the kernels read the
    scale bytes: same plan, same workspace."""
    assert ops.moe_plan(_args(wdtype=2, I=256, flags=ops.MOE_FLAG_MX_PACKED_SCALES)) == \
        ops.moe_plan(_args(wdtype=2, I=256))


def test_pack_mx_scales_validation():
    L = ops.lib()
    f, g = C.c_void_p(FAKE), C.c_void_p(FAKE + (1 << 30))
    assert L.moe_pack_mx_scales(f, 2, 20, 128, g, None) == ops.MOE_ERR_UNSUPPORTED    # rows % 16
    assert L.moe_pack_mx_scales(f, 2, 16, 96, g, None) == ops.MOE_ERR_UNSUPPORTED     # K % 128
    assert L.moe_pack_mx_scales(f, 0, 16, 128, g, None) == ops.MOE_ERR_UNSUPPORTED    # no experts
    assert L.moe_pack_mx_scales(f, -1, 16, 128, g, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_pack_mx_scales(f, 2, -16, 128, g, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_pack_mx_scales(None, 2, 16, 128, g, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_pack_mx_scales(f, 2, 16, 128, None, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_pack_mx_scales(f, 2, 16, 128, C.c_void_p(FAKE + 64), None) == ops.MOE_ERR_INVALID_ARG  # overlap
    assert L.moe_pack_mx_scales(None, 2, 0, 128, None, None) == ops.MOE_OK             # nothing to pack


def test_forward_workspace_errors():
    a = _args()
    need = ops.moe_forward_workspace(a)
    L = ops.lib()
    assert L.moe_forward(C.byref(a), C.c_void_p(FAKE), need - 1, None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_forward(C.byref(a), None, need, None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_forward(C.byref(a), C.c_void_p(FAKE + 16), need, None) == ops.MOE_ERR_WORKSPACE


def test_forward_zero_tokens_is_a_noop():
    a = _args(T=0, ptr=None)
    assert ops.lib().moe_forward(C.byref(a), None, 0, None) == ops.MOE_OK


def test_route_align_quant_validation():
    L = ops.lib()
    f = C.c_void_p(FAKE)
    assert L.moe_route(f, 4, 8, 9, 1, f, f, None) == ops.MOE_ERR_INVALID_ARG       # topk > E
    assert L.moe_route(f, 4, 0, 1, 1, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_route(f, 4, 2000, 8, 1, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, 4, 8, 2, 1, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_route(None, 0, 8, 2, 1, None, None, None) == ops.MOE_OK           # no tokens
    assert L.moe_align(f, 4, 2, 8, 0, f, f, f, None, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align(f, 4, 2, 8, 16, None, f, f, None, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align(C.c_void_p(FAKE + 1), 4, 2, 8, 16, f, f, f, None, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act(f, 4, 100, f, f, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_act(f, -1, 128, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act(C.c_void_p(FAKE + 8), 4, 128, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act(None, 0, 128, None, None, None) == ops.MOE_OK
    assert L.moe_quant_act_mx(f, 4, 100, f, f, None) == ops.MOE_ERR_UNSUPPORTED
    assert L.moe_quant_act_mx(f, -1, 32, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act_mx(C.c_void_p(FAKE + 8), 4, 32, f, f, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_quant_act_mx(None, 0, 32, None, None, None) == ops.MOE_OK


def test_decode_layer_validation():
    """moe_decode_layer: shapes outside its scope and missing buffers are
    rejected on the host before any launch."""
    L = ops.lib()
    f = C.c_void_p(FAKE)

    def call(a, logits=None, ids_out=FAKE, w_out=FAKE, sync=FAKE, ws=FAKE, nbytes=1 << 40):
        return L.moe_decode_layer(C.byref(a), None if logits is None else C.c_void_p(logits), 1,
                                  None if ids_out is None else C.c_void_p(ids_out),
                                  None if w_out is None else C.c_void_p(w_out),
                                  None if sync is None else C.c_void_p(sync),
                                  None if ws is None else C.c_void_p(ws), nbytes, None)
    assert ops.moe_plan(_args())["decode_layer"] == 1
    assert call(_args(T=64)) == ops.MOE_ERR_UNSUPPORTED              # 512 slots
    assert call(_args(H=4160)) == ops.MOE_ERR_UNSUPPORTED            # H % 256 != 0
    assert call(_args(block_m=32)) == ops.MOE_ERR_UNSUPPORTED        # only 16-row blocks
    assert call(_args(path=ops.MOE_PATH_LARGE_M, T=4096)) == ops.MOE_ERR_UNSUPPORTED
    assert call(_args(), sync=None) == ops.MOE_ERR_INVALID_ARG
    assert call(_args(), sync=FAKE + 2) == ops.MOE_ERR_INVALID_ARG
    assert call(_args(), logits=FAKE, ids_out=None) == ops.MOE_ERR_INVALID_ARG
    assert call(_args(), logits=FAKE, w_out=None) == ops.MOE_ERR_INVALID_ARG
    assert call(_args(E=4, k=8), logits=FAKE) in (ops.MOE_ERR_INVALID_ARG, ops.MOE_ERR_UNSUPPORTED)
    assert call(_args(ptr=None)) == ops.MOE_ERR_INVALID_ARG
    assert call(_args(), ws=None) == ops.MOE_ERR_WORKSPACE
    assert call(_args(), nbytes=16) == ops.MOE_ERR_WORKSPACE
    assert call(_args(T=0, ptr=None), sync=None, ws=None) in (ops.MOE_OK, ops.MOE_ERR_INVALID_ARG)
    del f


@pytest.mark.parametrize("T,k,E", [(0, 8, 16), (255, 8, 64), (256, 8, 64), (4096, 8, 128), (8192, 8, 256),
                                   (1000, 64, 1024)])
def test_align_scratch_bytes(T, k, E):
    R = T * k
    n = ops.moe_align_scratch_bytes(T, k, E)
    if R <= 8192:
        assert n == 0
    else:
        groups = -(-R // 1024)
        assert n >= 2 * groups * E * 4 and n % 256 == 0


def test_align_ws_validation():
    L = ops.lib()
    assert L.moe_align_scratch_bytes(-1, 8, 16) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_scratch_bytes(16, 0, 16) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_scratch_bytes(16, 8, 1025) == ops.MOE_ERR_INVALID_ARG
    need = L.moe_align_scratch_bytes(4096, 8, 128)
    ptrs = [C.c_void_p(FAKE)] * 4
    # scratch missing, too small, misaligned: rejected before any device work
    assert L.moe_align_ws(C.c_void_p(FAKE), 4096, 8, 128, 64, *ptrs, None, 0, None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_align_ws(C.c_void_p(FAKE), 4096, 8, 128, 64, *ptrs, C.c_void_p(FAKE), need - 4,
                          None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_align_ws(C.c_void_p(FAKE), 4096, 8, 128, 64, *ptrs, C.c_void_p(FAKE + 2), need,
                          None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_align_ws(None, 4096, 8, 128, 64, *ptrs, C.c_void_p(FAKE), need, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_align_ws(C.c_void_p(FAKE), 4096, 8, 128, 0, *ptrs, C.c_void_p(FAKE), need,
                          None) == ops.MOE_ERR_INVALID_ARG


def test_decode_layer_status_word():
    """decode_layer_status raises when the barrier buffer's error word is set
    (as the kernel leaves it after a timed-out wait) and re-zeroes the buffer;
    a clean buffer passes.  The word is set from the host here."""
    import torch
    sync = torch.zeros(ops.MOE_SYNC_WORDS, dtype=torch.int32)
    ops.decode_layer_status(sync)
    sync[ops.MOE_SYNC_ERROR] = 1
    sync[3] = 7
    with pytest.raises(ops.DecodeLayerTimeout) as ei:
        ops.decode_layer_status(sync)
    assert ei.value.status == ops.MOE_ERR_HIP and "undefined" in str(ei.value)
    assert int(sync.abs().sum()) == 0


def test_forward_noalloc_rejects_layers_beyond_its_array():
    """moe_forward_noalloc checks the workspace size against its static array
    before any device work: a prefill-sized layer (0.66 GB of workspace) gets
    MOE_ERR_WORKSPACE, invalid arguments their usual status."""
    L = ops.lib()
    a = _args(T=4096)
    assert ops.moe_forward_workspace(a) > ops.MOE_NOALLOC_MAX_BYTES
    assert L.moe_forward_noalloc(C.byref(a), None) == ops.MOE_ERR_WORKSPACE
    assert L.moe_forward_noalloc(None, None) == ops.MOE_ERR_INVALID_ARG
    assert L.moe_forward_noalloc(C.byref(_args(k=0)), None) == ops.MOE_ERR_INVALID_ARG
    assert ops.moe_forward_workspace(_args()) <= ops.MOE_NOALLOC_MAX_BYTES     # the decode layer fits
