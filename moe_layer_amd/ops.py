"""Python binding of libmoe_mi355x.so (include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  If the
library is missing the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

# MOE_MI355X_LIB points the binding at another build of the same library
_LIB_PATH = os.environ.get("MOE_MI355X_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                              "libmoe_mi355x.so")
_lib = None

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_WDTYPE_BF16, MOE_WDTYPE_FP8_E4M3, MOE_WDTYPE_MXFP8 = 0, 1, 2
MOE_PATH_AUTO, MOE_PATH_SMALL_M, MOE_PATH_LARGE_M = 0, 1, 2
MOE_FLAG_WEIGHT_ON_INPUT, MOE_FLAG_MX_PACKED_SCALES = 1, 2
MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_QUANT_GROUP, MOE_MX_BLOCK = 1024, 64, 128, 32

# every entry point include/moe.h declares
EXPORTS = ("moe_status_string", "moe_version", "moe_route", "moe_align_capacity", "moe_align",
           "moe_align_scratch_bytes", "moe_align_ws",
           "moe_quant_act", "moe_quant_act_mx", "moe_pack_mx_scales", "moe_plan", "moe_forward_workspace", "moe_forward",
           "moe_forward_profiled", "moe_decode_layer", "moe_forward_noalloc")
MOE_NUM_STAGES = 5
MOE_NOALLOC_MAX_BYTES = 64 << 20
MOE_SYNC_WORDS, MOE_SYNC_ERROR = 640, 576
STAGE_NAMES = ("align", "quant_act", "gemm1", "gemm2", "combine")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} ({status})")


class ForwardArgs(C.Structure):
    _fields_ = [("T", C.c_int32), ("E", C.c_int32), ("H", C.c_int32), ("I", C.c_int32),
                ("topk", C.c_int32), ("wdtype", C.c_int32),
                ("x", C.c_void_p), ("w13", C.c_void_p), ("w13_scale", C.c_void_p),
                ("w2", C.c_void_p), ("w2_scale", C.c_void_p),
                ("topk_ids", C.c_void_p), ("topk_weights", C.c_void_p), ("out", C.c_void_p),
                ("path", C.c_int32), ("block_m", C.c_int32),
                ("flags", C.c_int32), ("clamp_limit", C.c_float)]


class PlanInfo(C.Structure):
    _fields_ = [("path", C.c_int32), ("block_m", C.c_int32), ("capacity", C.c_int64),
                ("num_blocks", C.c_int32), ("gemm1_cols", C.c_int32), ("gemm2_cols", C.c_int32),
                ("decode_layer", C.c_int32), ("workspace_bytes", C.c_int64),
                ("off_sorted_ids", C.c_int64), ("off_expert_ids", C.c_int64),
                ("off_num_post_padded", C.c_int64), ("off_xq", C.c_int64), ("off_xs", C.c_int64),
                ("off_inter", C.c_int64), ("off_inter_scale", C.c_int64), ("off_y", C.c_int64)]


def lib() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m moe_layer_amd.build`")
        L = C.CDLL(_LIB_PATH)
        vp, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
        L.moe_status_string.restype = C.c_char_p
        L.moe_status_string.argtypes = [C.c_int]
        L.moe_version.restype = C.c_int
        L.moe_route.restype = C.c_int
        L.moe_route.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        L.moe_align_capacity.restype = i64
        L.moe_align_capacity.argtypes = [i32, i32, i32, i32]
        L.moe_align.restype = C.c_int
        L.moe_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.moe_align_scratch_bytes.restype = i64
        L.moe_align_scratch_bytes.argtypes = [i32, i32, i32]
        L.moe_align_ws.restype = C.c_int
        L.moe_align_ws.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp, i64, vp]
        L.moe_quant_act.restype = C.c_int
        L.moe_quant_act.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_quant_act_mx.restype = C.c_int
        L.moe_quant_act_mx.argtypes = [vp, i32, i32, vp, vp, vp]
        L.moe_pack_mx_scales.restype = C.c_int
        L.moe_pack_mx_scales.argtypes = [vp, i32, i32, i32, vp, vp]
        L.moe_plan.restype = C.c_int
        L.moe_plan.argtypes = [C.POINTER(ForwardArgs), C.POINTER(PlanInfo)]
        L.moe_forward_workspace.restype = i64
        L.moe_forward_workspace.argtypes = [C.POINTER(ForwardArgs)]
        L.moe_forward.restype = C.c_int
        L.moe_forward.argtypes = [C.POINTER(ForwardArgs), vp, i64, vp]
        L.moe_forward_profiled.restype = C.c_int
        L.moe_forward_profiled.argtypes = [C.POINTER(ForwardArgs), vp, i64, vp, C.POINTER(C.c_void_p), i32]
        L.moe_forward_noalloc.restype = C.c_int
        L.moe_forward_noalloc.argtypes = [C.POINTER(ForwardArgs), vp]
        L.moe_decode_layer.restype = C.c_int
        L.moe_decode_layer.argtypes = [C.POINTER(ForwardArgs), vp, i32, vp, vp, vp, vp, i64, vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


moe_status_string = status_string


def moe_version() -> int:
    return lib().moe_version()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(device=None):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def moe_route(logits: torch.Tensor, topk: int, renormalize: bool = True, topk_ids=None, topk_weights=None):
    """Router softmax + top-k on fp32 logits [T, E]; returns (ids int32 [T,k], weights fp32 [T,k])."""
    assert logits.dtype == torch.float32 and logits.is_contiguous() and logits.dim() == 2
    T, E = logits.shape
    if topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((T, topk), dtype=torch.float32, device=logits.device)
    _check("moe_route", lib().moe_route(_ptr(logits), T, E, topk, int(bool(renormalize)), _ptr(topk_ids),
                                        _ptr(topk_weights), _stream(logits.device)))
    return topk_ids, topk_weights


def moe_align_capacity(T: int, topk: int, E: int, block_m: int) -> int:
    cap = lib().moe_align_capacity(T, topk, E, block_m)
    if cap < 0:
        raise MoeError("moe_align_capacity", int(cap))
    return int(cap)


def moe_align(topk_ids: torch.Tensor, E: int, block_m: int, with_inv: bool = True):
    """Expert-sorted, block-padded alignment of int32 ids [T, k]."""
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() and topk_ids.dim() == 2
    T, k = topk_ids.shape
    cap = moe_align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(-(-cap // block_m), dtype=torch.int32, device=dev)
    ntpp = torch.empty(1, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev) if with_inv else None
    _check("moe_align", lib().moe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(expert_ids),
                                        _ptr(ntpp), _ptr(inv), _stream(dev)))
    return dict(sorted_token_ids=sorted_ids, expert_ids=expert_ids, num_tokens_post_padded=ntpp, inv=inv)


def moe_align_scratch_bytes(T: int, topk: int, E: int) -> int:
    n = lib().moe_align_scratch_bytes(T, topk, E)
    if n < 0:
        raise MoeError("moe_align_scratch_bytes", int(n))
    return int(n)


def moe_align_ws(topk_ids: torch.Tensor, E: int, block_m: int, with_inv: bool = True, scratch=None):
    """moe_align on many workgroups (above 8192 routed slots; the same outputs)."""
    assert topk_ids.dtype == torch.int32 and topk_ids.is_contiguous() and topk_ids.dim() == 2
    T, k = topk_ids.shape
    cap = moe_align_capacity(T, k, E, block_m)
    dev = topk_ids.device
    need = moe_align_scratch_bytes(T, k, E)
    if scratch is None and need > 0:
        scratch = torch.empty(need, dtype=torch.uint8, device=dev)
    sorted_ids = torch.empty(cap, dtype=torch.int32, device=dev)
    expert_ids = torch.empty(-(-cap // block_m), dtype=torch.int32, device=dev)
    ntpp = torch.empty(1, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev) if with_inv else None
    _check("moe_align_ws", lib().moe_align_ws(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(expert_ids),
                                              _ptr(ntpp), _ptr(inv), _ptr(scratch),
                                              0 if scratch is None else scratch.numel(), _stream(dev)))
    return dict(sorted_token_ids=sorted_ids, expert_ids=expert_ids, num_tokens_post_padded=ntpp, inv=inv)


def moe_quant_act(x: torch.Tensor):
    """Per-row, per-128-column fp8 quantisation of bf16 x; returns (codes uint8, scales fp32)."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.dim() == 2
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, max(cols // MOE_QUANT_GROUP, 1)), dtype=torch.float32, device=x.device)
    _check("moe_quant_act", lib().moe_quant_act(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _stream(x.device)))
    return codes, scales


def moe_quant_act_mx(x: torch.Tensor):
    """Per-row, per-32-column MXFP8 quantisation of bf16 x; returns (codes uint8,
    E8M0 scale bytes uint8)."""
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.dim() == 2
    rows, cols = x.shape
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, max(cols // MOE_MX_BLOCK, 1)), dtype=torch.uint8, device=x.device)
    _check("moe_quant_act_mx", lib().moe_quant_act_mx(_ptr(x), rows, cols, _ptr(codes), _ptr(scales),
                                                      _stream(x.device)))
    return codes, scales


def moe_pack_mx_scales(scales: torch.Tensor) -> torch.Tensor:
    """The tile-packed copy of an MXFP8 weight's E8M0 scale bytes [E, rows, K/32]
    (moe_pack_mx_scales; pass it with ``mx_packed_scales=True``)."""
    assert scales.dtype == torch.uint8 and scales.is_contiguous() and scales.dim() == 3
    E, rows, kb = scales.shape
    packed = torch.empty_like(scales)
    _check("moe_pack_mx_scales", lib().moe_pack_mx_scales(_ptr(scales), E, rows, kb * MOE_MX_BLOCK, _ptr(packed),
                                                          _stream(scales.device)))
    return packed


def _u8(t):
    if t is None:
        return None
    return t.view(torch.uint8) if t.dtype == torch.float8_e4m3fn else t


def forward_args(x, w13, w2, topk_ids, topk_weights, w13_scale=None, w2_scale=None, out=None,
                 path=MOE_PATH_AUTO, block_m=0, shape=None, weight_on_input=False,
                 clamp_limit=0.0, mx_packed_scales=False) -> ForwardArgs:
    """Build the moe_forward_args struct.  With ``shape=(T, E, H, I, topk, wdtype)``
    the tensors may be None (for planning and validation).  ``weight_on_input``
    and ``clamp_limit`` select the layer variants (0: no clamp);
    ``mx_packed_scales`` says the MXFP8 scales come from moe_pack_mx_scales."""
    if shape is None:
        T, H = x.shape
        E, twoI, _ = w13.shape
        topk = topk_ids.shape[1]
        fp8 = w13.dtype in (torch.uint8, torch.float8_e4m3fn)
        # fp8 weights with fp32 block scales, or with E8M0 byte scales (MXFP8)
        mx = fp8 and w13_scale is not None and w13_scale.dtype == torch.uint8
        shape = (T, E, H, twoI // 2, topk,
                 MOE_WDTYPE_MXFP8 if mx else MOE_WDTYPE_FP8_E4M3 if fp8 else MOE_WDTYPE_BF16)
    T, E, H, I, topk, wdtype = shape
    a = ForwardArgs()
    a.T, a.E, a.H, a.I, a.topk, a.wdtype = T, E, H, I, topk, wdtype
    a.x, a.w13, a.w13_scale = _ptr(x), _ptr(_u8(w13)), _ptr(w13_scale)
    a.w2, a.w2_scale = _ptr(_u8(w2)), _ptr(w2_scale)
    a.topk_ids, a.topk_weights, a.out = _ptr(topk_ids), _ptr(topk_weights), _ptr(out)
    a.path, a.block_m = path, block_m
    a.flags = (MOE_FLAG_WEIGHT_ON_INPUT if weight_on_input else 0) | \
        (MOE_FLAG_MX_PACKED_SCALES if mx_packed_scales else 0)
    a.clamp_limit = clamp_limit
    return a


def moe_plan(args: ForwardArgs) -> dict:
    info = PlanInfo()
    _check("moe_plan", lib().moe_plan(C.byref(args), C.byref(info)))
    return {name: getattr(info, name) for name, _ in PlanInfo._fields_}


def moe_forward_workspace(args: ForwardArgs) -> int:
    n = lib().moe_forward_workspace(C.byref(args))
    if n < 0:
        raise MoeError("moe_forward_workspace", int(n))
    return int(n)


def moe_forward(x, w13, w2, topk_ids, topk_weights, w13_scale=None, w2_scale=None, out=None,
                workspace=None, path=MOE_PATH_AUTO, block_m=0, weight_on_input=False, clamp_limit=0.0,
                mx_packed_scales=False):
    """The fused MoE layer: bf16 x [T,H], w13 [E,2I,H], w2 [E,H,I] (bf16; or
    e4m3 with fp32 128x128 block scales; or e4m3 with E8M0 uint8 scales per row
    and 32 K elements, MXFP8, row-major or, with ``mx_packed_scales``, from
    moe_pack_mx_scales), int32 ids [T,k], fp32 weights [T,k].
    ``weight_on_input``: the router weight scales GEMM1's input row instead of
    GEMM2's output; ``clamp_limit`` > 0: SwiGLU clamp (gate <= L, |up| <= L).
    Returns (out bf16 [T,H], workspace)."""
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    a = forward_args(x, w13, w2, topk_ids, topk_weights, w13_scale, w2_scale, out, path, block_m,
                     weight_on_input=weight_on_input, clamp_limit=clamp_limit, mx_packed_scales=mx_packed_scales)
    need = moe_forward_workspace(a)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _check("moe_forward", lib().moe_forward(C.byref(a), _ptr(workspace), workspace.numel(), _stream(x.device)))
    return out, workspace


def moe_forward_noalloc(x, w13, w2, topk_ids, topk_weights, w13_scale=None, w2_scale=None, out=None,
                        path=MOE_PATH_AUTO, block_m=0, weight_on_input=False, clamp_limit=0.0,
                        mx_packed_scales=False):
    """moe_forward with the library's static per-GPU workspace
    (moe_forward_noalloc: for callers that cannot allocate device memory;
    up to MOE_NOALLOC_MAX_BYTES of workspace).  Returns out."""
    T, H = x.shape
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    a = forward_args(x, w13, w2, topk_ids, topk_weights, w13_scale, w2_scale, out, path, block_m,
                     weight_on_input=weight_on_input, clamp_limit=clamp_limit, mx_packed_scales=mx_packed_scales)
    _check("moe_forward_noalloc", lib().moe_forward_noalloc(C.byref(a), _stream(x.device)))
    return out


def moe_forward_profiled(args: ForwardArgs, workspace: torch.Tensor, events, stream=None):
    """moe_forward on prepared args with HIP events recorded around its stages.
    ``events``: MOE_NUM_STAGES + 1 torch.cuda.Event(enable_timing=True) objects;
    they are recorded on ``stream`` (default: the current stream), the stream
    the kernels run on."""
    s = torch.cuda.current_stream() if stream is None else stream
    for e in events:                      # make sure the underlying hipEvent_t exists
        if e.cuda_event == 0:
            e.record(s)
    arr = (C.c_void_p * len(events))(*[C.c_void_p(e.cuda_event) for e in events])
    _check("moe_forward_profiled", lib().moe_forward_profiled(
        C.byref(args), _ptr(workspace), workspace.numel(), C.c_void_p(s.cuda_stream), arr, len(events)))


_SYNC = {}


def decode_sync(device, stream=None) -> torch.Tensor:
    """A zeroed barrier buffer for moe_decode_layer, kept per (device, stream)
    and reused: every call leaves it zero, and calls that share a buffer must
    be ordered on one stream (include/moe.h)."""
    dev = torch.device(device)
    s = torch.cuda.current_stream(dev) if stream is None else stream
    key = (dev.index or 0, int(s.cuda_stream))
    if key not in _SYNC:
        _SYNC[key] = torch.zeros(MOE_SYNC_WORDS, dtype=torch.int32, device=dev)
    return _SYNC[key]


class DecodeLayerTimeout(MoeError):
    """A grid-barrier wait of moe_decode_layer exceeded its bound (the device
    could not keep every workgroup resident): that call's output is undefined."""

    def __init__(self, word: int):
        self.word = word
        RuntimeError.__init__(self, f"moe_decode_layer: a grid-barrier wait timed out (sync[MOE_SYNC_ERROR] = "
                                    f"{word}); the output of that call is undefined")
        self.status = MOE_ERR_HIP


def decode_layer_status(sync: torch.Tensor) -> None:
    """Check a moe_decode_layer barrier buffer after the calls that used it:
    reads sync[MOE_SYNC_ERROR] (this waits for the buffer's stream), and if a
    barrier wait timed out re-zeroes the buffer, as include/moe.h requires
    before its next use, and raises DecodeLayerTimeout.  While that word is
    set, the outputs of the calls since it was last clear are invalid."""
    word = int(sync[MOE_SYNC_ERROR].item())
    if word != 0:
        sync.zero_()
        raise DecodeLayerTimeout(word)


def moe_decode_layer(x, w13, w2, topk_ids=None, topk_weights=None, w13_scale=None, w2_scale=None,
                     router_logits=None, topk=None, renormalize=True, out=None, workspace=None, sync=None,
                     weight_on_input=False, clamp_limit=0.0, mx_packed_scales=False, check=True):
    """The layer for few tokens as one kernel launch (the weight-streaming
    path with 16-row blocks).  With fp32 ``router_logits`` [T,E] it routes
    them (top ``topk``) into topk_ids / topk_weights (allocated when None);
    else it uses the given routing.  ``sync``: the barrier buffer (default:
    one per device and current stream).  With ``check`` the call waits for
    the stream and raises DecodeLayerTimeout if a barrier wait timed out
    (decode_layer_status); without it, call decode_layer_status before
    trusting the output.  Returns (out, topk_ids, topk_weights, workspace)."""
    T, H = x.shape
    dev = x.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if router_logits is not None and topk_ids is None:
        topk_ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
        topk_weights = torch.empty((T, topk), dtype=torch.float32, device=dev)
    a = forward_args(x, w13, w2, topk_ids, topk_weights, w13_scale, w2_scale, out, MOE_PATH_SMALL_M, 16,
                     weight_on_input=weight_on_input, clamp_limit=clamp_limit, mx_packed_scales=mx_packed_scales)
    need = moe_forward_workspace(a)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    sync = decode_sync(dev) if sync is None else sync
    if router_logits is not None:
        st = lib().moe_decode_layer(C.byref(a), _ptr(router_logits), int(bool(renormalize)), _ptr(topk_ids),
                                    _ptr(topk_weights), _ptr(sync), _ptr(workspace), workspace.numel(), _stream(dev))
    else:
        st = lib().moe_decode_layer(C.byref(a), None, 0, None, None, _ptr(sync), _ptr(workspace),
                                    workspace.numel(), _stream(dev))
    _check("moe_decode_layer", st)
    if check:
        decode_layer_status(sync)
    return out, topk_ids, topk_weights, workspace
