"""Helpers shared by the GPU tests: upload seeded workloads, evaluate the
oracle on all or sampled tokens, and the comparison rules.

Comparison rules
  * integer / index / byte outputs: bit-exact;
  * route weights: |w - w_o| <= 2^-24 (2 max|d| + k + 4) w_o, d = l_j - l_max
    (fp32 subtraction, exp within 1 ulp, k-term sum, one division);
  * layer output (bf16): the output's own rounding (half a bf16 ulp of the
    unrounded oracle value) is not charged; pass iff
        max_i(|gpu_i - o_i| - ulp_bf16(o_i)/2) <= tau * RMS(o)
    with tau = 2e-2 for bf16 weights and 6e-2 for fp8 and MXFP8, RMS over the compared
    outputs of the unrounded fp64 oracle.
"""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle as O
from moe_layer_amd import ops
from moe_layer_amd.workloads import CONFIGS, Config, Workload

TAU = {"bf16": 2e-2, "fp8": 6e-2, "mxfp8": 6e-2}


def log(msg: str):
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def bits_to_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


class DeviceLayer:
    """Expert weights of one (E, H, I, dtype, seed) on the GPU, filled on demand
    for the experts a test routes to (experts never routed stay zero and are
    never read).  Host copies of the layer-format weights are kept for the
    oracle."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self.wl = Workload(cfg)
        E, H, I = cfg.E, cfg.H, cfg.I
        d = dev()
        if cfg.wdtype == "bf16":
            self.w13 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=d)
            self.w2 = torch.zeros((E, H, I), dtype=torch.bfloat16, device=d)
            self.s13 = self.s2 = None
        elif cfg.wdtype == "fp8":
            self.w13 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=d)
            self.w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=d)
            self.s13 = torch.ones((E, 2 * I // 128, H // 128), dtype=torch.float32, device=d)
            self.s2 = torch.ones((E, H // 128, I // 128), dtype=torch.float32, device=d)
        else:   # mxfp8: E8M0 scale bytes per row and 32 K elements (127 = 1.0)
            self.w13 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=d)
            self.w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=d)
            self.s13 = torch.full((E, 2 * I, H // 32), 127, dtype=torch.uint8, device=d)
            self.s2 = torch.full((E, H, I // 32), 127, dtype=torch.uint8, device=d)
        self.host = {}

    def ensure(self, experts):
        need = sorted(set(int(e) for e in experts) - set(self.host))
        if not need:
            return
        t0 = time.time()

        def put(e, w):
            c13, s13, c2, s2 = w
            self.host[e] = w
            if self.cfg.wdtype == "bf16":
                self.w13[e].copy_(bits_to_bf16(c13))
                self.w2[e].copy_(bits_to_bf16(c2))
            else:
                self.w13[e].copy_(torch.from_numpy(c13))
                self.w2[e].copy_(torch.from_numpy(c2))
                self.s13[e].copy_(torch.from_numpy(s13))
                self.s2[e].copy_(torch.from_numpy(s2))

        self.wl.expert_weights_many(need, put)
        torch.cuda.synchronize()
        log(f"uploaded {len(need)} experts of {self.cfg.name} in {time.time() - t0:.1f}s")

    def exact(self, e):
        """fp64 weights of expert e as the layer sees them."""
        c13, s13, c2, s2 = self.host[int(e)]
        if self.cfg.wdtype == "bf16":
            return O.bf16_bits_to_f64(c13), O.bf16_bits_to_f64(c2)
        if self.cfg.wdtype == "mxfp8":
            return O.dequant_mx(c13, s13), O.dequant_mx(c2, s2)
        return O.dequant_block(c13, s13), O.dequant_block(c2, s2)


_LAYERS = {}


def layer_for(cfg: Config) -> DeviceLayer:
    key = (cfg.E, cfg.H, cfg.I, cfg.wdtype, cfg.seed)
    if key not in _LAYERS:
        _LAYERS[key] = DeviceLayer(cfg)
    return _LAYERS[key]


def routing(cfg: Config):
    """(ids int32 [T,k], oracle fp64 weights [T,k], fp32 logits or None)."""
    wl = Workload(cfg)
    if cfg.routing == "given":
        ids, tw = wl.given_routing()
        return ids, tw.astype(np.float64), None
    lg = wl.logits()
    ids, w = O.route(lg, cfg.topk)
    return ids, w, lg


def oracle_tokens(layer: DeviceLayer, x64: np.ndarray, ids: np.ndarray, tw: np.ndarray, tokens,
                  weight_on_input: bool = False, clamp_limit: float = 0.0) -> np.ndarray:
    """Unrounded oracle output rows for the given tokens, one expert at a time
    (with the layer variants as moe_forward takes them: clamp_limit 0 = none)."""
    tokens = np.asarray(tokens)
    fp8 = layer.cfg.wdtype != "bf16"
    group = 32 if layer.cfg.wdtype == "mxfp8" else 128
    out = np.zeros((len(tokens), x64.shape[1]))
    slots = [(i, j) for i, t in enumerate(tokens) for j in range(ids.shape[1])]
    by_e = {}
    for i, j in slots:
        e = int(ids[tokens[i], j])
        if 0 <= e < layer.cfg.E:
            by_e.setdefault(e, []).append((i, j))
    for e, lst in sorted(by_e.items()):
        w13, w2 = layer.exact(e)
        rows_i = [i for i, _ in lst]
        y = O.expert_rows(x64, w13, w2, tokens[rows_i], [tw[tokens[i], j] for i, j in lst], fp8=fp8,
                          group=group, weight_on_input=weight_on_input,
                          clamp_limit=float(clamp_limit) if clamp_limit > 0 else None)
        np.add.at(out, rows_i, y)
    return out


def compare_output(gpu_bf16: np.ndarray, o: np.ndarray):
    """(excess/RMS, raw max-abs/RMS, bf16-floor/RMS) for bf16 outputs vs the oracle."""
    rms = float(np.sqrt(np.mean(o ** 2)))
    a = np.abs(o)
    _, ex = np.frexp(np.where(a > 0, a, 1.0))
    ulp = np.where(a > 0, np.ldexp(1.0, ex - 1 - 7), 2.0 ** -133)
    err = np.abs(gpu_bf16 - o)
    floor = float(np.max(np.abs(O.round_bf16(o) - o)))
    return float(np.max(err - ulp / 2)) / rms, float(np.max(err)) / rms, floor / rms


def route_weight_tol(lg: np.ndarray, ids: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    d = np.abs(sel - sel[:, :1]).max(axis=1, keepdims=True)
    k = ids.shape[1]
    return 2.0 ** -24 * (2 * d + k + 4) * np.abs(w_o)


def run_forward(layer: DeviceLayer, x_bits: np.ndarray, ids: np.ndarray, tw32: np.ndarray, **kw):
    d = dev()
    x = bits_to_bf16(x_bits).to(d)
    ids_t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(d)
    tw_t = torch.from_numpy(np.ascontiguousarray(tw32, dtype=np.float32)).to(d)
    out, ws = ops.moe_forward(x, layer.w13, layer.w2, ids_t, tw_t, layer.s13, layer.s2, **kw)
    torch.cuda.synchronize()
    return out, ws, (x, ids_t, tw_t)
