"""Seeded synthetic inputs for the fused MoE layer.

This module only draws random numbers and casts them to the layer's input
formats (with torch's CPU casts).  It holds none of the layer's arithmetic and
serves the tests, the benchmark and the oracle alike.

Every tensor comes from ``numpy.random.default_rng([seed, tensor_id, index])``
(PCG64), so one expert's weights can be drawn, uploaded and later redrawn on
their own.  Shapes and value distributions follow the workloads the fused-MoE
pages describe (P2, the block-fp8 test of vLLM PR #64760: x ~ N(0,1)/10,
E=256, H=4096, I=256, topk=8, 128x128 weight blocks; softmax router weights):

  tiny     T=64   E=8   H=256  I=512  k=2  fp32 values (run as bf16 / fp8)
  decode   T=16   E=128 H=4096 I=1536 k=8  bf16
  prefill  T=4096 E=128 H=4096 I=1536 k=8  bf16
  fp8      T=1024 E=256 H=4096 I=256  k=8  e4m3 weights, 128x128 fp32 scales
  mxfp8    T=1024 E=256 H=4096 I=256  k=8  e4m3 weights, E8M0 scale per row and 32 K
  skew     T=8192 E=256 H=7168 I=2048 k=8  bf16, Zipf-biased router logits

Distributions: x ~ N(0, 0.1^2); router matrix W_r ~ N(0, 0.02^2); w13 rows
~ N(0, 1/H), w2 rows ~ N(0, 1/I) (standard deviation 1/sqrt(fan_in)).
Router logits are fl32(x_bf16 . W_r + bias), computed in fp64 and rounded once
to fp32; the router GEMM sits in front of the layer's routing step, and both
the oracle and the GPU consume the same fp32 logits.
"""

from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, replace

import numpy as np

# tensor ids of the seed sequence
TID_X, TID_WR, TID_W13, TID_W2, TID_IDS, TID_TW, TID_RANK = range(7)


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    E: int
    H: int
    I: int
    topk: int
    wdtype: str            # "bf16", "fp8" (128x128 block scales) or "mxfp8"
    routing: str           # "logits" (route from router logits) or "given"
    skew: bool = False
    seed: int = 0

    def with_tokens(self, T: int) -> "Config":
        return replace(self, T=T)


CONFIGS = {
    "tiny": Config("tiny", 64, 8, 256, 512, 2, "bf16", "logits"),
    "decode": Config("decode", 16, 128, 4096, 1536, 8, "bf16", "logits"),
    "prefill": Config("prefill", 4096, 128, 4096, 1536, 8, "bf16", "logits"),
    "fp8": Config("fp8", 1024, 256, 4096, 256, 8, "fp8", "given"),
    "mxfp8": Config("mxfp8", 1024, 256, 4096, 256, 8, "mxfp8", "given"),
    "skew": Config("skew", 8192, 256, 7168, 2048, 8, "bf16", "logits", skew=True),
}

# Zipf ranking for the skewed workload: expert of rank r (1-based, from a seeded
# permutation) gets bias SKEW_LAMBDA * (-1.1 * ln r) for r <= SKEW_ACTIVE, and
# SKEW_DEAD_BIAS beyond, so the hottest expert receives about ten times the
# mean load and the last experts receive none.  SKEW_LAMBDA was fitted on the
# seed-0 draw by tests/golden/calibrate_skew.py (max load / mean in [9.5, 10.5]).
SKEW_ZIPF_S = 1.1
SKEW_ACTIVE = 224
SKEW_DEAD_BIAS = -1.0e4
SKEW_LAMBDA = 0.0485


def _rng(seed: int, tid: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([seed, tid, index])


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (torch's CPU cast, round to nearest even) as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_weight_block_fp8(w: np.ndarray, block: int = 128):
    """Static weight quantisation done by the caller before the layer runs:
    per 128x128 block, scale = amax / 448 in fp32, codes = e4m3(w / scale)
    with torch's CPU cast (OCP E4M3FN, round to nearest even).  Returns
    (codes uint8 [N, K], scales fp32 [N/128, K/128])."""
    import torch
    N, K = w.shape
    wb = np.ascontiguousarray(w, dtype=np.float32).reshape(N // block, block, K // block, block)
    amax = np.abs(wb).max(axis=(1, 3)).astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (wb / scale[:, None, :, None]).astype(np.float32)
    q = np.clip(q, -448.0, 448.0).reshape(N, K)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def quantize_weight_mx(w: np.ndarray, block: int = 32):
    """Static MXFP8 conversion done by the caller, as the OCP microscaling
    format defines it: per row and 32-element block along K the shared
    exponent is floor(log2 amax) - 8 (8 = the largest e4m3 exponent), stored
    as an E8M0 byte (exponent + 127), and the elements are w / 2^exponent
    clamped to +-448 and cast with torch's CPU cast (E4M3FN, nearest even).
    Returns (codes uint8 [N, K], scales uint8 [N, K/32])."""
    import torch
    N, K = w.shape
    wb = np.ascontiguousarray(w, dtype=np.float32).reshape(N, K // block, block)
    amax = np.abs(wb).max(axis=2).astype(np.float64)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))          # amax = m 2^e, m in [0.5, 1)
    x = np.where(amax > 0, e - 1 - 8, -127).clip(-127, 127)
    q = (wb.astype(np.float64) / np.ldexp(1.0, x)[:, :, None]).astype(np.float32)
    q = np.clip(q, -448.0, 448.0).reshape(N, K)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, (x + 127).astype(np.uint8)


class Workload:
    """Lazily drawn inputs of one configuration."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self._x = None
        self._logits = None

    # -- activations -------------------------------------------------------
    def x_f32(self) -> np.ndarray:
        """x ~ N(0, 0.1^2) [T, H] fp32; the first T tokens of the draw for the
        full token count of the named configuration."""
        if self._x is None:
            c = self.cfg
            full_T = CONFIGS[c.name].T if c.name in CONFIGS else c.T
            n = max(full_T, c.T)
            x = _rng(c.seed, TID_X).standard_normal((n, c.H), dtype=np.float32)
            self._x = (x[: c.T] * np.float32(0.1)).astype(np.float32)
        return self._x

    def x_bf16_bits(self) -> np.ndarray:
        return to_bf16_bits(self.x_f32())

    def x_exact(self) -> np.ndarray:
        """The bf16 activations as exact fp64 values."""
        return bf16_bits_to_f32(self.x_bf16_bits()).astype(np.float64)

    # -- router ------------------------------------------------------------
    def router_matrix(self) -> np.ndarray:
        c = self.cfg
        return (_rng(c.seed, TID_WR).standard_normal((c.H, c.E), dtype=np.float32)
                * np.float32(0.02)).astype(np.float32)

    def router_bias(self, lam: float = SKEW_LAMBDA) -> np.ndarray:
        """Per-expert router bias: zero, or the Zipf ranking of the skewed
        workload scaled by ``lam``."""
        c = self.cfg
        if not c.skew:
            return np.zeros(c.E)
        perm = _rng(c.seed, TID_RANK).permutation(c.E)
        rank = np.empty(c.E, dtype=np.int64)
        rank[perm] = np.arange(1, c.E + 1)
        b = lam * (-SKEW_ZIPF_S * np.log(rank.astype(np.float64)))
        return np.where(rank <= SKEW_ACTIVE, b, SKEW_DEAD_BIAS)

    def router_product(self) -> np.ndarray:
        """x_bf16 . W_r in fp64 [T, E] (before the bias and the fp32 rounding)."""
        return self.x_exact() @ self.router_matrix().astype(np.float64)

    def logits(self) -> np.ndarray:
        """fl32(x_bf16 . W_r + bias) [T, E] fp32."""
        if self._logits is None:
            b = self.router_bias()
            self._logits = (self.router_product() + b[None, :]).astype(np.float32)
        return self._logits

    # -- routing given directly (fp8 workload) ------------------------------
    def given_routing(self):
        """ids: per token the first topk entries of a seeded permutation of the
        experts (no repeats, generator order); weights: softmax of N(0,1) over
        the k slots, as fp32."""
        from scipy.special import softmax
        c = self.cfg
        g = _rng(c.seed, TID_IDS)
        ids = np.stack([g.permutation(c.E)[: c.topk] for _ in range(c.T)]).astype(np.int32)
        z = _rng(c.seed, TID_TW).standard_normal((c.T, c.topk))
        tw = softmax(z, axis=1).astype(np.float32)
        return ids, tw

    # -- expert weights ------------------------------------------------------
    def w13_f32(self, e: int) -> np.ndarray:
        c = self.cfg
        w = np.empty((2 * c.I, c.H), dtype=np.float32)
        _rng(c.seed, TID_W13, e).standard_normal(out=w, dtype=np.float32)
        w *= np.float32(1.0 / math.sqrt(c.H))
        return w

    def w2_f32(self, e: int) -> np.ndarray:
        c = self.cfg
        w = np.empty((c.H, c.I), dtype=np.float32)
        _rng(c.seed, TID_W2, e).standard_normal(out=w, dtype=np.float32)
        w *= np.float32(1.0 / math.sqrt(c.I))
        return w

    def expert_weights(self, e: int):
        """Layer-format weights of expert e.
        bf16: (w13 bits uint16 [2I,H], None, w2 bits uint16 [H,I], None)
        fp8 : (w13 codes, w13 scales [2I/128,H/128], w2 codes, w2 scales)
        mxfp8: (w13 codes, w13 E8M0 [2I,H/32], w2 codes, w2 E8M0 [H,I/32])"""
        w13, w2 = self.w13_f32(e), self.w2_f32(e)
        if self.cfg.wdtype == "bf16":
            return to_bf16_bits(w13), None, to_bf16_bits(w2), None
        if self.cfg.wdtype == "mxfp8":
            c13, s13 = quantize_weight_mx(w13)
            c2, s2 = quantize_weight_mx(w2)
            return c13, s13, c2, s2
        c13, s13 = quantize_weight_block_fp8(w13)
        c2, s2 = quantize_weight_block_fp8(w2)
        return c13, s13, c2, s2

    def expert_weights_many(self, experts, fn=None):
        """expert_weights for several experts on a thread pool; ``fn(e, w)`` is
        called in expert order (e.g. to upload each expert and drop it).  At
        most two experts per worker are held at once."""
        experts = list(experts)
        out = {}
        nt = _threads()
        with _cf.ThreadPoolExecutor(nt) as ex:
            futs = {}
            nxt = 0
            for e in experts:
                while nxt < len(experts) and len(futs) < 2 * nt:
                    futs[experts[nxt]] = ex.submit(self.expert_weights, experts[nxt])
                    nxt += 1
                w = futs.pop(e).result()
                if fn is None:
                    out[e] = w
                else:
                    fn(e, w)
        return out


# ----------------------------------------------------------------------------
# Exact-sum layers: inputs on which every partial sum of the gate/up GEMM is
# an exact fp32 value, whatever order the products are added in, so the
# rounding points after it (bf16 gate/up, SiLU, product, fp8 codes) have one
# correct result that a test can demand bit for bit.
# ----------------------------------------------------------------------------

def _e4m3_bytes(v: np.ndarray) -> np.ndarray:
    """Values already on the E4M3FN grid -> their bytes (torch's CPU cast)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def exact_sum_layer(T: int, E: int, H: int, I: int, topk: int, wdtype: str, seed: int = 0,
                    pow2_route_weights: bool = False, hot_expert: int | None = None):
    """A seeded layer whose activations are i/8 with i uniform in [-7, 7] and
    whose weights are j/128 with j uniform in [-15, 15] (bf16), or e4m3 codes
    of j/2 (4 significant bits at most) times a power-of-two block scale drawn
    from {2^-5, 2^-6, 2^-7} (fp8: per 128x128 block; MXFP8: an E8M0 byte per
    row and 32 K elements).  Every product is an integer of at most 105 times
    2^-11 or coarser, and |sum| < 2^24 of those units for H < 2^17, so fp32
    accumulation is exact in any order; the sums carry about 10 significant
    bits, so bf16(h) is a real rounding.  x survives the fp8 activation
    quantisation unchanged (at most 3 significant bits, scaled by a power of
    two).

    Routing: ids uniform over [0, E) with duplicates, plus one unrouted slot
    (id -1) and one id E when T * topk > 4; ``hot_expert`` takes a third of
    the tokens' first slot.  Weights: softmax of N(0, 1) in fp32, or powers
    of two from {1, 1/2, 1/4} with ``pow2_route_weights`` (scaling h by them
    is exact).  Returns dict(x_bits uint16 [T,H], ids int32 [T,k], tw fp32
    [T,k], experts: list of layer-format (w13, s13, w2, s2) per expert, as
    Workload.expert_weights gives them)."""
    from scipy.special import softmax
    g = np.random.default_rng([seed, 100 + TID_X])
    x = g.integers(-7, 8, size=(T, H)).astype(np.float32) / np.float32(8.0)
    gi = np.random.default_rng([seed, 100 + TID_IDS])
    ids = gi.integers(0, E, size=(T, topk)).astype(np.int32)
    if hot_expert is not None:
        ids[: T // 3, 0] = hot_expert
    if T * topk > 4:
        ids[0, topk - 1] = -1
        ids[min(1, T - 1), 0] = E
    gt = np.random.default_rng([seed, 100 + TID_TW])
    if pow2_route_weights:
        tw = np.ldexp(1.0, -gt.integers(0, 3, size=(T, topk))).astype(np.float32)
    else:
        tw = softmax(gt.standard_normal((T, topk)), axis=1).astype(np.float32)
    experts = []
    for e in range(E):
        ge = np.random.default_rng([seed, 100 + TID_W13, e])
        w13i = ge.integers(-15, 16, size=(2 * I, H)).astype(np.float32)
        w2i = ge.integers(-15, 16, size=(H, I)).astype(np.float32)
        if wdtype == "bf16":
            experts.append((to_bf16_bits(w13i / 128), None, to_bf16_bits(w2i / 128), None))
        elif wdtype == "fp8":
            s13 = np.ldexp(1.0, -ge.integers(5, 8, size=(2 * I // 128, H // 128))).astype(np.float32)
            s2 = np.ldexp(1.0, -ge.integers(5, 8, size=(H // 128, I // 128))).astype(np.float32)
            experts.append((_e4m3_bytes(w13i / 2), s13, _e4m3_bytes(w2i / 2), s2))
        elif wdtype == "mxfp8":
            s13 = (127 - ge.integers(5, 8, size=(2 * I, H // 32))).astype(np.uint8)
            s2 = (127 - ge.integers(5, 8, size=(H, I // 32))).astype(np.uint8)
            experts.append((_e4m3_bytes(w13i / 2), s13, _e4m3_bytes(w2i / 2), s2))
        else:
            raise ValueError(wdtype)
    return dict(x_bits=to_bf16_bits(x), ids=ids, tw=tw, experts=experts)
