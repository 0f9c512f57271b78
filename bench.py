#!/usr/bin/env python3
"""Throughput of the fused MoE layer on one MI355X.

One step = one pass of the whole layer over one batch of synthetic tokens,
inputs resident in HBM: moe_route (router softmax + top-k on fp32 logits) and
moe_forward (alignment, [fp8 activation quant], GEMM1 + SiLU-mul epilogue,
GEMM2 with the router weight, top-k combine).  The fp8 and mxfp8 workloads are
handed their routing, as the pages' block-fp8 test is, so their step is
moe_forward alone.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

Prints one JSON line.  ``value`` is tokens/s of the whole step; ``roofline``
describes the dominant kernel (GEMM1), timed with HIP events recorded on the
stream it runs on; ``layer`` the whole step against the layer's roofline;
``cpu_baseline`` is the fp64 oracle on a bounded token sample on this host.
The default run (the decode layer) also times the prefill layer (T=4096,
E=128, H=4096, I=1536, top-8, bf16) and adds it as ``prefill``: the metric's
second half, its matrix-core fraction; and the block-fp8 layer (T=1024,
E=256, H=4096, I=256, top-8, e4m3 weights with 128x128 scales) as ``fp8``.
``--no-prefill`` skips both extra records, ``--no-fp8`` the fp8 one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused-MoE layer tokens/s; decode HBM GB/s and prefill MFMA TFLOP/s % of peak"
HBM_PEAK_GBS = 8000.0
# dense matrix-core peaks of the instruction each GEMM runs on: GEMM1 always
# multiplies bf16 operands (fp8 and MXFP8 weights are dequantised to bf16 in
# registers, exactly, so that its fp32 results are accurate); GEMM2 runs on the
# weights' own type
GEMM1_PEAK_TFLOPS = 2500.0
GEMM2_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0}
# dense peak of the layer's own weight type (what an fp8 layer is graded on)
LAYER_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0}
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "prefill", "fp8", "mxfp8", "skew"])
    ap.add_argument("--tokens", type=int, default=None, help="use the first T tokens of the workload")
    ap.add_argument("--block-m", type=int, default=0)
    ap.add_argument("--path", type=int, default=0)
    ap.add_argument("--mx-row-major-scales", action="store_true",
                    help="MXFP8: pass the weight scales row-major instead of packed by moe_pack_mx_scales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-layer", action="store_true",
                    help="run each step as one moe_decode_layer launch (routing inside the kernel)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill and fp8 records the default decode run adds")
    ap.add_argument("--prefill-steps", type=int, default=20)
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the fp8-layer record the default decode run adds")
    ap.add_argument("--fp8-steps", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region run one plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


# sources each dominant kernel is built from (its HBM traffic counters are
# valid only while these are unchanged)
KERNEL_SOURCES = {"small": ("gemm_small.hip", "dev_gemm_small.h", "common.h"),
                  "large": ("gemm_large.hip", "common.h"),
                  "large_q": ("gemm_large_q.hip", "common.h"),
                  "mx": ("gemm_mx.hip", "dev_gemm_mx.h", "common.h")}


def kernel_source_digest(path: str) -> str:
    """sha256 prefix of the kernel's sources with their // comments and blank
    lines removed (a comment edit does not change what the counters saw)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_layer_amd", "csrc")
    for name in KERNEL_SOURCES[path]:
        for line in open(os.path.join(csrc, name), encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def read_traffic(workload: str, digest: str):
    """HBM bytes per GEMM1 launch from the committed counter summary, if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(PROFILES, "hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    for line in open(path):
        f = line.split()
        if len(f) >= 4 and not line.startswith("#") and f[0] == workload and f[1] == digest:
            return float(f[3])
    return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): this layer is measured on a "
              "single MI355X; multi-GPU sharding is described, not run.", file=sys.stderr)
        sys.exit(2)

    rec = measure(args, args.workload, args.tokens, args.steps, args.warmup, not args.no_cpu_baseline,
                  args.copy_calibration)
    if args.workload == "decode" and not args.tokens and not args.no_prefill and not args.decode_layer:
        # the metric's prefill half: the prefill layer's matrix-core fraction,
        # timed in the same run (20 steps after 5 of warm-up, ~2 ms each)
        import gc
        import torch
        gc.collect()
        torch.cuda.empty_cache()
        p = measure(args, "prefill", None, args.prefill_steps, 5, False, False)
        rec["prefill"] = {
            "workload": p["config"]["workload"], "steps": p["steps"], "warmup": p["warmup"],
            "ms_per_step": p["ms_per_step"], "tokens_per_s": p["value"],
            "mfma_frac": p["layer"]["mfma_frac"], "hbm_frac": p["layer"]["hbm_frac"],
            "tflops": p["layer"]["tflops"], "roofline_frac": p["layer"]["roofline_frac"],
            "gemm1": {k: p["roofline"][k] for k in ("kernel", "kernel_ms", "mfma_frac", "hbm_frac", "traffic")},
            "gemm2_ms": p["layer"]["stage_ms"]["gemm2"], "stage_ms": p["layer"]["stage_ms"],
            "active_experts": p["layer"]["active_experts"],
        }
    if args.workload == "decode" and not args.tokens and not args.no_prefill and not args.no_fp8 \
            and not args.decode_layer:
        # the block-fp8 layer, timed in the same run
        import gc
        import torch
        gc.collect()
        torch.cuda.empty_cache()
        q = measure(args, "fp8", None, args.fp8_steps, 5, False, False)
        rec["fp8"] = {
            "workload": q["config"]["workload"], "steps": q["steps"], "warmup": q["warmup"],
            "path": q["config"]["path"], "ms_per_step": q["ms_per_step"], "tokens_per_s": q["value"],
            "hbm_frac": q["layer"]["hbm_frac"], "mfma_frac": q["layer"]["mfma_frac"],
            "roofline_frac": q["layer"]["roofline_frac"],
            "gemm1": {k: q["roofline"][k] for k in ("kernel", "kernel_ms", "hbm_frac", "traffic")},
            "stage_ms": q["layer"]["stage_ms"],
        }
    print(json.dumps(rec), flush=True)


def measure(args, workload, tokens, steps, warmup, with_cpu, copy_calibration):
    """Time one workload; returns its JSON record (without printing it)."""
    import torch
    from moe_layer_amd import ops
    from moe_layer_amd.workloads import CONFIGS, Workload

    d = torch.device("cuda", 0)
    cfg = CONFIGS[workload]
    if tokens:
        cfg = cfg.with_tokens(tokens)
    wl = Workload(cfg)
    fp8 = cfg.wdtype in ("fp8", "mxfp8")
    mx = cfg.wdtype == "mxfp8"
    T, E, H, I, k = cfg.T, cfg.E, cfg.H, cfg.I, cfg.topk
    log(f"workload {cfg.name} T={T} E={E} H={H} I={I} k={k} {cfg.wdtype}")

    x = torch.from_numpy(wl.x_bf16_bits().view(np.int16)).view(torch.bfloat16).to(d)
    if cfg.routing == "logits":
        logits = torch.from_numpy(wl.logits()).to(d)
        ids, tw = ops.moe_route(logits, k)
    else:
        logits = None
        ids_np, tw_np = wl.given_routing()
        ids = torch.from_numpy(ids_np).to(d)
        tw = torch.from_numpy(tw_np).to(d)
    torch.cuda.synchronize()
    ids_host = ids.cpu().numpy()
    active = np.unique(ids_host[(ids_host >= 0) & (ids_host < E)])
    log(f"{len(active)} active experts; drawing and uploading their weights")

    if mx:
        w13 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=d)
        w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=d)
        s13 = torch.full((E, 2 * I, H // 32), 127, dtype=torch.uint8, device=d)
        s2 = torch.full((E, H, I // 32), 127, dtype=torch.uint8, device=d)
    elif fp8:
        w13 = torch.zeros((E, 2 * I, H), dtype=torch.uint8, device=d)
        w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=d)
        s13 = torch.ones((E, 2 * I // 128, H // 128), dtype=torch.float32, device=d)
        s2 = torch.ones((E, H // 128, I // 128), dtype=torch.float32, device=d)
    else:
        w13 = torch.zeros((E, 2 * I, H), dtype=torch.bfloat16, device=d)
        w2 = torch.zeros((E, H, I), dtype=torch.bfloat16, device=d)
        s13 = s2 = None

    # the CPU-baseline sample: the first n tokens (at most 16, and few enough
    # that they route to at most 96 experts) and the experts they route to
    n_cpu = args.cpu_sample_tokens or 1
    if not args.cpu_sample_tokens:
        while n_cpu < min(T, 16) and len(np.unique(ids_host[:n_cpu + 1])) <= 96:
            n_cpu += 1
    cpu_experts = set(np.unique(ids_host[:n_cpu]).tolist())
    host_keep = {}
    t0 = time.time()

    def put(e, w):
        c13, sc13, c2, sc2 = w
        if fp8:
            w13[e].copy_(torch.from_numpy(c13))
            w2[e].copy_(torch.from_numpy(c2))
            s13[e].copy_(torch.from_numpy(sc13))
            s2[e].copy_(torch.from_numpy(sc2))
        else:
            w13[e].copy_(torch.from_numpy(c13.view(np.int16)).view(torch.bfloat16))
            w2[e].copy_(torch.from_numpy(c2.view(np.int16)).view(torch.bfloat16))
        if e in cpu_experts and with_cpu:
            host_keep[e] = w

    wl.expert_weights_many(active.tolist(), put)
    torch.cuda.synchronize()
    log(f"weights ready in {time.time() - t0:.1f}s")

    out = torch.empty((T, H), dtype=torch.bfloat16, device=d)
    # MXFP8 scales: repacked once with the weights (a static weight conversion,
    # outside the timed region) unless the row-major layout is asked for
    packed = mx and not args.mx_row_major_scales
    if packed:
        s13, s2 = ops.moe_pack_mx_scales(s13), ops.moe_pack_mx_scales(s2)
        torch.cuda.synchronize()
    fargs = ops.forward_args(x, w13, w2, ids, tw, s13, s2, out, args.path, args.block_m, mx_packed_scales=packed)
    plan = ops.moe_plan(fargs)
    ws = torch.empty(plan["workspace_bytes"], dtype=torch.uint8, device=d)
    lib = ops.lib()
    import ctypes as C

    use_dl = args.decode_layer
    if use_dl and not plan["decode_layer"]:
        raise SystemExit("--decode-layer: moe_decode_layer does not take this workload (moe_plan)")
    sync = torch.zeros(ops.MOE_SYNC_WORDS, dtype=torch.int32, device=d)

    def step():
        if use_dl:
            st = lib.moe_decode_layer(C.byref(fargs), C.c_void_p(logits.data_ptr()) if logits is not None else None,
                                      1, C.c_void_p(ids.data_ptr()), C.c_void_p(tw.data_ptr()),
                                      C.c_void_p(sync.data_ptr()), C.c_void_p(ws.data_ptr()), ws.numel(),
                                      C.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(ops.status_string(st))
            return
        if logits is not None:
            ops.moe_route(logits, k, True, ids, tw)
        st = lib.moe_forward(C.byref(fargs), C.c_void_p(ws.data_ptr()), ws.numel(),
                             C.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(ops.status_string(st))

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps

    # per-stage durations on the stream the kernels run on
    n_ev = ops.MOE_NUM_STAGES + 1
    stage_ms = np.zeros(ops.MOE_NUM_STAGES)
    for _ in range(steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        ops.moe_forward_profiled(fargs, ws, evs)
        torch.cuda.synchronize()
        stage_ms += np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(ops.MOE_NUM_STAGES)])
    stage_ms /= steps

    if copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=d)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- algorithmic work ---------------------------------------------------
    bw = 1 if fp8 else 2
    na = len(active)
    R = T * k
    # weight scales: fp32 per 128x128 block (fp8) or one E8M0 byte per 32 (mxfp8)
    sc = (lambda n, kk: n * kk // 32) if mx else (lambda n, kk: (n // 128) * (kk // 128) * 4) if fp8 \
        else (lambda n, kk: 0)
    w13_bytes = na * (2 * I * H * bw + sc(2 * I, H))
    w2_bytes = na * (H * I * bw + sc(H, I))
    x_bytes = T * H * 2
    out_bytes = T * H * 2
    route_bytes = T * k * 8 + (T * E * 4 if logits is not None else 0)
    layer_bytes = w13_bytes + w2_bytes + x_bytes + out_bytes + route_bytes
    layer_flops = 6.0 * R * H * I
    # GEMM1: weights of the active experts, activations in, intermediate out
    act_scale = 1 / 32 if mx else 4 / 128   # activation scale bytes per element (fp8 paths)
    g1_bytes = w13_bytes + (T * H * (1 + act_scale) if fp8 else x_bytes) + R * I * (1 + act_scale if fp8 else 2)
    g1_flops = 4.0 * R * H * I
    g1_ms = stage_ms[2]
    # The dominant kernel's roofline: its lower bound is the larger of
    # (algorithmic bytes / HBM peak) and (flops / MFMA peak); report against
    # that bound, and both fractions beside it.  The peak is the dense peak of
    # the layer's weight type (fp8 layers: 5.0 PF/s, although their GEMM1
    # multiplies on the bf16 cores; that instruction's own ceiling is reported
    # beside it as mfma_frac_instr).
    peak_tf = LAYER_PEAK_TFLOPS[cfg.wdtype]
    g1_gbs = g1_bytes / (g1_ms * 1e-3) / 1e9
    g1_tfs = g1_flops / (g1_ms * 1e-3) / 1e12
    hbm_bound = g1_bytes / (HBM_PEAK_GBS * 1e9) >= g1_flops / (peak_tf * 1e12)
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(g1_gbs / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "mfma", "achieved": round(g1_tfs, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(g1_tfs / peak_tf, 4)}
    large = plan["path"] == 2
    fp8w = cfg.wdtype != "bf16"
    digest = kernel_source_digest(("large_q" if fp8w else "large") if large else "mx" if mx else "small")
    roof["traffic"] = read_traffic(cfg.name if not tokens else f"{cfg.name}@{T}", digest)
    roof["kernel"] = ("gemm_large_q_kernel<1> (LDS-tiled fp8/MXFP8 GEMM1 + SiLU-mul-quant epilogue)"
                      if large and fp8w
                      else "gemm_large_kernel<1> (LDS-tiled GEMM1 + SiLU-mul epilogue)" if large
                      else "gemm1_mx_kernel (weight-streaming MXFP8 GEMM1 + SiLU-mul-quant epilogue)" if mx
                      else "gemm1_small_kernel (weight-streaming GEMM1 + SiLU-mul epilogue)")
    roof["kernel_ms"] = round(float(g1_ms), 5)
    roof["algorithmic_bytes"] = int(g1_bytes)
    roof["algorithmic_flops"] = g1_flops
    roof["hbm_frac"] = round(g1_gbs / HBM_PEAK_GBS, 4)
    roof["mfma_frac"] = round(g1_tfs / peak_tf, 4)
    roof["mfma_frac_instr"] = round(g1_tfs / GEMM1_PEAK_TFLOPS, 4)
    roof["scope"] = "one kernel (GEMM1 + epilogue); the whole step's fractions are in 'layer'"
    if use_dl:
        # one launch per step: the dominant kernel is the whole layer
        if int(sync.abs().sum()) != 0:
            raise RuntimeError(f"decode layer barrier buffer not clean: {sync.cpu().numpy()}")
        l_gbs = layer_bytes / (ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(l_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(l_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                "kernel": "decode_layer_kernel (route, align, GEMM1 + SiLU-mul, GEMM2, combine in one launch)",
                "kernel_ms": round(float(ms), 5), "algorithmic_bytes": int(layer_bytes),
                "algorithmic_flops": layer_flops, "hbm_frac": round(l_gbs / HBM_PEAK_GBS, 4),
                "mfma_frac": None, "scope": "the whole layer (one launch)"}

    mfma_floor_s = g1_flops / (GEMM1_PEAK_TFLOPS * 1e12) + (layer_flops - g1_flops) / (
        GEMM2_PEAK_TFLOPS[cfg.wdtype] * 1e12)

    # ---- CPU baseline: the oracle on a bounded sample ---------------------
    cpu = None
    if with_cpu:
        cpu = cpu_baseline(cfg, wl, ids_host, tw.cpu().numpy(), host_keep, n_cpu, logits is not None)

    rec = {
        "metric": METRIC, "value": round(T / (ms * 1e-3), 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.wdtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE layer T={T} E={E} H={H} I={I} topk={k} {cfg.wdtype}",
                   "T": T, "E": E, "H": H, "I": I, "topk": k, "weights": cfg.wdtype,
                   "block_m": plan["block_m"], "path": ["auto", "small_m", "large_m"][plan["path"]],
                   "gemm1_mfma": "bf16", "gemm2_mfma": "bf16" if plan["path"] == 2 else cfg.wdtype,
                   "launch": "one decode-layer kernel" if use_dl else "one kernel per stage",
                   **({"mx_scales": "packed" if packed else "row-major"} if mx else {}),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "layer": {"active_experts": int(na), "algorithmic_bytes": int(layer_bytes), "flops": layer_flops,
                  "hbm_gbs": round(layer_bytes / (ms * 1e-3) / 1e9, 1),
                  "hbm_frac": round(layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "tflops": round(layer_flops / (ms * 1e-3) / 1e12, 2),
                  # against the dense peak of the weight type (fp8: 5.0 PF/s)
                  "mfma_frac": round(layer_flops / (LAYER_PEAK_TFLOPS[cfg.wdtype] * 1e12) / (ms * 1e-3), 4),
                  # against the instructions the kernels use (GEMM1 on bf16 cores, GEMM2 on the weight type's)
                  "mfma_frac_instr": round(mfma_floor_s / (ms * 1e-3), 4),
                  "roofline_frac": round(max(layer_bytes / (HBM_PEAK_GBS * 1e9),
                                             layer_flops / (LAYER_PEAK_TFLOPS[cfg.wdtype] * 1e12)) / (ms * 1e-3), 4),
                  "stage_ms": {n: round(float(v), 5) for n, v in zip(ops.STAGE_NAMES, stage_ms)},
                  "kernel_digest": digest},
    }
    return rec


def cpu_baseline(cfg, wl, ids, tw32, host_w, n, routed_from_logits):
    """Time the fp64 oracle (route + forward) on the first n tokens."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    E, H, I = cfg.E, cfg.H, cfg.I
    fp8 = cfg.wdtype in ("fp8", "mxfp8")
    mx = cfg.wdtype == "mxfp8"
    x64 = wl.x_exact()[:n]
    # only the sample's experts, renumbered 0..m-1 (ids are remapped the same way)
    experts = sorted(host_w)
    remap = np.full(E, -1, dtype=np.int64)
    remap[experts] = np.arange(len(experts))
    w13 = np.empty((len(experts), 2 * I, H))
    w2 = np.empty((len(experts), H, I))
    for i, e in enumerate(experts):
        c13, s13, c2, s2 = host_w[e]
        if mx:
            w13[i], w2[i] = O.dequant_mx(c13, s13), O.dequant_mx(c2, s2)
        elif fp8:
            w13[i], w2[i] = O.dequant_block(c13, s13), O.dequant_block(c2, s2)
        else:
            w13[i], w2[i] = O.bf16_bits_to_f64(c13), O.bf16_bits_to_f64(c2)
    lg = wl.logits()[:n] if routed_from_logits else None
    reps, t_total = 0, 0.0
    while reps < 3 or (t_total < 10.0 and reps < 5000):
        t0 = time.perf_counter()
        if lg is not None:
            ids_o, tw_o = O.route(lg, cfg.topk)
        else:
            ids_o, tw_o = ids[:n], tw32[:n].astype(np.float64)
        O.forward(x64, w13, w2, remap[ids_o], tw_o, fp8=fp8, group=32 if mx else 128)
        t_total += time.perf_counter() - t0
        reps += 1
    t = t_total / reps
    return {"value": round(n / t, 2), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens, route + forward in fp64, mean of {reps} runs "
                      f"({t:.2f} s each)"}


if __name__ == "__main__":
    main()
