#!/usr/bin/env python3
"""Benchmark of one GPU's share of the deterministic fused MoE layer, forward + backward.

One step = mok_layer_fwd (router top-k, schedule table, pull dispatch through the ring, grouped
SwiGLU expert GEMMs, weighted combine) followed by mok_layer_bwd (reverse combine, router-weight
gradient fused into SwiGLU backward, dX, dW_gate, dW_up, dW_down) on the DeepSeek-V3-shaped
local share: 64 source segments x 2,048 tokens, hidden 7168, 256 experts, top-8, expert
intermediate 2048, experts 0-3 local, minibatch 2,368 rows, 256 MiB ring, BF16.

Layer tokens/s = 2,048 source tokens per GPU (the unit of the "Mixture-of-Kittens (MoK)"
benchmark section) / step time. Prints one JSON line (see the keys below).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

# MI355X published peaks.
PEAK_BF16_TFLOPS = 2516.6       # dense BF16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_MXFP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0

TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic_layer_fwd_dsv3_bf16.md")
CSRC = os.path.join(HERE, "combine_router_top_schedule_amd", "csrc")


# The sources the fused forward kernel (k_layer_fwd) is compiled from: its file and every header
# it includes. A stored HBM-traffic figure for that kernel is valid only for these.
FUSED_FWD_SOURCES = ("k_fused.hip", "k_ffn.h", "k_gemm.h", "mok_rows.h", "mok_device.h",
                     "mok_internal.h", os.path.join("..", "..", "include", "mok.h"))


def csrc_digest() -> str:
    """Digest of the fused forward kernel's sources."""
    h = hashlib.sha256()
    for name in FUSED_FWD_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(os.path.basename(name).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch of the fused forward kernel from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None when it is absent or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    d = re.search(r"^csrc_digest:\s*([0-9a-f]+)", text, re.M)
    if not m or not d or d.group(1) != csrc_digest():
        return None
    return int(m.group(1))


def cpu_baseline(cfg, target_s: float = 12.0) -> dict:
    """The oracle (fp64 numpy) forward + backward on the tokens of the first n source segments,
    on this host's cores. n is sized from a one-segment run so that the timed sample takes about
    `target_s`; n segments are n/S of a step's work, so oracle tokens/s = T * n / (S * t)."""
    import math
    import numpy as np
    import datagen
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    W = mo.weights_from_bits(datagen.weights(cfg), cfg.dtype)
    align = 32 if cfg.dtype == "mxfp8" else 1

    def run(n):
        tok = np.arange(n * cfg.T)
        lg = datagen.logits(cfg, tok)
        xs = np.concatenate([datagen.x_segment(cfg, s) for s in range(n)])
        ds = np.concatenate([datagen.dout_segment(cfg, s) for s in range(n)])
        t0 = time.perf_counter()
        fw = mo.forward(mo.bf16_rows(xs), lg, W, cfg.K, cfg.e0, cfg.E_loc, cfg.M, align)
        mo.backward(fw, mo.bf16_rows(ds), W, cfg.K, cfg.e0, cfg.E_loc, cfg.E)
        return time.perf_counter() - t0, int((fw.sched.perm >= 0).sum())

    n = 1
    t, pairs = run(1)
    while t < target_s and n < cfg.S:
        n = min(cfg.S, max(2 * n, math.ceil(n * target_s / max(t, 1e-3))))
        t, pairs = run(n)
    return {"value": round(cfg.T * n / (cfg.S * t), 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"oracle fwd+bwd on source segments 0..{n - 1} of {cfg.S} ({n * cfg.T} "
                      f"tokens, {pairs} local pairs) in {t:.2f} s = {n}/{cfg.S} of a step"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3", choices=["dsv3", "kimi", "kimi_mx_skew"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--minibatch", type=int, default=0,
                    help="override the workload's minibatch rows M (ring granularity)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time mok_layer_fwd alone (minibatch sweeps); not the headline metric")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the layer is one "
              "GPU's share of an expert-parallel layer and has no multi-GPU path.",
              file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: WORLD_SIZE > 1 is not supported (one GPU only)", file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import datagen
    import combine_router_top_schedule_amd as mok
    from combine_router_top_schedule_amd.layer import MokLayer

    cfg = datagen.CONFIGS[args.workload]
    if args.minibatch:
        cfg = cfg.replace(M=args.minibatch)
    mx = cfg.dtype == "mxfp8"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    d = mok.desc_from_config(cfg)
    L = MokLayer(d, device=dev, staged=False, fused=True)
    buf = np.empty((cfg.N, cfg.H), dtype=np.uint16)
    x = up(datagen.x_all(cfg, buf))
    dout = up(datagen.dout_all(cfg, buf))
    del buf
    logits = torch.from_numpy(datagen.logits(cfg)).to(dev)
    w = datagen.weights(cfg)
    L.set_weights(up(w["wg"]), up(w["wu"]), up(w["wd"]))
    del w
    out = torch.empty((cfg.N, cfg.H), dtype=torch.int16, device=dev)
    dx = torch.empty_like(out)
    x_seg, out_seg, dout_seg, dx_seg = (L.segs(t) for t in (x, out, dout, dx))
    dp = torch.empty(cfg.N * cfg.K, dtype=torch.float32, device=dev)
    dlogits = (torch.empty((cfg.N, cfg.E), dtype=torch.float32, device=dev)
               if cfg.E_loc == cfg.E else None)
    dwg = torch.empty((cfg.E_loc, cfg.I, cfg.H), dtype=torch.float32, device=dev)
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((cfg.E_loc, cfg.H, cfg.I), dtype=torch.float32, device=dev)

    # A plain copy of known size: its rocprofv3 FETCH_SIZE / WRITE_SIZE calibrate the counters.
    cal = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cal2 = torch.empty_like(cal)
    cal2.copy_(cal)
    del cal, cal2

    def step():
        L.forward(x_seg, logits, out_seg)
        if not args.forward_only:
            L.backward(dout_seg, x_seg, dx_seg, dp, dlogits, dwg, dwu, dwd)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    st = mok.mok_device_status(L.ws)
    if st != 0:
        raise RuntimeError(f"device status {mok.STATUS.get(st, st)} after warmup")

    def events(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for a, b in ev:   # record once so the underlying HIP events exist
            a.record()
            b.record()
        return ev

    # ---- timed region: K steps; HIP events around the fused forward kernel of every step ----
    K = args.steps
    kev = events(K)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    wall0 = time.perf_counter()
    t0.record()
    for i in range(K):
        mok.mok_trace_kernel(mok.MOK_TRACE_FUSED_FWD, *kev[i])
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    mok.mok_trace_kernel(mok.MOK_TRACE_NONE)
    ms = t0.elapsed_time(t1) / K
    fused_ms = sum(a.elapsed_time(b) for a, b in kev) / K
    st = mok.mok_device_status(L.ws)
    if st != 0:
        raise RuntimeError(f"device status {mok.STATUS.get(st, st)} after the timed steps")

    # ---- after the timed region: the other kernel groups, one untimed step each ----
    groups = {}
    for name, kid in (() if args.forward_only else
                      (("a_gemm_and_dwd", mok.MOK_TRACE_BWD_GEMM1),
                       ("dx_gemm_and_dwg_dwu", mok.MOK_TRACE_BWD_GEMM2))):
        (a, b), = events(1)
        mok.mok_trace_kernel(kid, a, b)
        step()
        torch.cuda.synchronize()
        mok.mok_trace_kernel(mok.MOK_TRACE_NONE)
        groups[name] = round(a.elapsed_time(b), 4)

    P = int(L.header()[0])
    HI = cfg.H * cfg.I
    fwd_flop = 6.0 * P * HI
    step_flop = (6.0 if args.forward_only else 18.0) * P * HI
    peak = PEAK_MXFP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    achieved = fwd_flop / (fused_ms * 1e-3) / 1e12
    # the committed counter summary covers the default DeepSeek-V3 BF16 run only
    traffic = stored_traffic() if (args.workload == "dsv3" and not args.minibatch
                                   and not args.forward_only) else None
    tokens_s = cfg.T / (ms * 1e-3)
    line = {
        "metric": ("MoE layer tokens/sec fwd only on 1 MI355X (minibatch sweep)" if args.forward_only
                   else "MoE layer tokens/sec fwd+bwd on 1 MI355X; % MFMA peak and % HBM BW"),
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded PCG64: X, dOut ~ N(0,1), logits ~ N(0,1), W ~ N(0,0.02^2))",
        "config": {"workload": f"{cfg.name} local share, {'fwd' if args.forward_only else 'fwd+bwd'}",
                   "hidden": cfg.H,
                   "experts": cfg.E, "top_k": cfg.K, "intermediate": cfg.I,
                   "local_experts": cfg.E_loc, "segments": cfg.S,
                   "tokens_per_segment": cfg.T, "minibatch": cfg.M,
                   "ring_mib": cfg.ring_bytes >> 20, "pairs": P},
        "roofline": {"bound": "mfma", "kernel": "k_layer_fwd (fused forward)",
                     "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "detail": {"pairs_per_s": round(P / (ms * 1e-3), 1),
                   "step_tflops": round(step_flop / (ms * 1e-3) / 1e12, 1),
                   "step_frac_of_mfma_peak": round(step_flop / (ms * 1e-3) / 1e12 / peak, 4),
                   "fused_fwd_ms": round(fused_ms, 4), "bwd_group_ms": groups,
                   "wall_s": round(wall, 3)},
    }
    if not args.no_cpu_baseline and not args.forward_only:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    rc = main()
    if rc:
        sys.exit(rc)
