#!/usr/bin/env python3
"""Benchmark of one GPU's share of the deterministic fused MoE layer, forward + backward.

One step = mok_layer_fwd (router top-k, schedule table, pull dispatch through the ring, grouped
SwiGLU expert GEMMs, weighted combine) followed by mok_layer_bwd (reverse combine, router-weight
gradient fused into SwiGLU backward, dX, dW_gate, dW_up, dW_down) on the DeepSeek-V3-shaped
local share: 64 source segments x 2,048 tokens, hidden 7168, 256 experts, top-8, expert
intermediate 2048, experts 0-3 local, 256 MiB ring, BF16. The minibatch is the library's
default, the smallest that fills two full waves of 256 x 256 tiles on every CU (8,192 rows on
MI355X); --minibatch overrides it.

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
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

# MI355X published peaks.
PEAK_BF16_TFLOPS = 2516.6       # dense BF16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_MXFP8_TFLOPS = 5033.2
PEAK_HBM_GBS = 8000.0

CSRC = os.path.join(HERE, "combine_router_top_schedule_amd", "csrc")
HEADER = os.path.join("..", "..", "include", "mok.h")

# The three GEMM launches of a step, with the sources each is compiled from (its file and every
# header it includes) and the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of its HBM
# traffic on the DeepSeek-V3 BF16 workload. A stored figure is used only while the kernel's
# sources hash to the digest recorded with it.
KERNELS = {
    "k_layer_fwd": dict(trace=1, flop_per_phi=6.0,
                        what="fused forward: dispatch, gate/up + SwiGLU, down + push",
                        sources=("k_fused.hip", "k_ffn.h", "k_gemm.h", "mok_rows.h",
                                 "mok_device.h", "mok_internal.h", HEADER),
                        traffic="traffic_layer_fwd_dsv3_bf16.md"),
    "k_bwd_gemms<0>": dict(trace=2, flop_per_phi=4.0,
                           what="a-GEMM with dp + SwiGLU backward, and dW_down",
                           sources=("k_bwd.hip", "k_bwd.h", "k_ffn.h", "k_gemm.h", "mok_rows.h",
                                    "mok_device.h", "mok_internal.h", HEADER),
                           traffic="traffic_bwd_gemm1_dsv3_bf16.md"),
    "k_bwd_gemms<1>": dict(trace=3, flop_per_phi=8.0,
                           what="dx GEMM + push, and dW_gate, dW_up",
                           sources=("k_bwd.hip", "k_bwd.h", "k_ffn.h", "k_gemm.h", "mok_rows.h",
                                    "mok_device.h", "mok_internal.h", HEADER),
                           traffic="traffic_bwd_gemm2_dsv3_bf16.md"),
}


def csrc_digest(sources) -> str:
    """Digest of a kernel's sources."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(os.path.basename(name).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from its committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when it is absent or was taken on other kernel sources."""
    k = KERNELS[kernel]
    try:
        text = open(os.path.join(HERE, "profiles", k["traffic"])).read()
    except OSError:
        return None
    m = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    d = re.search(r"^csrc_digest:\s*([0-9a-f]+)", text, re.M)
    if not m or not d or d.group(1) != csrc_digest(k["sources"]):
        return None
    return int(m.group(1))


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        m = re.search(r"^Model name:\s*(.+)$", out, re.M)
        return m.group(1).strip() if m else "unknown"
    except Exception:
        return "unknown"


def cpu_baseline(cfg, target_s: float = 4.0) -> dict:
    """The oracle (fp64 numpy, untuned) forward + backward on the tokens of the first n source
    segments, on this host's cores: n is sized from a one-segment run so one timed run takes about
    `target_s`, and the value is the median of 3 runs (n segments are n/S of a step's work, so
    oracle tokens/s = T * n / (S * t)). Then one run of one segment with the BLAS pool held to a
    single thread."""
    import math
    import statistics
    import numpy as np
    import datagen
    from oracle import moe_oracle as mo
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threadpool_limits = None
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
    if t < target_s and cfg.S > 1:
        n = min(cfg.S, max(2, math.ceil(target_s / max(t, 1e-3))))
    times = []
    for _ in range(3):
        t, pairs = run(n)
        times.append(t)
    t = statistics.median(times)
    one = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1, _ = run(1)
        one = round(cfg.T / (cfg.S * t1), 3)
    return {"value": round(cfg.T * n / (cfg.S * t), 3), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model(), "one_thread_value": one,
            "sample": f"oracle fwd+bwd on source segments 0..{n - 1} of {cfg.S} ({n * cfg.T} "
                      f"tokens, {pairs} local pairs): median of 3 runs "
                      f"{', '.join(f'{x:.2f}' for x in times)} s = {n}/{cfg.S} of a step; "
                      f"one_thread_value: segment 0 alone with one BLAS thread"}


def staged_line(args, cfg, L, mok, torch, x_seg, logits, out_seg) -> dict:
    """The staged forward, timed whole and with HIP events around its pull-dispatch gather and
    its merge (every touched token), each against the HBM peak with its algorithmic bytes:
    dispatch reads and writes every local pair's row (plus the row map), the merge reads every
    pair's pushed row and each touched token's indices and gates and writes its output row."""
    def step():
        L.forward_staged(x_seg, logits, out_seg)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(K):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / K
    hdr = L.header()
    P, rows, U = int(hdr[0]), int(hdr[1]), int(hdr[2])
    mx = cfg.dtype == "mxfp8"
    row_out = cfg.H + cfg.H // 32 if mx else 2 * cfg.H
    work = {"k_dispatch": (mok.MOK_TRACE_DISPATCH, P * cfg.H * 2 + P * row_out + rows * 4,
                           "pull-dispatch gather (P rows read from the segments, written in "
                           "expert order" + (", quantised" if mx else "") + ")"),
            "k_combine": (mok.MOK_TRACE_COMBINE, P * cfg.H * 2 + U * cfg.H * 2 + U * cfg.K * 8,
                          "weighted merge of every touched token (P pushed rows read, U output "
                          "rows written)")}
    kernels = {}
    for name, (tr, nbytes, what) in work.items():
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        for a, b in ev:
            a.record()
            b.record()
        for i in range(K):
            mok.mok_trace_kernel(tr, *ev[i])
            step()
        torch.cuda.synchronize()
        mok.mok_trace_kernel(mok.MOK_TRACE_NONE)
        t = sum(a.elapsed_time(b) for a, b in ev) / K
        gbs = nbytes / (t * 1e-3) / 1e9
        kernels[name] = {"what": what, "avg_ms": round(t, 4), "bytes": int(nbytes),
                         "gb_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    return {
        "metric": "MoE layer tokens/sec fwd, staged path (dispatch and merge bandwidth)",
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded PCG64: X ~ N(0,1), logits ~ N(0,1), W ~ N(0,0.02^2))",
        "config": {"workload": f"{cfg.name} local share, staged fwd", "hidden": cfg.H,
                   "experts": cfg.E, "top_k": cfg.K, "intermediate": cfg.I,
                   "local_experts": cfg.E_loc, "segments": cfg.S, "tokens_per_segment": cfg.T,
                   "minibatch": cfg.M, "pairs": P, "touched_tokens": U},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["gb_s"],
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": kernels[dom]["hbm_frac"],
                     "traffic": None},
        "detail": {"kernels": kernels},
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="dsv3", choices=["dsv3", "kimi", "kimi_mx_skew"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ring-mib", type=int, default=0,
                    help="override the workload's ring size (MiB): how many row tiles stay resident")
    ap.add_argument("--minibatch", type=int, default=0,
                    help="override the workload's minibatch rows M (ring granularity)")
    ap.add_argument("--forward-only", action="store_true",
                    help="time mok_layer_fwd alone (minibatch sweeps); not the headline metric")
    ap.add_argument("--tune", action="store_true",
                    help="run mok_autotune first (minibatch and dispatch-CU split for this shape)")
    ap.add_argument("--staged", action="store_true",
                    help="time the staged forward (mok_schedule, mok_dispatch, mok_expert_ffn, "
                         "mok_combine over every touched token) and report the dispatch gather "
                         "and the merge against HBM bandwidth; not the headline metric")
    ap.add_argument("--trace", action="store_true",
                    help="after the timed steps, run one forward with the phase trace on "
                         "(MOK_FLAG_TRACE) and report its summary under detail.fused_trace")
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

    # minibatch: --minibatch, else 0 (the library's two-wave default; the test configs keep
    # their own M to exercise the minibatch cut)
    cfg = datagen.CONFIGS[args.workload].replace(M=args.minibatch)
    if args.ring_mib:
        cfg = cfg.replace(ring_bytes=args.ring_mib << 20)
    mx = cfg.dtype == "mxfp8"
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    d = mok.desc_from_config(cfg)
    L = MokLayer(d, device=dev, staged=args.staged, fused=not args.staged)
    M_used = int(L.sizes.minibatch)
    cfg = cfg.replace(M=M_used)   # what every later descriptor and the oracle sample use
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

    if args.staged:
        line = staged_line(args, cfg, L, mok, torch, x_seg, logits, out_seg)
        del L, x, dout, logits, out, dx, x_seg, out_seg, dout_seg, dx_seg
        torch.cuda.synchronize()
        print(json.dumps(line), flush=True)
        return 0

    tuning = None
    if args.tune:
        print("[bench] autotune", file=sys.stderr, flush=True)
        tuned, best, table = L.autotune(x_seg, logits, out_seg, reps=3)
        tuning = {"minibatch": tuned.minibatch_tokens, "comm_cus": tuned.comm_cus,
                  "fwd_ms": round(best, 4),
                  "table": [[m, c, round(t, 4)] for m, c, t in table]}
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

    # ---- after the timed region: the two backward GEMM launches, each over K more steps ----
    kernel_ms = {"k_layer_fwd": fused_ms}
    if not args.forward_only:
        for name in ("k_bwd_gemms<0>", "k_bwd_gemms<1>"):
            ev = events(K)
            for i in range(K):
                mok.mok_trace_kernel(KERNELS[name]["trace"], *ev[i])
                step()
            torch.cuda.synchronize()
            mok.mok_trace_kernel(mok.MOK_TRACE_NONE)
            kernel_ms[name] = sum(a.elapsed_time(b) for a, b in ev) / K
            del ev

    P = int(L.header()[0])
    HI = cfg.H * cfg.I
    step_flop = (6.0 if args.forward_only else 18.0) * P * HI
    peak = PEAK_MXFP8_TFLOPS if mx else PEAK_BF16_TFLOPS
    # the committed counter summaries cover the default DeepSeek-V3 BF16 run only
    default_run = (args.workload == "dsv3" and not args.minibatch and not args.forward_only
                   and not args.ring_mib)
    kernels = {}
    for name, t in kernel_ms.items():
        k = KERNELS[name]
        ach = k["flop_per_phi"] * P * HI / (t * 1e-3) / 1e12
        traffic = stored_traffic(name) if default_run else None
        kernels[name] = {"what": k["what"], "avg_ms": round(t, 4), "tflops": round(ach, 1),
                         "frac_of_mfma_peak": round(ach / peak, 4), "traffic_bytes": traffic,
                         "hbm_frac": (round(traffic / (t * 1e-3) / (PEAK_HBM_GBS * 1e9), 4)
                                      if traffic else None)}
    dominant = max(kernel_ms, key=kernel_ms.get)
    dk = kernels[dominant]
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
        "roofline": {"bound": "mfma", "kernel": f"{dominant} ({dk['what']})",
                     "achieved": dk["tflops"], "peak": peak, "unit": "TFLOP/s",
                     "frac": dk["frac_of_mfma_peak"], "traffic": dk["traffic_bytes"],
                     "traffic_hbm_frac": dk["hbm_frac"]},
        "detail": {"pairs_per_s": round(P / (ms * 1e-3), 1),
                   "step_tflops": round(step_flop / (ms * 1e-3) / 1e12, 1),
                   "step_frac_of_mfma_peak": round(step_flop / (ms * 1e-3) / 1e12 / peak, 4),
                   "kernels": kernels, "wall_s": round(wall, 3)},
    }
    if tuning:
        line["detail"]["autotune"] = tuning
        line["config"]["minibatch"] = tuning["minibatch"]
        line["config"]["comm_cus"] = tuning["comm_cus"]
    if args.trace:
        # one more forward on a layer whose descriptor asks for the phase trace (outside the
        # timed region; the trace costs a few clock reads and one record store per item)
        from combine_router_top_schedule_amd import trace
        dt = mok.desc_from_config(cfg, flags=mok.MOK_FLAG_TRACE)
        if tuning:
            dt.minibatch_tokens, dt.comm_cus = tuning["minibatch"], tuning["comm_cus"]
        Lt = MokLayer(dt, device=dev, staged=False, fused=True)
        Lt.w = L.w
        for _ in range(2):
            Lt.forward(x_seg, logits, out_seg)
        torch.cuda.synchronize()
        rec, count = trace.read(Lt.ws, Lt.sizes)
        line["detail"]["fused_trace"] = dict(trace.summarize(rec), dropped=int(count - len(rec)))
        del Lt
    # release what this run created on the device before the interpreter exits (the library's
    # trace hook is already off): events, buffers and the layer
    del kev, t0, t1
    del L, x, dout, logits, out, dx, dp, dlogits, dwg, dwu, dwd, x_seg, out_seg, dout_seg, dx_seg
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and not args.forward_only:
        print("[bench] cpu baseline (oracle sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    rc = main()
    if rc:
        sys.exit(rc)
