"""Phase trace of the fused forward (``MOK_FLAG_TRACE``): read the records the persistent kernel
leaves in its workspace and summarise how its workgroups spent the launch.

Each record is one item of one workgroup: a prologue gather or gather of a row tile (dispatch),
a gate/up column tile or a down column tile (GEMM), with three times on the device's 100 MHz
constant clock: when the workgroup started waiting for the item's inputs, when they were there,
and when its results were stored and signalled. The split into a dispatch group and a GEMM
group that hand work over through counters follows "把 MoE 通信延迟从 103μs 压到 18μs",
section 03 part ②; the summary shows how much of the GEMM group's time goes to waiting.
"""
from __future__ import annotations

import numpy as np

RECORD = np.dtype([("wg", "<i4"), ("info", "<i4"), ("tile", "<i4"), ("item", "<i4"),
                   ("t_wait", "<u8"), ("t_begin", "<u8"), ("t_end", "<u8"), ("pad", "<u8")])
KINDS = {1: "prologue_gather", 2: "gather", 3: "gate_up", 4: "down"}
TICK_US = 0.01          # s_memrealtime runs at 100 MHz
WS_TRACE_COUNT_WORD = 3


def read(ws, sizes):
    """(records, count) from a workspace tensor after a traced forward has finished: records is
    a numpy array of RECORD (at most sizes.trace_records of them), count the number the kernel
    tried to write (larger than the capacity when records were dropped)."""
    count = _word(ws, WS_TRACE_COUNT_WORD)
    n = min(count, int(sizes.trace_records))
    off = int(sizes.trace_offset)
    raw = ws[off:off + n * RECORD.itemsize].cpu().numpy()
    return raw.view(RECORD), count


def _word(ws, i):
    import torch
    return int(ws[4 * i:4 * i + 4].view(torch.int32).item())


def fields(rec):
    """kind, xcd and macrobatch columns decoded from the info word."""
    info = rec["info"].astype(np.int64)
    return info & 0xFF, (info >> 8) & 0xFF, info >> 16


def summarize(rec) -> dict:
    """Per-kind item counts and mean times, and the GEMM group's busy / waiting fractions over
    the traced span (from the first wait to the last signal)."""
    if len(rec) == 0:
        return {"records": 0}
    kind, xcd, _ = fields(rec)
    t0 = int(rec["t_wait"].min())
    t1 = int(rec["t_end"].max())
    span = (t1 - t0) * TICK_US
    out = {"records": int(len(rec)), "span_us": round(span, 2), "kinds": {}}
    for k, name in KINDS.items():
        m = kind == k
        if not m.any():
            continue
        work = (rec["t_end"][m] - rec["t_begin"][m]).astype(np.int64) * TICK_US
        wait = (rec["t_begin"][m] - rec["t_wait"][m]).astype(np.int64) * TICK_US
        out["kinds"][name] = {"items": int(m.sum()), "mean_work_us": round(float(work.mean()), 2),
                              "mean_wait_us": round(float(wait.mean()), 2)}
    g = kind >= 3
    if g.any():
        wgs = np.unique(rec["wg"][g])
        busy = float(((rec["t_end"][g] - rec["t_begin"][g]).astype(np.int64)).sum()) * TICK_US
        wait = float(((rec["t_begin"][g] - rec["t_wait"][g]).astype(np.int64)).sum()) * TICK_US
        total = len(wgs) * span
        out["gemm_workers"] = int(len(wgs))
        out["gemm_busy_frac"] = round(busy / total, 4)
        out["gemm_wait_frac"] = round(wait / total, 4)
        # the tail: per XCD, when its last GEMM item ended, relative to the end of the launch
        ends = {int(x): (t1 - int(rec["t_end"][g & (xcd == x)].max())) * TICK_US
                for x in np.unique(xcd[g])}
        out["xcd_idle_tail_us"] = {x: round(v, 2) for x, v in sorted(ends.items())}
    return out
