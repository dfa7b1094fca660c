"""Python binding of libmok, the MI355X (gfx950) deterministic fused MoE layer.

Argument marshalling only: every step of the layer runs in the HIP kernels of libmok.so. The
functions keep the C names (``mok_schedule``, ``mok_dispatch``, ``mok_expert_ffn``,
``mok_combine``, ``mok_layer_fwd``, ``mok_layer_bwd``, ``mok_quantize_mx``) and take torch
tensors for device buffers; torch is used for device memory and the current stream only.

The library is built in place by ``combine_router_top_schedule_amd.build`` (``__graft_entry__``
calls it). Importing this package without the built library raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmok.so")

MOK_BF16, MOK_MXFP8 = 0, 1
MOK_FLAG_SKIP_ONE_SIGNAL = 0x1
MOK_FLAG_TRACE = 0x2
MOK_FLAG_POISON = 0x4
STATUS = {0: "MOK_OK", 1: "MOK_ERR_NULL", 2: "MOK_ERR_SHAPE", 3: "MOK_ERR_DTYPE",
          4: "MOK_ERR_ALIGN", 5: "MOK_ERR_WORKSPACE", 6: "MOK_ERR_RING", 7: "MOK_ERR_HIP",
          8: "MOK_ERR_DEVICE_TIMEOUT", 9: "MOK_ERR_UNSUPPORTED", 10: "MOK_ERR_SCRATCH"}
MOK_SCRATCH_BYTES = 1 << 20


class MokDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("num_segments", ctypes.c_int32), ("tokens_per_segment", ctypes.c_int32),
                ("expert_begin", ctypes.c_int32), ("num_local_experts", ctypes.c_int32),
                ("minibatch_tokens", ctypes.c_int32), ("comm_cus", ctypes.c_int32),
                ("ring_bytes", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class MokSizes(ctypes.Structure):
    _fields_ = [("saved_bytes", ctypes.c_size_t), ("ws_bytes", ctypes.c_size_t),
                ("bwd_ws_bytes", ctypes.c_size_t),
                ("slots_bytes", ctypes.c_size_t), ("xd_bytes", ctypes.c_size_t),
                ("act_bytes", ctypes.c_size_t), ("wq_bytes", ctypes.c_size_t),
                ("rows_max", ctypes.c_int64), ("ring_slots", ctypes.c_int32),
                ("minibatch", ctypes.c_int32), ("slot_bytes", ctypes.c_int64),
                ("perm_offset", ctypes.c_int64), ("tokpos_offset", ctypes.c_int64),
                ("touched_offset", ctypes.c_int64), ("x_slot_bytes", ctypes.c_int64),
                ("ring_min_bytes", ctypes.c_int64), ("tiles_offset", ctypes.c_int64),
                ("tiles_max", ctypes.c_int64), ("trace_offset", ctypes.c_int64),
                ("trace_records", ctypes.c_int64), ("h_slot_bytes", ctypes.c_int64),
                ("packed_bytes", ctypes.c_int64)]


_P = ctypes.c_void_p


class MokWeights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("wg", "wu", "wd", "wg_q", "wg_s", "wu_q", "wu_s", "wd_q",
                                  "wd_s", "wgt_q", "wgt_s", "wut_q", "wut_s", "wdt_q", "wdt_s",
                                  "packed")]


class MokTuneResult(ctypes.Structure):
    _fields_ = [("minibatch_tokens", ctypes.c_int32), ("comm_cus", ctypes.c_int32),
                ("ms", ctypes.c_float)]


class MokWeightGrads(ctypes.Structure):
    _fields_ = [("dwg", _P), ("dwu", _P), ("dwd", _P)]


# name -> (restype, argtypes); mirrors include/mok.h
_SIGS = {
    "mok_abi_version": (ctypes.c_int, []),
    "mok_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "mok_query_sizes": (ctypes.c_int, [ctypes.POINTER(MokDesc), ctypes.POINTER(MokSizes)]),
    "mok_workspace_size": (ctypes.c_int, [ctypes.POINTER(MokDesc), ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t)]),
    "mok_two_wave_floor": (ctypes.c_int64, [ctypes.c_int32] * 4),
    "mok_schedule": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, _P, _P, _P, _P]),
    "mok_schedule_noalloc": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, _P, _P, _P]),
    "mok_router_fwd": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, _P, _P]),
    "mok_router_ws_size": (ctypes.c_int, [ctypes.POINTER(MokDesc), ctypes.POINTER(ctypes.c_size_t)]),
    "mok_router_bwd": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, _P, _P, _P, _P, _P]),
    "mok_dispatch": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, _P, _P, _P]),
    "mok_expert_ffn": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, ctypes.POINTER(MokWeights),
                                      _P, _P, _P, _P]),
    "mok_combine": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, _P, _P, _P, _P, _P]),
    "mok_layer_fwd": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, ctypes.POINTER(MokWeights),
                                     _P, _P, _P, _P, _P, _P, _P, _P]),
    "mok_macro_ws_size": (ctypes.c_int, [ctypes.POINTER(MokDesc), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_size_t)]),
    "mok_layer_fwd_macro": (ctypes.c_int, [ctypes.POINTER(MokDesc), ctypes.c_int32, _P, _P,
                                           ctypes.POINTER(MokWeights), _P, _P, _P, _P, _P, _P,
                                           _P, _P]),
    "mok_layer_bwd": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, ctypes.POINTER(MokWeights),
                                     _P, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.POINTER(MokWeightGrads), _P, _P]),
    "mok_quantize_mx": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                       ctypes.c_int32, _P, _P, _P]),
    "mok_pack_weights": (ctypes.c_int, [ctypes.POINTER(MokDesc), ctypes.POINTER(MokWeights), _P,
                                        _P]),
    "mok_device_status": (ctypes.c_int, [_P, _P, ctypes.POINTER(ctypes.c_int)]),
    "mok_autotune": (ctypes.c_int, [ctypes.POINTER(MokDesc), _P, _P, ctypes.POINTER(MokWeights),
                                    _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                    ctypes.POINTER(MokDesc), ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(MokTuneResult), ctypes.c_int32,
                                    ctypes.POINTER(ctypes.c_int32)]),
    "mok_device_cus": (ctypes.c_int32, []),
    "mok_trace_kernel": (ctypes.c_int, [ctypes.c_int32, _P, _P]),
}

(MOK_TRACE_NONE, MOK_TRACE_FUSED_FWD, MOK_TRACE_BWD_GEMM1, MOK_TRACE_BWD_GEMM2, MOK_TRACE_DISPATCH,
 MOK_TRACE_COMBINE) = range(6)

_lib = None


def lib():
    """Load libmok.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmok.so not found at {LIB_PATH}; build it first "
                               "(python -m combine_router_top_schedule_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


class MokError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)} "
                         f"({lib().mok_status_str(code).decode()})")
        self.code = code


def _check(fn: str, code: int):
    if code != 0:
        raise MokError(fn, code)


def desc(H, E, K, I, S, T, e0, E_loc, M=0, ring_bytes=0, dtype="bf16", comm_cus=0, flags=0) -> MokDesc:
    dt = {"bf16": MOK_BF16, "mxfp8": MOK_MXFP8}[dtype] if isinstance(dtype, str) else int(dtype)
    return MokDesc(H, E, K, I, S, T, e0, E_loc, M, comm_cus, ring_bytes, dt, flags)


def desc_from_config(cfg, M: Optional[int] = None, ring_bytes: Optional[int] = None, **kw) -> MokDesc:
    """Descriptor for a ``datagen.Config``-like object (fields S, T, H, E, K, I, e0, E_loc, M,
    ring_bytes, dtype)."""
    return desc(cfg.H, cfg.E, cfg.K, cfg.I, cfg.S, cfg.T, cfg.e0, cfg.E_loc,
                cfg.M if M is None else M, cfg.ring_bytes if ring_bytes is None else ring_bytes,
                cfg.dtype, **kw)


def query_sizes(d: MokDesc) -> MokSizes:
    s = MokSizes()
    _check("mok_query_sizes", lib().mok_query_sizes(ctypes.byref(d), ctypes.byref(s)))
    return s


def workspace_size(d: MokDesc):
    """(ws_bytes, saved_bytes, slot_bytes) of the fused entry points."""
    ws, sv, sl = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check("mok_workspace_size", lib().mok_workspace_size(ctypes.byref(d), ctypes.byref(ws),
                                                          ctypes.byref(sv), ctypes.byref(sl)))
    return int(ws.value), int(sv.value), int(sl.value)


def two_wave_floor(cus: int, tile_m: int, tile_n: int, intermediate: int) -> int:
    return int(lib().mok_two_wave_floor(cus, tile_m, tile_n, intermediate))


def abi_version() -> int:
    return int(lib().mok_abi_version())


def device_cus() -> int:
    return int(lib().mok_device_cus())


# ------------------------------------------------------------------------ tensor marshalling

def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("libmok takes device tensors only")


def seg_table(rows, S: int, T: int):
    """Device array of S base pointers into a [S*T][H] tensor (one [T][H] block per segment)."""
    import torch
    base = rows.data_ptr()
    step = T * rows.shape[1] * rows.element_size()
    ptrs = torch.tensor([base + s * step for s in range(S)], dtype=torch.int64)
    return ptrs.to(rows.device)


def weights_struct(wg=None, wu=None, wd=None, **mx) -> MokWeights:
    w = MokWeights()
    w.wg, w.wu, w.wd = _ptr(wg), _ptr(wu), _ptr(wd)
    for k, v in mx.items():
        setattr(w, k, _ptr(v))
    return w


def mok_schedule(d: MokDesc, logits, topk_idx, topk_p, saved, ws, stream=None):
    _need_cuda(logits, topk_idx, topk_p, saved, ws)
    _check("mok_schedule", lib().mok_schedule(ctypes.byref(d), _ptr(logits), _ptr(topk_idx),
                                              _ptr(topk_p), _ptr(saved), _ptr(ws), _stream(stream)))


def mok_schedule_noalloc(d: MokDesc, logits, topk_idx, topk_p, saved, stream=None):
    _need_cuda(logits, topk_idx, topk_p, saved)
    _check("mok_schedule_noalloc", lib().mok_schedule_noalloc(ctypes.byref(d), _ptr(logits),
                                                              _ptr(topk_idx), _ptr(topk_p),
                                                              _ptr(saved), _stream(stream)))


def mok_router_fwd(d: MokDesc, x_seg, wr, logits, stream=None):
    _need_cuda(x_seg, wr, logits)
    _check("mok_router_fwd", lib().mok_router_fwd(ctypes.byref(d), _ptr(x_seg), _ptr(wr),
                                                  _ptr(logits), _stream(stream)))


def router_ws_size(d: MokDesc) -> int:
    n = ctypes.c_size_t()
    _check("mok_router_ws_size", lib().mok_router_ws_size(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def mok_router_bwd(d: MokDesc, x_seg, wr, dlogits, dwr, dx_seg, ws, stream=None):
    _need_cuda(x_seg, wr, dlogits, dwr, dx_seg, ws)
    _check("mok_router_bwd", lib().mok_router_bwd(ctypes.byref(d), _ptr(x_seg), _ptr(wr),
                                                  _ptr(dlogits), _ptr(dwr), _ptr(dx_seg),
                                                  _ptr(ws), _stream(stream)))


def mok_dispatch(d: MokDesc, saved, x_seg, xd, ws, stream=None):
    _need_cuda(saved, x_seg, xd, ws)
    _check("mok_dispatch", lib().mok_dispatch(ctypes.byref(d), _ptr(saved), _ptr(x_seg), _ptr(xd),
                                              _ptr(ws), _stream(stream)))


def mok_expert_ffn(d: MokDesc, saved, xd, w: MokWeights, act, slots, ws, stream=None):
    _need_cuda(saved, xd, act, slots, ws)
    _check("mok_expert_ffn", lib().mok_expert_ffn(ctypes.byref(d), _ptr(saved), _ptr(xd),
                                                  ctypes.byref(w), _ptr(act), _ptr(slots),
                                                  _ptr(ws), _stream(stream)))


def mok_combine(d: MokDesc, saved, topk_idx, topk_p, slots, out_seg, ws, stream=None):
    _need_cuda(saved, topk_idx, topk_p, slots, out_seg, ws)
    _check("mok_combine", lib().mok_combine(ctypes.byref(d), _ptr(saved), _ptr(topk_idx),
                                            _ptr(topk_p), _ptr(slots), _ptr(out_seg), _ptr(ws),
                                            _stream(stream)))


def mok_layer_fwd(d: MokDesc, x_seg, logits, w: MokWeights, out_seg, topk_idx, topk_p, saved,
                  ring, slots, ws, stream=None):
    _need_cuda(x_seg, logits, out_seg, topk_idx, topk_p, saved, ring, slots, ws)
    _check("mok_layer_fwd", lib().mok_layer_fwd(ctypes.byref(d), _ptr(x_seg), _ptr(logits),
                                                ctypes.byref(w), _ptr(out_seg), _ptr(topk_idx),
                                                _ptr(topk_p), _ptr(saved), _ptr(ring),
                                                _ptr(slots), _ptr(ws), _stream(stream)))


def macro_ws_size(d: MokDesc, num_macro: int) -> int:
    n = ctypes.c_size_t()
    _check("mok_macro_ws_size", lib().mok_macro_ws_size(ctypes.byref(d), int(num_macro),
                                                        ctypes.byref(n)))
    return int(n.value)


def mok_layer_fwd_macro(d: MokDesc, x_segs, logits, w: MokWeights, out_segs, topk_idx, topk_p,
                        saved, ring, slots, ws, stream=None):
    """Lists (one entry per macrobatch) for every per-call argument."""
    B = len(x_segs)
    for lst in (logits, out_segs, topk_idx, topk_p, saved, slots):
        if len(lst) != B:
            raise ValueError("one entry per macrobatch in every list")
        _need_cuda(*lst)
    _need_cuda(*x_segs, ring, ws)
    arr = lambda ts: (ctypes.c_void_p * B)(*[_ptr(t) for t in ts])
    _check("mok_layer_fwd_macro", lib().mok_layer_fwd_macro(
        ctypes.byref(d), B, arr(x_segs), arr(logits), ctypes.byref(w), arr(out_segs),
        arr(topk_idx), arr(topk_p), arr(saved), _ptr(ring), arr(slots), _ptr(ws),
        _stream(stream)))


def mok_layer_bwd(d: MokDesc, dout_seg, x_seg, w: MokWeights, topk_idx, topk_p, saved, ring,
                  slots, dx_seg, dp, dlogits, dwg, dwu, dwd, ws, stream=None):
    _need_cuda(dout_seg, x_seg, topk_idx, topk_p, saved, ring, slots, dx_seg, dp, dwg, dwu, dwd, ws)
    g = MokWeightGrads(_ptr(dwg), _ptr(dwu), _ptr(dwd))
    _check("mok_layer_bwd", lib().mok_layer_bwd(ctypes.byref(d), _ptr(dout_seg), _ptr(x_seg),
                                                ctypes.byref(w), _ptr(topk_idx), _ptr(topk_p),
                                                _ptr(saved), _ptr(ring), _ptr(slots),
                                                _ptr(dx_seg), _ptr(dp), _ptr(dlogits),
                                                ctypes.byref(g), _ptr(ws), _stream(stream)))


def mok_quantize_mx(src, transpose: bool, codes, scales, stream=None):
    """Quantise a BF16 tensor [batch][rows][cols] (or [rows][cols]) to MXFP8."""
    _need_cuda(src, codes, scales)
    shape = tuple(src.shape)
    batch, rows, cols = (1,) + shape if len(shape) == 2 else shape
    _check("mok_quantize_mx", lib().mok_quantize_mx(batch, rows, cols, _ptr(src), int(transpose),
                                                    _ptr(codes), _ptr(scales), _stream(stream)))


def mok_pack_weights(d: MokDesc, w: MokWeights, packed, stream=None):
    """Pack the weights of `w` (BF16 values or MXFP8 codes and scales) into `packed`
    (sizes.packed_bytes, 256-byte aligned)."""
    _need_cuda(packed)
    _check("mok_pack_weights", lib().mok_pack_weights(ctypes.byref(d), ctypes.byref(w),
                                                      _ptr(packed), _stream(stream)))


def mok_autotune(d: MokDesc, x_seg, logits, w: MokWeights, out_seg, topk_idx, topk_p, saved,
                 ring, slots, ws, reps: int = 3, stream=None):
    """Returns (tuned descriptor, best ms, [(minibatch, comm_cus, ms), ...])."""
    _need_cuda(x_seg, logits, out_seg, topk_idx, topk_p, saved, ring, slots, ws)
    tuned, best = MokDesc(), ctypes.c_float()
    res = (MokTuneResult * 64)()
    n = ctypes.c_int32(0)
    _check("mok_autotune", lib().mok_autotune(ctypes.byref(d), _ptr(x_seg), _ptr(logits),
                                              ctypes.byref(w), _ptr(out_seg), _ptr(topk_idx),
                                              _ptr(topk_p), _ptr(saved), _ptr(ring), _ptr(slots),
                                              _ptr(ws), _stream(stream), int(reps),
                                              ctypes.byref(tuned), ctypes.byref(best), res, 64,
                                              ctypes.byref(n)))
    return tuned, float(best.value), [(r.minibatch_tokens, r.comm_cus, float(r.ms))
                                      for r in res[:n.value]]


def mok_device_status(ws, stream=None) -> int:
    out = ctypes.c_int(0)
    _check("mok_device_status", lib().mok_device_status(_ptr(ws), _stream(stream), ctypes.byref(out)))
    return int(out.value)


def mok_trace_kernel(kernel: int, before=None, after=None):
    """Record torch.cuda.Event `before` / `after` around one kernel group of the next calls
    (benchmark measurement; MOK_TRACE_NONE switches it off)."""
    b = None if before is None else int(before.cuda_event)
    a = None if after is None else int(after.cuda_event)
    _check("mok_trace_kernel", lib().mok_trace_kernel(int(kernel), b, a))
