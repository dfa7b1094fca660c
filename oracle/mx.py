"""MXFP8 quantiser: E4M3 elements in blocks of 32 sharing one UE8M0 power-of-two scale.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say only that the layer runs in MXFP8 and that activation quantisation is folded
into dispatch, the grouped GEMM and SwiGLU ("把 MoE 通信延迟从 103μs 压到 18μs", section 03
part ③ on the ring token buffer; "Mixture-of-Kittens (MoK)", benchmark section). The format
itself is the OCP Microscaling Formats (MX) v1.0 definition:

* E4M3 ("FN" variant): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; subnormals at
  exponent field 0 (value m/8 * 2^-6); largest normal 0x7E = 448; 0x7F/0xFF are NaN; no inf.
* UE8M0 scale: an unsigned exponent byte, value 2^(code-127); 0xFF is NaN.
* Block scale: X = 2^(floor(log2(amax)) - 8), where 8 is the exponent of E4M3's largest
  normal; elements are V/X rounded to nearest-even in E4M3 and saturated to +-448.

Readings where the spec leaves a choice (they must match the kernels bit for bit):

* amax = 0 gives scale code 0 and all-zero codes (the exponent clamps at -127).
* The shared exponent is clamped to [-127, 127]; the scale code never reaches 0xFF.
* A value that rounds to zero keeps its sign (0x80 for negative inputs).
* NaN is never produced; inputs are finite.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 32


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3 code bytes -> float64 values (NaN codes decode to NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    sub = man / 8.0 * 2.0 ** -6
    nor = (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7.0)
    mag = np.where(ex == 0, sub, nor)
    mag = np.where((ex == 0xF) & (man == 0x7), np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round finite float64 values to E4M3, nearest-even, saturating to +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    # Binade exponent k with 2^k <= a < 2^(k+1); subnormal spacing below 2^-6.
    _, fe = np.frexp(np.where(a > 0, a, 1.0))
    k = fe.astype(np.int64) - 1
    k = np.maximum(k, -6)
    step = np.exp2((k - 3).astype(np.float64))       # 3 mantissa bits
    q = np.rint(a / step) * step                      # np.rint: ties to even
    q = np.minimum(q, E4M3_MAX)
    # Encode the (now representable) magnitude.
    _, qe = np.frexp(np.where(q > 0, q, 1.0))
    qk = qe.astype(np.int64) - 1
    is_sub = q < 2.0 ** -6
    man_sub = np.rint(q / 2.0 ** -9).astype(np.int64)
    man_nor = np.rint((q / np.exp2(qk.astype(np.float64)) - 1.0) * 8.0).astype(np.int64)
    field = np.where(is_sub, man_sub, ((qk + 7) << 3) | man_nor)
    field = np.where(q == 0, 0, field)
    sign = (np.signbit(x)).astype(np.int64) << 7
    return (sign | field).astype(np.uint8)


def _block_scale_exp(amax: np.ndarray) -> np.ndarray:
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
    e = fe.astype(np.int64) - 1 - 8                   # floor(log2 amax) - emax(E4M3)
    e = np.where(amax > 0, e, -127)
    return np.clip(e, -127, 127)


def quantize(v: np.ndarray, axis: int = -1):
    """Quantise ``v`` in blocks of 32 along ``axis`` (its length must be a multiple of 32).

    Returns (codes uint8 with v's shape, scales uint8 with v's shape but axis length / 32).
    """
    v = np.asarray(v, dtype=np.float64)
    vm = np.moveaxis(v, axis, -1)
    n = vm.shape[-1]
    if n % BLOCK:
        raise ValueError("quantised axis must be a multiple of 32")
    blk = vm.reshape(vm.shape[:-1] + (n // BLOCK, BLOCK))
    amax = np.abs(blk).max(axis=-1)
    e = _block_scale_exp(amax)
    codes = e4m3_encode(blk / np.exp2(e.astype(np.float64))[..., None])
    codes = codes.reshape(vm.shape)
    scales = (e + 127).astype(np.uint8)
    return np.moveaxis(codes, -1, axis), np.moveaxis(scales, -1, axis)


def dequantize(codes: np.ndarray, scales: np.ndarray, axis: int = -1) -> np.ndarray:
    """Inverse of ``quantize``: decode(code) * 2^(scale-127), float64."""
    cm = np.moveaxis(np.asarray(codes), axis, -1)
    sm = np.moveaxis(np.asarray(scales), axis, -1).astype(np.float64)
    vals = e4m3_decode(cm).reshape(cm.shape[:-1] + (cm.shape[-1] // BLOCK, BLOCK))
    out = vals * np.exp2(sm - 127.0)[..., None]
    return np.moveaxis(out.reshape(cm.shape), -1, axis)


def _sliced(fn, v: np.ndarray, axis: int, workers: int) -> np.ndarray:
    """Apply ``fn`` (which blocks along ``axis``) to slices of ``v`` along another axis, in
    ``workers`` threads. Every block lies inside one slice, so the result is the same as one
    call on the whole array; numpy releases the interpreter lock inside its loops."""
    axis = axis % v.ndim
    if workers <= 1 or v.ndim < 2:
        return fn(v)
    other = 0 if axis != 0 else 1
    n = v.shape[other]
    bounds = np.linspace(0, n, min(workers, n) + 1).astype(int)
    parts = [np.take(v, np.arange(a, b), axis=other) for a, b in zip(bounds[:-1], bounds[1:])]
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(parts)) as ex:
        return np.concatenate(list(ex.map(fn, parts)), axis=other)


def fake_quant(v: np.ndarray, axis: int = -1, workers: int = 1) -> np.ndarray:
    """dequantize(quantize(v)) along ``axis`` (``workers`` > 1: in parallel slices)."""
    v = np.asarray(v, dtype=np.float64)

    def one(a):
        c, s = quantize(a, axis)
        return dequantize(c, s, axis)

    return _sliced(one, v, axis, workers)


def fake_quant_rows_padded(v: np.ndarray, workers: int = 1) -> np.ndarray:
    """Quantise a [rows][cols] operand in blocks of 32 along rows, zero-padding the last block.

    Used for weight-gradient GEMMs, whose reduction axis is the token axis of one expert.
    """
    v = np.asarray(v, dtype=np.float64)
    r = v.shape[0]
    pad = (-r) % BLOCK
    vp = np.concatenate([v, np.zeros((pad,) + v.shape[1:])], axis=0) if pad else v
    return fake_quant(vp, axis=0, workers=workers)[:r]
