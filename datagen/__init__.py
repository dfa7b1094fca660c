"""Seeded synthetic inputs for the MoE layer, shared by the CPU oracle and the HIP path.

This module only draws random numbers and encodes them to the storage formats the layer
consumes (BF16 bit patterns, fp32 logits). It holds none of the layer's arithmetic: no top-k,
no gating, no schedule, no GEMM, no quantisation. Both sides read the arrays it returns.

Every tensor has its own counter-keyed PCG64 stream, ``SeedSequence([seed, tensor, part])``, so
any one segment of a large tensor can be regenerated on its own (the full-size parity tests
rebuild only the segments their sampled tokens live in).

Workload shapes come from the layer description on the "Mixture-of-Kittens (MoK)" pages: a
local share of an expert-parallel layer at EP 64 with 2,048 tokens per source rank (benchmark
section), hidden 7168 and expert intermediate 2048 (the explainer page, section on SM
partitioning and minibatch size). The expert counts and top-k are DeepSeek-V3 (256 / top-8)
and Kimi-K2 (384 / top-8) shaped.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# Stream ids: one per tensor kind.
_LOGITS, _X, _WG, _WU, _WD, _DOUT, _WR = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    S: int                # source segments (stand-ins for peer ranks)
    T: int                # tokens per segment
    H: int                # hidden size
    E: int                # routed experts
    K: int                # top-k
    I: int                # expert intermediate size
    e0: int               # first local expert
    E_loc: int            # number of local experts
    M: int                # minibatch rows (ring granularity)
    ring_bytes: int       # fixed ring buffer size
    x_std: float = 1.0
    w_std: float = 0.02
    logit_std: float = 1.0
    dout_std: float = 1.0
    zipf_s: float = 0.0   # 0 = no Zipf bias on the logits
    zipf_alpha: float = 0.0
    dtype: str = "bf16"   # "bf16" or "mxfp8"
    seed: int = 0

    @property
    def N(self) -> int:
        return self.S * self.T

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


MiB = 1 << 20

# Zipf bias strength for the skewed workload. With logits N(0,1) + alpha*ln pmf_Zipf(e+1; 1.2)
# over 384 experts, alpha = 0.2 gives the six local experts (0..5) about 6x their balanced
# share of (token, expert) pairs. The value was found by bisection with the oracle's top-k
# (oracle/calibrate_zipf.py); tests/test_oracle_pins.py re-checks that the skew lies in 4..8.
ZIPF_ALPHA_KIMI = 0.2

CONFIGS = {
    # 64 tokens, hidden 128, 8 experts, top-2, intermediate 256, all experts local.
    "tiny": Config("tiny", S=1, T=64, H=128, E=8, K=2, I=256, e0=0, E_loc=8, M=16,
                   ring_bytes=16 * MiB,
                   x_std=0.02, w_std=0.02, logit_std=1.0, dout_std=1.0),
    # DeepSeek-V3-shaped local share: experts 0..3 of 256, 64 x 2048 source tokens.
    "dsv3": Config("dsv3", S=64, T=2048, H=7168, E=256, K=8, I=2048, e0=0, E_loc=4,
                   M=2368, ring_bytes=256 * MiB),
    # Kimi-K2-shaped local share: experts 0..5 of 384.
    "kimi": Config("kimi", S=64, T=2048, H=7168, E=384, K=8, I=2048, e0=0, E_loc=6,
                   M=2368, ring_bytes=256 * MiB),
    # Kimi-K2 shapes, MXFP8, Zipf-skewed routing.
    "kimi_mx_skew": Config("kimi_mx_skew", S=64, T=2048, H=7168, E=384, K=8, I=2048, e0=0,
                           E_loc=6, M=2368, ring_bytes=256 * MiB, zipf_s=1.2,
                           zipf_alpha=ZIPF_ALPHA_KIMI, dtype="mxfp8"),
}


def _rng(cfg: Config, tensor: int, part: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, tensor, part])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Encode finite fp32 values to BF16 bit patterns, round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode BF16 bit patterns to fp32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_bias(cfg: Config) -> np.ndarray:
    """Per-expert logit bias alpha * ln pmf_Zipf(e+1; s) over experts 0..E-1 (fp64)."""
    if cfg.zipf_s == 0.0 or cfg.zipf_alpha == 0.0:
        return np.zeros(cfg.E, dtype=np.float64)
    k = np.arange(1, cfg.E + 1, dtype=np.float64)
    w = k ** (-cfg.zipf_s)
    return cfg.zipf_alpha * np.log(w / w.sum())


def logits(cfg: Config, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits fp32 [N][E] (or only ``rows``). One stream per segment."""
    segs = range(cfg.S) if rows is None else sorted(set((np.asarray(rows) // cfg.T).tolist()))
    bias = zipf_bias(cfg)
    def one(s):
        z = _rng(cfg, _LOGITS, s).standard_normal((cfg.T, cfg.E), dtype=np.float32)
        z *= np.float32(cfg.logit_std)
        if bias.any():
            z = (z.astype(np.float64) + bias[None, :]).astype(np.float32)
        return s, z

    with ThreadPoolExecutor(_threads()) as ex:
        table = dict(ex.map(one, segs))
    if rows is None:
        return np.concatenate([table[s] for s in segs], axis=0)
    rows = np.asarray(rows)
    return np.stack([table[r // cfg.T][r % cfg.T] for r in rows]) if len(rows) else \
        np.zeros((0, cfg.E), np.float32)


def _seg_bf16(cfg: Config, tensor: int, s: int, std: float) -> np.ndarray:
    z = _rng(cfg, tensor, s).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    z *= np.float32(std)
    return f32_to_bf16_bits(z)


def x_segment(cfg: Config, s: int) -> np.ndarray:
    """Token activations of segment s, BF16 bits [T][H]."""
    return _seg_bf16(cfg, _X, s, cfg.x_std)


def dout_segment(cfg: Config, s: int) -> np.ndarray:
    """Upstream gradient of segment s, BF16 bits [T][H]."""
    return _seg_bf16(cfg, _DOUT, s, cfg.dout_std)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def fill_segments(cfg: Config, seg_fn, out: Optional[np.ndarray] = None) -> np.ndarray:
    """All segments of a [N][H] BF16 tensor, generated in parallel into ``out``."""
    if out is None:
        out = np.empty((cfg.N, cfg.H), dtype=np.uint16)

    def one(s):
        out[s * cfg.T:(s + 1) * cfg.T] = seg_fn(cfg, s)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(one, range(cfg.S)))
    return out


def x_all(cfg: Config, out: Optional[np.ndarray] = None) -> np.ndarray:
    return fill_segments(cfg, x_segment, out)


def dout_all(cfg: Config, out: Optional[np.ndarray] = None) -> np.ndarray:
    return fill_segments(cfg, dout_segment, out)


def rows_of(cfg: Config, seg_fn, rows: np.ndarray) -> np.ndarray:
    """Gather token rows (global ids) by regenerating only the segments they live in."""
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), cfg.H), dtype=np.uint16)
    for s in sorted(set((rows // cfg.T).tolist())):
        seg = seg_fn(cfg, s)
        sel = np.nonzero(rows // cfg.T == s)[0]
        out[sel] = seg[rows[sel] % cfg.T]
    return out


def weights(cfg: Config) -> dict:
    """Local expert weights as BF16 bits: wg, wu [E_loc][I][H]; wd [E_loc][H][I].

    In MXFP8 mode these are the BF16 masters; each side quantises them itself.
    """
    out = {}
    for name, tid, shape in (("wg", _WG, (cfg.I, cfg.H)), ("wu", _WU, (cfg.I, cfg.H)),
                             ("wd", _WD, (cfg.H, cfg.I))):
        mats = []
        for e in range(cfg.E_loc):
            z = _rng(cfg, tid, cfg.e0 + e).standard_normal(shape, dtype=np.float32)
            z *= np.float32(cfg.w_std)
            mats.append(f32_to_bf16_bits(z))
        out[name] = np.stack(mats)
    return out


def router_weight(cfg: Config, std: Optional[float] = None) -> np.ndarray:
    """Router gate weights as BF16 bits [E][H] (the reduction axis contiguous), ~N(0, std^2);
    by default std = logit_std / (x_std * sqrt(H)), so the logits X W_r^T have the spread of the
    workload's direct logits."""
    if std is None:
        std = cfg.logit_std / (cfg.x_std * np.sqrt(cfg.H))
    z = _rng(cfg, _WR, 0).standard_normal((cfg.E, cfg.H), dtype=np.float32)
    z *= np.float32(std)
    return f32_to_bf16_bits(z)
