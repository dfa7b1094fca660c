"""Crafted inputs that pin where the MXFP8 layer quantises, and along which axis.

Each case is a tiny layer (H = I = 128, K = 1 so every gate p is 1) whose operands are built
from two magnitudes: 1-ish values and TINY = 1.5 * 2^-20. Inside one 32-element block whose
largest magnitude is about 1, TINY falls below half the smallest E4M3 subnormal under the
block's scale (2^-9 * 2^-8), so quantising that block flushes it to zero; a block holding only
TINY values (or TINY next to zeros) keeps it. An operand that varies along one axis only is
therefore left unchanged when it is blocked along the other axis and loses its TINY entries
when blocked along the varying one. Routing the TINY entries' contribution into an output
column of its own turns "quantised along the right axis" into "that column is exactly zero".

The builders only lay out numbers; they hold none of the layer's arithmetic. Values are float64
and exactly representable in BF16 (so the GPU tests can feed the same bits).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

TINY = 1.5 * 2.0 ** -20
H = I = 128


@dataclasses.dataclass
class Crafted:
    x: np.ndarray            # [N][H]
    dout: np.ndarray         # [N][H]
    logits: np.ndarray       # [N][E] fp32
    wg: np.ndarray           # [E_loc][I][H]
    wu: np.ndarray
    wd: np.ndarray           # [E_loc][H][I]
    K: int = 1

    @property
    def N(self) -> int:
        return self.x.shape[0]

    @property
    def E(self) -> int:
        return self.logits.shape[1]


def _even(n):
    return np.arange(n) % 2 == 0


def _single(x, dout, wg, wu, wd) -> Crafted:
    N = x.shape[0]
    return Crafted(x, dout, np.zeros((N, 1), np.float32), wg[None], wu[None], wd[None])


def dispatch_x_along_h(N: int = 64) -> Crafted:
    """X varies along H only (1 at even h, TINY at odd h): blocked along H the odd columns of the
    dispatched rows become 0; blocked along tokens nothing changes. Gate row 32 sums the odd
    columns (g[:, 32] = 0 exactly when they flush), row 0 the even ones; with u = 1 there, Wd sends
    h[:, 0] to output column 0 and h[:, 32] (its own 32-block of I) to column 1: out[:, 1] == 0."""
    x = np.where(_even(H)[None, :], 1.0, TINY) * np.ones((N, H))
    wg = np.zeros((I, H)); wg[0, _even(H)] = 1.0; wg[32, ~_even(H)] = 1.0
    wu = np.zeros((I, H)); wu[0, 0] = 1.0; wu[32, 0] = 1.0
    wd = np.zeros((H, I)); wd[0, 0] = 1.0; wd[1, 32] = 1.0
    return _single(x, np.ones((N, H)), wg, wu, wd)


def swiglu_h_along_i(N: int = 64) -> Crafted:
    """h varies along I only: g = 6 at even i, -24 at odd i, u = 1, so h = silu(g) u is ~6 at
    even i and ~-9e-10 at odd i. Blocked along I the odd entries flush; the down GEMM sends
    even i to output column 0 and odd i to column 1, so y[:, 1] (and out[:, 1]) is exactly 0."""
    x = np.zeros((N, H)); x[:, 0] = 1.0
    wg = np.zeros((I, H)); wg[:, 0] = np.where(_even(I), 6.0, -24.0)
    wu = np.zeros((I, H)); wu[:, 0] = 1.0
    wd = np.zeros((H, I)); wd[0, _even(I)] = 1.0; wd[1, ~_even(I)] = 1.0
    return _single(x, np.ones((N, H)), wg, wu, wd)


def backward_d_along_h(N: int = 64) -> Crafted:
    """dOut varies along H only (1 at even h, TINY at odd h). Wd sends even h to a[:, 0] and odd
    h to a[:, 32], so blocked along H a[:, 32] is exactly 0. a[:, 32] (its own 32-block of I)
    only reaches dg[:, 32] and du[:, 32], which Wg, Wu send to dX column 2 (a[:, 0] reaches
    column 3): dX[:, 2] == 0."""
    x = np.zeros((N, H)); x[:, 2] = 1.0; x[:, 3] = 1.0
    wg = np.zeros((I, H)); wg[0, 3] = 1.0; wg[32, 2] = 1.0
    wu = np.zeros((I, H)); wu[0, 3] = 1.0; wu[32, 2] = 1.0
    wd = np.zeros((H, I)); wd[_even(H), 0] = 1.0; wd[~_even(H), 32] = 1.0
    dout = np.where(_even(H)[None, :], 1.0, TINY) * np.ones((N, H))
    return _single(x, dout, wg, wu, wd)


def backward_dgdu_along_i(N: int = 64) -> Crafted:
    """dg and du vary along I only: g = 6 / -24 and u = 1 at even / odd i, a = 128 for every i
    (dOut and Wd all ones), so dg ~ 130 vs ~-1e-7 and du ~ 766 vs ~-1e-7. Blocked along I the
    odd entries flush. Wg, Wu send even i to dX column 0 and odd i to column 1: dX[:, 1] == 0."""
    x = np.zeros((N, H)); x[:, 0] = 1.0; x[:, 1] = 1.0
    ev = _even(I)
    wg = np.zeros((I, H)); wg[ev, 0] = 6.0; wg[~ev, 1] = -24.0
    wu = np.zeros((I, H)); wu[ev, 0] = 1.0; wu[~ev, 1] = 1.0
    return _single(x, np.ones((N, H)), wg, wu, np.ones((H, I)))


def wgrad_x_along_tokens(N: int = 64) -> Crafted:
    """X column 0 varies along tokens only (1 on even tokens, TINY on odd ones); column 32 is 1
    everywhere and carries the gate/up inputs, so g, u, dg and du are the same on every token.
    Blocked along tokens the odd tokens' column 0 flushes: dWg[:, 0] * N == dWg[:, 32] * N_even
    exactly (likewise dWu). Blocked along H (one nonzero per block) nothing flushes."""
    x = np.zeros((N, H)); x[:, 32] = 1.0; x[:, 0] = np.where(_even(N), 1.0, TINY)
    wg = np.zeros((I, H)); wg[:, 32] = 6.0
    wu = np.zeros((I, H)); wu[:, 32] = 1.0
    return _single(x, np.ones((N, H)), wg, wu, np.ones((H, I)))


def wgrad_h_along_tokens(N: int = 64) -> Crafted:
    """h column 1 varies along tokens only: even tokens (x = e_0) have h ~ silu(6) in every
    column; odd tokens (x = e_32) have h = silu(6) * TINY in column 1 and 0 elsewhere (still
    nonzero after the forward's quantisation along I, its block holding nothing larger).
    dOut = e_0, p = 1: dWd[0, 1] = sum over tokens of Q_tokens(h)[:, 1], which is exactly
    N_even * h[even, 1] when the odd tokens flush."""
    x = np.zeros((N, H)); x[_even(N), 0] = 1.0; x[~_even(N), 32] = 1.0
    wg = np.zeros((I, H)); wg[:, 0] = 6.0; wg[1, 32] = 6.0
    wu = np.zeros((I, H)); wu[:, 0] = 1.0; wu[1, 32] = TINY
    dout = np.zeros((N, H)); dout[:, 0] = 1.0
    return _single(x, dout, wg, wu, np.ones((H, I)))


def wgrad_dgdu_pd_along_tokens(N: int = 64, odd_scale: float = TINY,
                               split_experts: bool = False) -> Crafted:
    """dOut rows are 1 on even tokens and `odd_scale` on odd ones, with x, g, u the same on every
    token; so a, dg, du and p*D of the odd tokens are `odd_scale` times the even tokens'. Within
    one expert, blocking along tokens flushes the odd tokens' dg, du and p*D: the weight
    gradients are then bit-identical to those with odd_scale = 0. With `split_experts`, even
    tokens go to expert 0 and odd tokens to expert 1 (two local experts): expert 1's blocks hold
    only its own rows, so its weight gradients stay nonzero."""
    x = np.zeros((N, H)); x[:, 0] = 1.0
    wg = np.zeros((I, H)); wg[:, 0] = 1.0
    wu = np.zeros((I, H)); wu[:, 0] = 1.0
    dout = np.where(_even(N)[:, None], 1.0, odd_scale) * np.ones((N, H))
    wd = np.ones((H, I))
    if not split_experts:
        return _single(x, dout, wg, wu, wd)
    logits = np.zeros((N, 2), np.float32)
    logits[_even(N), 0] = 1.0
    logits[~_even(N), 1] = 1.0
    return Crafted(x, dout, logits, np.stack([wg, wg]), np.stack([wu, wu]), np.stack([wd, wd]))


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """BF16 bit patterns of values that are exactly representable in BF16 (asserted)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    assert np.array_equal(f.astype(np.float64), np.asarray(a, dtype=np.float64))
    u = f.view(np.uint32)
    assert not (u & 0xFFFF).any(), "value not exact in BF16"
    return (u >> 16).astype(np.uint16)


# Gate of expert 0 in precision_ties: p0 = 0.5322, just above 272/512 (a tie of the E4M3 grid
# at scale 2^-9) and below the next BF16 value after it.
P0 = 0.5322


def precision_ties(N: int = 64) -> Crafted:
    """Values that sit between an E4M3 rounding tie and the next BF16 number above it, so that
    quantising the fp32 value rounds up while rounding to BF16 first lands on the tie and rounds
    to even (down). Two experts, K = 2, every token routed to both: p0 = P0 for expert 0 and
    1 - P0 for expert 1; x = e_0; dOut = e_0 + e_1.
      expert 0: g = 6, u = 1 (h = silu(6) -> 6.0 after quantisation), a = 0.1669921875 (Wd rows
                0 and 1 = 0.15625 and 0.0107421875, one E4M3 grid), so du = P0 a silu(6) and
                p D = P0 both sit at 272.3 / 512; Wu column 7 (x_7 = 0) carries du to dX[:, 7].
      expert 1: g = 0 (Wg column 9, x_9 = 0), u = 1, a = 2.2734375, so dg = (1 - P0) a / 2 sits at
                272.25 / 512; Wg column 9 carries it to dX[:, 9].
    Quantised from fp32 each of these becomes 288 / 512 = 0.5625 (from BF16: 256 / 512 = 0.5):
      dWd_0[0:2, :] = N * 0.5625 * 6 = 216;  dWu_0[:, 0] = N * 0.5625 = 36;
      dWg_1[:, 0] = N * 0.5625 = 36;  dX[:, 7] = dX[:, 9] = I * 0.5625 = 72."""
    c = np.float32(np.log(P0 / (1.0 - P0)))
    logits = np.zeros((N, 2), np.float32); logits[:, 0] = c
    x = np.zeros((N, H)); x[:, 0] = 1.0
    dout = np.zeros((N, H)); dout[:, 0] = 1.0; dout[:, 1] = 1.0
    wg = np.zeros((2, I, H)); wu = np.zeros((2, I, H)); wd = np.zeros((2, H, I))
    wg[0, :, 0] = 6.0; wu[0, :, 0] = 1.0; wu[0, :, 7] = 1.0
    wd[0, 0, :] = 0.15625; wd[0, 1, :] = 0.0107421875
    wg[1, :, 9] = 1.0; wu[1, :, 0] = 1.0
    wd[1, 0, :] = 2.25; wd[1, 1, :] = 0.0234375
    return Crafted(x, dout, logits, wg, wu, wd, K=2)
