"""Forward and backward of one GPU's share of the deterministic fused MoE layer, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain numpy, no blocking, no fusion:
each step is the definition written out, in the order the pages describe the layer.

Stage order, forward: router decision -> dispatch -> grouped GEMM -> combine back, then the
final weighted merge ("把 MoE 通信延迟从 103μs 压到 18μs", section 02 on MoE's communication
tax, and section 04 on what the layer benchmark covers). Backward mirrors it: pull the
upstream gradient back (reverse combine), SwiGLU backward with the router-weight gradient
computed inside it, push the input gradient back (reverse dispatch) ("Mixture-of-Kittens
(MoK)", sections on pull dispatch and on benchmarks; "Cursor Open-Sources Mixture-of-Kittens
(MoK)", Technical Details).

Notation: N source tokens (S segments of T), hidden H, E experts, top-k K, expert
intermediate I, local experts [e0, e0+E_loc). A pair id is n*K + k. Weights are stored with
the reduction axis contiguous: Wg, Wu [E_loc][I][H], Wd [E_loc][H][I]; so g = x Wg^T,
u = x Wu^T, y = h Wd^T.

Readings of points the pages leave open:

* gating is a softmax over the K selected logits (the tiny workload states it; no scaling);
* top-k orders experts by descending logit, ties to the lower expert id, -0.0 == +0.0;
* rows of one expert are placed in ascending token id;
* a token with no local expert gets no output row (the cross-GPU sum is out of scope);
* the oracle rounds no intermediate in BF16 mode; in MXFP8 mode it applies the quantiser at
  every GEMM operand, blocked along that GEMM's reduction axis.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from . import mx


# ---------------------------------------------------------------------------------------------
# Storage decoding (inputs arrive as BF16 bit patterns).

def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """BF16 bit patterns -> float64 (exact: BF16 is the top half of an fp32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# O0: the router's gate projection, the step before top-k, and its backward. The pages compute
# the router-weight gradient as part of the layer, SonicMoE-style, inside SwiGLU backward
# ("Mixture-of-Kittens (MoK)", benchmark section; "Cursor Open-Sources Mixture-of-Kittens
# (MoK)", Technical Details): dp comes out of SwiGLU backward, the top-k softmax backward turns
# it into dlogits (O13), and the projection's chain rule carries dlogits into W_r and X.

def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """logits[n, e] = sum_h x[n, h] wr[e, h] (fp64); wr is [E][H]."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(wr, dtype=np.float64).T


def router_backward(x: np.ndarray, wr: np.ndarray, dlogits: np.ndarray):
    """Chain rule of the projection: dW_r = dlogits^T x ([E][H]) and the router's share of the
    input gradient, dlogits wr ([N][H])."""
    dl = np.asarray(dlogits, dtype=np.float64)
    return dl.T @ np.asarray(x, dtype=np.float64), dl @ np.asarray(wr, dtype=np.float64)


# ---------------------------------------------------------------------------------------------
# O1 + O2: router top-k and gating.
# The router picks K experts per token anew every step, which is why per-expert loads are
# dynamic ("把 MoE 通信延迟从 103μs 压到 18μs", section 02).

def topk_gating(logits: np.ndarray, K: int):
    """Top-k experts per token and their softmax gating weights.

    Experts are ordered by (-logit, expert id) ascending: the largest logit first, equal
    logits to the lower id. p_k = exp(l_k - l_0) / sum_j exp(l_j - l_0) over the K selected
    logits, in fp64. Returns (idx int64 [N][K], p float64 [N][K]).
    """
    l = np.asarray(logits, dtype=np.float64)
    # A stable sort of -l keeps equal keys in ascending expert order; -0.0 and +0.0 compare
    # equal, so they are ties too.
    order = np.argsort(-l, axis=1, kind="stable")
    idx = order[:, :K].astype(np.int64)
    sel = np.take_along_axis(l, idx, axis=1)
    z = np.exp(sel - sel[:, :1])
    p = z / z.sum(axis=1, keepdims=True)
    return idx, p


# ---------------------------------------------------------------------------------------------
# O3: the schedule table. One table serves dispatch, combine and their backward mirrors: it
# counts the tokens each local expert receives, fixes each pair's row on the receiving side,
# and keeps an expert's rows contiguous ("Mixture-of-Kittens (MoK)", section on pull
# dispatch; "把 MoE 通信延迟从 103μs 压到 18μs", sections 02 and 03 part ①).

@dataclasses.dataclass
class Schedule:
    counts: np.ndarray     # int64 [E_loc]
    offsets: np.ndarray    # int64 [E_loc+1], exclusive prefix sum (with optional row padding)
    perm: np.ndarray       # int64 [rows]: expert-order row -> pair id n*K+k, -1 for pad rows
    tokpos: np.ndarray     # int64 [N*K]: pair id -> row, -1 for non-local pairs
    P: int                 # local pairs
    rows: int              # rows in expert order (P, plus padding when aligned)
    touched: np.ndarray    # int64 [U]: tokens with at least one local pair, ascending
    M: Optional[int] = None
    J: Optional[int] = None


def schedule(idx: np.ndarray, e0: int, E_loc: int, M: Optional[int] = None,
             row_align: int = 1) -> Schedule:
    """Build the schedule table from the router's choices.

    count[e] = number of (n, k) with idx[n, k] = e0 + e; rows for expert e are its pairs in
    ascending n (a token picks an expert at most once, so k is implied). With row_align > 1
    each expert's row range starts at a multiple of row_align (pad rows carry pair -1).
    Minibatch j covers rows [j*M, min(rows, (j+1)*M)).
    """
    idx = np.asarray(idx)
    N, K = idx.shape
    counts = np.array([(idx == e0 + e).sum() for e in range(E_loc)], dtype=np.int64)
    padded = ((counts + row_align - 1) // row_align) * row_align
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    rows = int(offsets[-1])
    perm = np.full(rows, -1, dtype=np.int64)
    tokpos = np.full(N * K, -1, dtype=np.int64)
    for e in range(E_loc):
        ns, ks = np.nonzero(idx == e0 + e)        # row-major order: ascending n
        pairs = ns * K + ks
        r = offsets[e] + np.arange(len(pairs))
        perm[r] = pairs
        tokpos[pairs] = r
    local = (idx >= e0) & (idx < e0 + E_loc)
    touched = np.nonzero(local.any(axis=1))[0].astype(np.int64)
    J = None if M is None else -(-rows // M)
    return Schedule(counts, offsets, perm, tokpos, int(counts.sum()), rows, touched, M, J)


def minibatch_rows(sched: Schedule, j: int):
    """Rows of minibatch j (ring slot j mod R)."""
    return range(j * sched.M, min(sched.rows, (j + 1) * sched.M))


# ---------------------------------------------------------------------------------------------
# Helpers for the expert FFN.

def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def _q32(v: np.ndarray) -> np.ndarray:
    """Round a computed value to fp32, the precision the kernels hold it in before they
    quantise it (so both sides take the quantisation decision at the same precision)."""
    return np.asarray(v, dtype=np.float32).astype(np.float64)


@dataclasses.dataclass
class Weights:
    """Local expert weights as float64 values, and how each GEMM sees them.

    BF16 mode: every view is the decoded BF16 master. MXFP8 mode: each GEMM's weight operand
    is quantised from the BF16 master along that GEMM's reduction axis.
    """
    wg: np.ndarray          # [E_loc][I][H] masters
    wu: np.ndarray
    wd: np.ndarray          # [E_loc][H][I]
    dtype: str = "bf16"

    def fwd_gate(self):     # g = x Wg^T: reduction over H
        return self.wg if self.dtype == "bf16" else mx.fake_quant(self.wg, axis=2)

    def fwd_up(self):
        return self.wu if self.dtype == "bf16" else mx.fake_quant(self.wu, axis=2)

    def fwd_down(self):     # y = h Wd^T: reduction over I
        return self.wd if self.dtype == "bf16" else mx.fake_quant(self.wd, axis=2)

    def bwd_down(self):     # a = D Wd: reduction over H
        return self.wd if self.dtype == "bf16" else mx.fake_quant(self.wd, axis=1)

    def bwd_gate(self):     # dx = dg Wg: reduction over I
        return self.wg if self.dtype == "bf16" else mx.fake_quant(self.wg, axis=1)

    def bwd_up(self):
        return self.wu if self.dtype == "bf16" else mx.fake_quant(self.wu, axis=1)


def weights_from_bits(w: dict, dtype: str = "bf16") -> Weights:
    return Weights(decode_bf16(w["wg"]), decode_bf16(w["wu"]), decode_bf16(w["wd"]), dtype)


# ---------------------------------------------------------------------------------------------
# Forward.

@dataclasses.dataclass
class Forward:
    idx: np.ndarray
    p: np.ndarray
    sched: Schedule
    xd: np.ndarray          # [rows][H] dispatched rows (as the GEMM sees them)
    g: np.ndarray           # [rows][I]
    u: np.ndarray
    h: np.ndarray           # [rows][I] as the down GEMM sees it
    y: np.ndarray           # [rows][H] expert outputs (unweighted)
    out: np.ndarray         # [U][H] merged outputs for sched.touched
    x_rows: np.ndarray      # [rows][H] dispatched rows before any quantisation


def dispatch(x_rows_of_pairs: np.ndarray, dtype: str) -> np.ndarray:
    """O4, pull dispatch: the receiving side reads each routed token's row itself and lays
    the rows out in expert order ("Mixture-of-Kittens (MoK)", section on pull dispatch;
    "把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ①). In MXFP8 mode the row is
    quantised along H on the way (section 03 part ③)."""
    if dtype == "bf16":
        return x_rows_of_pairs
    return mx.fake_quant(x_rows_of_pairs, axis=1)


def expert_ffn(xd: np.ndarray, sched: Schedule, W: Weights):
    """O5-O7, grouped SwiGLU expert FFN over each expert's contiguous rows.

    g = xd Wg_e^T, u = xd Wu_e^T, h = silu(g) * u, y = h Wd_e^T. MXFP8: h is quantised
    along I before the down GEMM (SwiGLU fused quantisation, section 03 part ③ of
    "把 MoE 通信延迟从 103μs 压到 18μs")."""
    rows, H = xd.shape
    I = W.wg.shape[1]
    g = np.zeros((rows, I)); u = np.zeros((rows, I)); h = np.zeros((rows, I))
    y = np.zeros((rows, H))
    Wg, Wu, Wd = W.fwd_gate(), W.fwd_up(), W.fwd_down()
    for e in range(len(sched.counts)):
        r = slice(int(sched.offsets[e]), int(sched.offsets[e]) + int(sched.counts[e]))
        g[r] = xd[r] @ Wg[e].T
        u[r] = xd[r] @ Wu[e].T
        he = silu(g[r]) * u[r]
        if W.dtype != "bf16" and he.shape[0]:
            he = mx.fake_quant(_q32(he), axis=1)
        h[r] = he
        y[r] = he @ Wd[e].T
    return g, u, h, y


def combine(y: np.ndarray, idx: np.ndarray, weight: Optional[np.ndarray], sched: Schedule,
            e0: int, E_loc: int) -> np.ndarray:
    """O8, push combine + final weighted merge.

    The expert side writes each result to its token's receive slot (pair id); the merge then
    sums, for each touched token n, weight[n,k] * y[tokpos(n*K+k)] over k ascending with
    idx[n,k] local ("把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ① and section 04).
    weight=None gives the unweighted sum (the input-gradient merge in backward).
    Returns [U][H] for the tokens in sched.touched.
    """
    N, K = idx.shape
    H = y.shape[1]
    out = np.zeros((len(sched.touched), H))
    for u_i, n in enumerate(sched.touched):
        acc = np.zeros(H)
        for k in range(K):
            if e0 <= idx[n, k] < e0 + E_loc:
                w = 1.0 if weight is None else weight[n, k]
                acc = acc + w * y[sched.tokpos[n * K + k]]
        out[u_i] = acc
    return out


def bf16_rows(source):
    """Row fetcher over BF16 bits: ``source`` is a [N][H] uint16 array or a function of token
    ids returning such rows. Returns ``fetch(token_ids) -> float64 [len][H]``."""
    if callable(source):
        return lambda rows: decode_bf16(source(rows))
    return lambda rows: decode_bf16(np.asarray(source)[rows])


def forward(x_fn, logits: np.ndarray, W: Weights, K: int, e0: int, E_loc: int,
            M: Optional[int] = None, row_align: int = 1) -> Forward:
    """Whole forward. ``x_fn(token_ids) -> float64 [len][H]`` fetches source rows (see
    ``bf16_rows``), so large workloads only decode the rows that are routed here."""
    idx, p = topk_gating(logits, K)
    sched = schedule(idx, e0, E_loc, M, row_align)
    H = W.wg.shape[2]
    x_rows = np.zeros((sched.rows, H))
    real = sched.perm >= 0
    if real.any():
        x_rows[real] = x_fn(sched.perm[real] // K)
    xd = dispatch(x_rows, W.dtype)
    if W.dtype != "bf16":
        xd[~real] = 0.0
    g, u, h, y = expert_ffn(xd, sched, W)
    out = combine(y, idx, p, sched, e0, E_loc)
    return Forward(idx, p, sched, xd, g, u, h, y, out, x_rows)


# ---------------------------------------------------------------------------------------------
# Backward of L = sum_n <dOut[n], out[n]>.

@dataclasses.dataclass
class Backward:
    dx: np.ndarray          # [U][H] input gradient for sched.touched
    dp: np.ndarray          # [N][K] router-weight gradient at local pairs (0 elsewhere)
    dwg: np.ndarray         # [E_loc][I][H]
    dwu: np.ndarray
    dwd: np.ndarray         # [E_loc][H][I]
    dlogits: Optional[np.ndarray]   # [N][E] when all experts are local, else None
    a: np.ndarray           # [rows][I] = D Wd_e
    dg: np.ndarray
    du: np.ndarray


def backward(fw: Forward, dout_fn, W: Weights, K: int, e0: int, E_loc: int,
             E: int) -> Backward:
    """O9-O13.

    O9  reverse combine: pull dOut rows for every local pair, D[r] = dOut[n(r)].
    O10 a = D Wd_e; router-weight gradient dp = <a, h> (equal to <dOut[n], y_r>), computed
        inside SwiGLU backward together with dh = p a,
        dg = dh * u * s(g) * (1 + g (1 - s(g))), du = dh * silu(g)
        ("Mixture-of-Kittens (MoK)", benchmark section; "Cursor Open-Sources
        Mixture-of-Kittens (MoK)", Technical Details).
    O11 dx_r = dg_r Wg_e + du_r Wu_e, pushed back and merged over k ascending.
    O12 dWg_e = sum_r dg_r^T x_r, dWu_e likewise, dWd_e = sum_r (p_r D_r)^T h_r.
    O13 when E_loc = E: s = sum_k p_k dp_k, dlogit[n, idx_k] = p_k (dp_k - s).
    """
    sched, idx, p = fw.sched, fw.idx, fw.p
    N = idx.shape[0]
    H = W.wg.shape[2]
    I = W.wg.shape[1]
    mxm = W.dtype != "bf16"
    real = sched.perm >= 0
    n_of = np.where(real, sched.perm // K, 0)
    k_of = np.where(real, sched.perm % K, 0)
    p_row = np.where(real, p[n_of, k_of], 0.0)
    D0 = np.zeros((sched.rows, H))
    if real.any():
        D0[real] = dout_fn(sched.perm[real] // K)
    D = mx.fake_quant(D0, axis=1) if mxm else D0
    Wd_b, Wg_b, Wu_b = W.bwd_down(), W.bwd_gate(), W.bwd_up()
    a = np.zeros((sched.rows, I)); dg = np.zeros_like(a); du = np.zeros_like(a)
    dxr = np.zeros((sched.rows, H))
    dp_row = np.zeros(sched.rows)
    dwg = np.zeros_like(W.wg); dwu = np.zeros_like(W.wu); dwd = np.zeros_like(W.wd)
    for e in range(E_loc):
        lo = int(sched.offsets[e]); c = int(sched.counts[e])
        r = slice(lo, lo + c)
        if c == 0:
            continue
        a[r] = D[r] @ Wd_b[e]
        dp_row[r] = (a[r] * fw.h[r]).sum(axis=1)
        dh = p_row[r][:, None] * a[r]
        sg = sigmoid(fw.g[r])
        dg[r] = dh * fw.u[r] * sg * (1.0 + fw.g[r] * (1.0 - sg))
        du[r] = dh * fw.g[r] * sg
        if mxm:
            dg_q = mx.fake_quant(_q32(dg[r]), axis=1)
            du_q = mx.fake_quant(_q32(du[r]), axis=1)
            dxr[r] = dg_q @ Wg_b[e] + du_q @ Wu_b[e]
            xs = mx.fake_quant_rows_padded(fw.x_rows[r])
            dwg[e] = mx.fake_quant_rows_padded(_q32(dg[r])).T @ xs
            dwu[e] = mx.fake_quant_rows_padded(_q32(du[r])).T @ xs
            dwd[e] = (mx.fake_quant_rows_padded(_q32(p_row[r][:, None] * D0[r])).T
                      @ mx.fake_quant_rows_padded(fw.h[r]))
        else:
            dxr[r] = dg[r] @ Wg_b[e] + du[r] @ Wu_b[e]
            dwg[e] = dg[r].T @ fw.xd[r]
            dwu[e] = du[r].T @ fw.xd[r]
            dwd[e] = (p_row[r][:, None] * D[r]).T @ fw.h[r]
    dx = combine(dxr, idx, None, sched, e0, E_loc)
    dp = np.zeros((N, K))
    dp.reshape(-1)[sched.perm[real]] = dp_row[real]
    dlogits = None
    if E_loc == E:
        s = (p * dp).sum(axis=1, keepdims=True)
        dl_sel = p * (dp - s)
        dlogits = np.zeros((N, E))
        np.put_along_axis(dlogits, idx, dl_sel, axis=1)
    return Backward(dx, dp, dwg, dwu, dwd, dlogits, a, dg, du)


def expert_wgrad_rows(x_rows: np.ndarray, dout_rows: np.ndarray, p_rows: np.ndarray, W: Weights,
                      e: int, gi, hi, workers: int = 1):
    """Rows ``gi`` of dWg_e and dWu_e and rows ``hi`` of dWd_e, from expert e's rows alone.

    x_rows, dout_rows: [R][H] the values of the source rows of expert e's pairs in schedule
    order (ascending token id), p_rows: [R] their gates. Same definitions as ``backward`` (O9-O12),
    restricted to the requested rows: row i of dWg_e and dWu_e needs column i of dg and du only,
    and row j of dWd_e column j of p*D and the whole h. In MXFP8 mode the weight-gradient
    operands are blocked along tokens, so quantising one column alone gives the same values as
    quantising the whole operand. ``workers`` parallelises the quantiser over slices.
    Returns (dWg rows [len(gi)][H], dWu rows, dWd rows [len(hi)][I])."""
    mxm = W.dtype != "bf16"
    gi, hi = np.asarray(gi), np.asarray(hi)
    xd = mx.fake_quant(x_rows, axis=1, workers=workers) if mxm else x_rows
    Wg, Wu = W.fwd_gate()[e], W.fwd_up()[e]
    D = mx.fake_quant(dout_rows, axis=1, workers=workers) if mxm else dout_rows
    # dg, du at columns gi (O10)
    g = xd @ Wg[gi].T
    u = xd @ Wu[gi].T
    a = D @ W.bwd_down()[e][:, gi]
    dh = p_rows[:, None] * a
    sg = sigmoid(g)
    dg = dh * u * sg * (1.0 + g * (1.0 - sg))
    du = dh * g * sg
    # the whole h of the expert's rows (O5-O6)
    gf = xd @ Wg.T
    hf = silu(gf) * (xd @ Wu.T)
    if mxm:
        hf = mx.fake_quant(_q32(hf), axis=1, workers=workers)
    pD = p_rows[:, None] * dout_rows[:, hi]
    if mxm:
        xs = mx.fake_quant_rows_padded(x_rows, workers=workers)
        dwg = mx.fake_quant_rows_padded(_q32(dg)).T @ xs
        dwu = mx.fake_quant_rows_padded(_q32(du)).T @ xs
        dwd = mx.fake_quant_rows_padded(_q32(pD)).T @ mx.fake_quant_rows_padded(hf, workers=workers)
    else:
        dwg = dg.T @ xd
        dwu = du.T @ xd
        dwd = pD.T @ hf
    return dwg, dwu, dwd


def loss(fw: Forward, dout: np.ndarray) -> float:
    """L = sum over touched tokens of <dOut[n], out[n]> (dout indexed by token id)."""
    return float((dout[fw.sched.touched] * fw.out).sum())
