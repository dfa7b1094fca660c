"""Pins for the CPU oracle: it is checked against things other than itself.

* the MXFP8 quantiser against hand-worked spec examples (tests/golden) and an exhaustive
  nearest-value search;
* top-k and gating against a pure-Python sort, closed forms and ties;
* the schedule table against its invariants and the brute force;
* forward and backward against the pure-Python brute force, special cases with closed forms
  (a single expert, all experts selected, identical experts), a dense masked computation, and
  central finite differences of the loss.
"""
import json
import math
import os

import numpy as np
import pytest

import datagen
from oracle import brute, mx
from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------ MXFP8 quantiser

def test_mx_spec_worked_examples():
    spec = json.load(open(os.path.join(GOLDEN, "mx_spec_examples.json")))
    for case in spec["block_cases"]:
        head = case["block_head"]
        block = np.zeros(32)
        block[:len(head)] = head
        codes, scales = mx.quantize(block[None, :], axis=1)
        assert int(scales[0, 0]) == case["scale"], case["note"]
        assert [int(c) for c in codes[0, :len(head)]] == case["codes_head"], case["note"]
    for case in spec["decode_cases"]:
        assert mx.e4m3_decode(np.array([case["code"]]))[0] == case["value"]


def _all_e4m3_values():
    codes = np.arange(256)
    vals = mx.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    return codes[ok], vals[ok]


def test_e4m3_roundtrip_all_codes():
    codes, vals = _all_e4m3_values()
    assert len(codes) == 254
    back = mx.e4m3_encode(vals)
    # +0 and -0 both decode to zero; every other code must come back exactly.
    assert np.array_equal(back, codes.astype(np.uint8))


def test_e4m3_encode_is_nearest_even_by_exhaustive_search():
    rng = np.random.default_rng(1)
    pos_codes = np.arange(0, 127)             # 0x00 .. 0x7E
    pos_vals = mx.e4m3_decode(pos_codes)
    x = np.concatenate([rng.uniform(0, 460, 4000), rng.uniform(0, 0.05, 4000),
                        pos_vals, (pos_vals[1:] + pos_vals[:-1]) / 2])   # ties included
    got = mx.e4m3_encode(x)
    for xi, gi in zip(x, got):
        d = np.abs(pos_vals - min(xi, 448.0))
        best = np.nonzero(d == d.min())[0]
        if len(best) == 1:
            want = pos_codes[best[0]]
        else:  # tie: even mantissa (lowest bit of the code clear)
            want = [c for c in pos_codes[best] if c % 2 == 0][0]
        assert gi == want, (xi, gi, want)


def test_mx_quantize_scale_rule_and_idempotence():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    codes, scales = mx.quantize(v, axis=1)
    blocks = np.abs(v).reshape(64, 8, 32).max(axis=2)
    want = np.floor(np.log2(blocks)).astype(int) - 8 + 127
    assert np.array_equal(scales.astype(int), want)
    dq = mx.dequantize(codes, scales, axis=1)
    assert np.all(np.abs(dq) <= 448.0 * np.exp2(scales.astype(float) - 127).repeat(32, axis=1))
    c2, s2 = mx.quantize(dq, axis=1)
    assert np.array_equal(mx.dequantize(c2, s2, axis=1), dq)
    # Relative error of each element is at most half a mantissa step (2^-4) unless it
    # saturated or fell into the subnormal range.
    scale = np.exp2(scales.astype(float) - 127).repeat(32, axis=1)
    normal = (np.abs(v) / scale >= 2.0 ** -6) & (np.abs(v) / scale <= 448)
    rel = np.abs(dq - v)[normal] / np.abs(v)[normal]
    assert rel.max() <= 2.0 ** -4 + 1e-12


def test_mx_quantize_along_other_axis_matches_transpose():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((96, 64))
    c0, s0 = mx.quantize(v, axis=0)
    c1, s1 = mx.quantize(v.T.copy(), axis=1)
    assert np.array_equal(c0, c1.T) and np.array_equal(s0, s1.T)


# ------------------------------------------------------------------------------ top-k + gating

def test_topk_matches_sorted_brute_force():
    rng = np.random.default_rng(4)
    for E, K in ((8, 2), (16, 5), (64, 8)):
        l = rng.choice(np.array([-1.0, 0.0, -0.0, 0.5, 2.0], dtype=np.float32), (2500, E))
        l2 = rng.standard_normal((2500, E)).astype(np.float32)
        for L in (l, l2):
            idx, p = mo.topk_gating(L, K)
            for n in range(0, len(L), 7):
                want = brute.topk(L[n].tolist(), K)
                assert idx[n].tolist() == want
                pw = brute.softmax([float(L[n][e]) for e in want])
                assert np.allclose(p[n], pw, rtol=0, atol=1e-15)


def test_topk_closed_forms_and_ties():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((1000, 8)).astype(np.float32)
    idx1, p1 = mo.topk_gating(l, 1)
    assert np.all(p1 == 1.0) and np.array_equal(idx1[:, 0], l.argmax(axis=1))
    idx2, p2 = mo.topk_gating(l, 2)
    l0 = np.take_along_axis(l, idx2[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(l, idx2[:, 1:], 1)[:, 0].astype(np.float64)
    assert np.allclose(p2[:, 0], 1.0 / (1.0 + np.exp(-(l0 - l1))), atol=1e-15)
    _, p8 = mo.topk_gating(l, 8)
    assert np.allclose(p8.sum(axis=1), 1.0, atol=1e-12)
    # All-equal logits pick experts 0..K-1 with equal weight.
    idx, p = mo.topk_gating(np.zeros((3, 10), np.float32), 4)
    assert np.array_equal(idx, np.tile(np.arange(4), (3, 1))) and np.allclose(p, 0.25)
    # -0.0 and +0.0 tie: lower id first.
    idx, _ = mo.topk_gating(np.array([[0.0, -0.0, -1.0], [-0.0, 0.0, -1.0]], np.float32), 2)
    assert idx.tolist() == [[0, 1], [0, 1]]


# ------------------------------------------------------------------------------ schedule

def _check_schedule_invariants(idx, s, e0, E_loc):
    N, K = idx.shape
    local = (idx >= e0) & (idx < e0 + E_loc)
    P = int(local.sum())
    assert s.P == P and s.counts.sum() == P
    assert np.all(np.diff(s.offsets) >= s.counts)
    real = s.perm[s.perm >= 0]
    # Each local (token, expert) pair is dispatched exactly once.
    assert len(real) == P and len(np.unique(real)) == P
    assert set(real.tolist()) == set(np.nonzero(local.reshape(-1))[0].tolist())
    assert np.array_equal(s.tokpos[real], np.nonzero(s.perm >= 0)[0])
    assert np.all(s.tokpos[~local.reshape(-1)] == -1)
    for e in range(E_loc):
        rows = s.perm[s.offsets[e]:s.offsets[e] + s.counts[e]]
        assert np.all(idx.reshape(-1)[rows] == e0 + e)
        assert np.all(np.diff(rows // K) > 0)          # ascending token id
    assert np.array_equal(s.touched, np.nonzero(local.any(axis=1))[0])


def test_schedule_invariants_and_brute_force():
    cfg = datagen.CONFIGS["tiny"]
    idx, _ = mo.topk_gating(datagen.logits(cfg), cfg.K)
    for e0, E_loc, align in ((0, 8, 1), (2, 3, 1), (0, 8, 32), (5, 3, 4)):
        s = mo.schedule(idx, e0, E_loc, M=16, row_align=align)
        _check_schedule_invariants(idx, s, e0, E_loc)
        assert np.all(s.offsets % align == 0)
        assert s.J == -(-s.rows // 16)
        # Brute force: the same pairs per expert, in the same order.
        for e in range(E_loc):
            want = [n * cfg.K + k for n in range(cfg.N) for k in range(cfg.K)
                    if idx[n, k] == e0 + e]
            assert s.perm[s.offsets[e]:s.offsets[e] + s.counts[e]].tolist() == want


def test_schedule_degenerate_cases():
    idx = np.array([[3, 4], [4, 5]])
    s = mo.schedule(idx, 0, 2, M=4)                    # no local pairs
    assert s.P == 0 and s.rows == 0 and len(s.touched) == 0 and s.J == 0
    idx = np.tile(np.array([[1, 0]]), (37, 1))          # every token routed to both experts
    s = mo.schedule(idx, 0, 2, M=16)
    assert s.counts.tolist() == [37, 37] and s.J == 5
    _check_schedule_invariants(idx, s, 0, 2)


def test_schedule_counts_near_balanced_at_dsv3_shape():
    cfg = datagen.CONFIGS["dsv3"].replace(S=8)
    idx, _ = mo.topk_gating(datagen.logits(cfg), cfg.K)
    s = mo.schedule(idx, cfg.e0, cfg.E_loc)
    mean = cfg.N * cfg.K / cfg.E
    assert np.all(np.abs(s.counts - mean) < 6 * math.sqrt(mean))
    _check_schedule_invariants(idx, s, cfg.e0, cfg.E_loc)


def test_zipf_skew_in_range():
    cfg = datagen.CONFIGS["kimi_mx_skew"].replace(S=4)
    idx, _ = mo.topk_gating(datagen.logits(cfg), cfg.K)
    local = ((idx >= cfg.e0) & (idx < cfg.e0 + cfg.E_loc)).sum()
    skew = (local / cfg.E_loc) / (cfg.N * cfg.K / cfg.E)
    assert 4.0 <= skew <= 8.0


# ------------------------------------------------------------------------------ layer vs brute

def _small(N=24, H=32, I=64, E=8, K=2, seed=11, x_std=0.5, w_std=0.3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((N, H)) * x_std
    L = rng.standard_normal((N, E)).astype(np.float32)
    Wg = rng.standard_normal((E, I, H)) * w_std
    Wu = rng.standard_normal((E, I, H)) * w_std
    Wd = rng.standard_normal((E, H, I)) * w_std
    dO = rng.standard_normal((N, H))
    return X, L, Wg, Wu, Wd, dO


def _run_oracle(X, L, Wg, Wu, Wd, dO, K, e0, E_loc, E, M=5):
    W = mo.Weights(Wg[e0:e0 + E_loc], Wu[e0:e0 + E_loc], Wd[e0:e0 + E_loc])
    fw = mo.forward(lambda r: X[r], L, W, K, e0, E_loc, M)
    bw = mo.backward(fw, lambda r: dO[r], W, K, e0, E_loc, E)
    return fw, bw


def _brute(X, L, Wg, Wu, Wd, dO, K, e0, E_loc):
    return brute.layer(X.tolist(), L.tolist(), Wg[e0:e0 + E_loc].tolist(),
                       Wu[e0:e0 + E_loc].tolist(), Wd[e0:e0 + E_loc].tolist(), dO.tolist(),
                       K, e0, E_loc)


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (3, 2)])
def test_layer_matches_brute_force(e0, E_loc):
    X, L, Wg, Wu, Wd, dO = _small()
    N, K, E = X.shape[0], 2, 8
    fw, bw = _run_oracle(X, L, Wg, Wu, Wd, dO, K, e0, E_loc, E)
    b = _brute(X, L, Wg, Wu, Wd, dO, K, e0, E_loc)
    assert fw.idx.tolist() == b["idx"]
    assert np.allclose(fw.p, b["p"], atol=1e-14)
    touched = [n for n in range(N) if b["out"][n] is not None]
    assert fw.sched.touched.tolist() == touched
    assert np.allclose(fw.out, np.array([b["out"][n] for n in touched]), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw.dx, np.array([b["dX"][n] for n in touched]), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw.dp, np.array(b["dp"]), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw.dwg, np.array(b["dWg"]), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw.dwu, np.array(b["dWu"]), rtol=1e-12, atol=1e-12)
    assert np.allclose(bw.dwd, np.array(b["dWd"]), rtol=1e-12, atol=1e-12)
    if E_loc == E:
        assert np.allclose(bw.dlogits, np.array(b["dlogits"]), rtol=1e-12, atol=1e-12)
    else:
        assert bw.dlogits is None


def _ffn(x, wg, wu, wd):
    g = x @ wg.T
    return (g / (1 + np.exp(-g)) * (x @ wu.T)) @ wd.T


def test_single_expert_is_plain_swiglu_ffn():
    X, L, Wg, Wu, Wd, dO = _small(E=1)
    fw, _ = _run_oracle(X, L[:, :1], Wg, Wu, Wd, dO, 1, 0, 1, 1)
    assert np.allclose(fw.out, _ffn(X, Wg[0], Wu[0], Wd[0]), rtol=1e-12, atol=1e-12)


def test_all_experts_selected_is_dense_softmax_mixture():
    X, L, Wg, Wu, Wd, dO = _small(E=4)
    fw, _ = _run_oracle(X, L[:, :4], Wg, Wu, Wd, dO, 4, 0, 4, 4)
    l = L[:, :4].astype(np.float64)
    sm = np.exp(l - l.max(1, keepdims=True)); sm /= sm.sum(1, keepdims=True)
    dense = sum(sm[:, e:e + 1] * _ffn(X, Wg[e], Wu[e], Wd[e]) for e in range(4))
    assert np.allclose(fw.out, dense, rtol=1e-12, atol=1e-12)


def test_dense_masked_equals_dispatched():
    X, L, Wg, Wu, Wd, dO = _small(N=40)
    K, e0, E_loc = 2, 2, 4
    fw, _ = _run_oracle(X, L, Wg, Wu, Wd, dO, K, e0, E_loc, 8)
    # Every local expert on every token, then masked by the routing weights.
    mask = np.zeros((X.shape[0], E_loc))
    for n in range(X.shape[0]):
        for k in range(K):
            if e0 <= fw.idx[n, k] < e0 + E_loc:
                mask[n, fw.idx[n, k] - e0] = fw.p[n, k]
    dense = sum(mask[:, e:e + 1] * _ffn(X, Wg[e0 + e], Wu[e0 + e], Wd[e0 + e])
                for e in range(E_loc))
    assert np.allclose(fw.out, dense[fw.sched.touched], rtol=1e-12, atol=1e-12)


def test_identical_experts_weights_sum_to_softmax_mass():
    X, L, Wg, Wu, Wd, dO = _small(N=30)
    for e in range(8):
        Wg[e], Wu[e], Wd[e] = Wg[0], Wu[0], Wd[0]
    for e0, E_loc in ((0, 8), (1, 3)):
        fw, _ = _run_oracle(X, L, Wg, Wu, Wd, dO, 2, e0, E_loc, 8)
        local = (fw.idx >= e0) & (fw.idx < e0 + E_loc)
        mass = (fw.p * local).sum(axis=1)[fw.sched.touched]
        if E_loc == 8:
            assert np.allclose(mass, 1.0)
        want = mass[:, None] * _ffn(X[fw.sched.touched], Wg[0], Wu[0], Wd[0])
        assert np.allclose(fw.out, want, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------------------ finite differences

def _loss(X, L, Wg, Wu, Wd, dO, K, e0, E_loc):
    W = mo.Weights(Wg[e0:e0 + E_loc], Wu[e0:e0 + E_loc], Wd[e0:e0 + E_loc])
    fw = mo.forward(lambda r: X[r], L, W, K, e0, E_loc)
    return mo.loss(fw, dO)


def test_gradients_match_central_finite_differences():
    cfg = datagen.CONFIGS["tiny"]
    X = mo.decode_bf16(datagen.x_all(cfg))
    L = datagen.logits(cfg)
    w = datagen.weights(cfg)
    Wg, Wu, Wd = (mo.decode_bf16(w[k]) for k in ("wg", "wu", "wd"))
    dO = mo.decode_bf16(datagen.dout_all(cfg))
    K, e0, E_loc, E = cfg.K, 0, cfg.E_loc, cfg.E
    fw, bw = _run_oracle(X, L, Wg, Wu, Wd, dO, K, e0, E_loc, E)
    rng = np.random.default_rng(7)
    eps = 1e-6

    def fd(arr, pos, f):
        old = arr[pos]
        arr[pos] = old + eps; lp = f()
        arr[pos] = old - eps; lm = f()
        arr[pos] = old
        return (lp - lm) / (2 * eps)

    f = lambda: _loss(X, L, Wg, Wu, Wd, dO, K, e0, E_loc)
    checks = []
    for _ in range(12):
        n = rng.integers(cfg.N); c = rng.integers(cfg.H)
        u_i = int(np.searchsorted(fw.sched.touched, n))
        checks.append((fd(X, (n, c), f), bw.dx[u_i, c]))
    for arr, grad in ((Wg, bw.dwg), (Wu, bw.dwu), (Wd, bw.dwd)):
        for _ in range(12):
            pos = tuple(rng.integers(s) for s in arr.shape)
            checks.append((fd(arr, pos, f), grad[pos]))
    # Router gradient: logits (skipping tokens whose K-th / (K+1)-th gap is tiny, where top-k
    # is not differentiable).
    Ls = np.sort(L.astype(np.float64), axis=1)[:, ::-1]
    L64 = L.astype(np.float64)
    for _ in range(16):
        n = rng.integers(cfg.N); e = rng.integers(E)
        if Ls[n, K - 1] - Ls[n, K] < 100 * eps:
            continue
        fl = lambda: _loss(X, L64, Wg, Wu, Wd, dO, K, e0, E_loc)
        checks.append((fd(L64, (n, e), fl), bw.dlogits[n, e]))
    for fdv, an in checks:
        assert abs(fdv - an) <= 1e-6 * max(abs(an), 1e-3), (fdv, an)


def test_router_weight_gradient_identity():
    """dp from SwiGLU backward, <a, h>, equals <dOut[n], y_r> computed from the expert output."""
    X, L, Wg, Wu, Wd, dO = _small(N=50)
    fw, bw = _run_oracle(X, L, Wg, Wu, Wd, dO, 2, 0, 8, 8)
    s = fw.sched
    for r in range(s.rows):
        pair = s.perm[r]
        n, k = divmod(int(pair), 2)
        assert np.isclose(bw.dp[n, k], dO[n] @ fw.y[r], rtol=1e-12, atol=1e-12)
    # dp perturbation: dL/dp[n,k] by finite differences on the combine weights.
    n, k = int(s.perm[3] // 2), int(s.perm[3] % 2)
    base = mo.combine(fw.y, fw.idx, fw.p, s, 0, 8)
    p2 = fw.p.copy(); p2[n, k] += 1e-6
    bump = mo.combine(fw.y, fw.idx, p2, s, 0, 8)
    dL = ((bump - base) * dO[s.touched]).sum() / 1e-6
    assert np.isclose(dL, bw.dp[n, k], rtol=1e-6)


# ------------------------------------------------------------------------------ MXFP8 layer

def test_mxfp8_layer_with_exact_inputs_matches_bf16_layer():
    """If every GEMM operand is already representable in its MX blocking the quantiser is the
    identity, so the MXFP8 layer equals the BF16 layer on the same values."""
    rng = np.random.default_rng(9)
    N, H, I, E, K = 40, 64, 64, 4, 2
    # Powers of two with small exponent spread are exact in E4M3 under any block scale
    # whose block maximum is within 2^8 of every element.
    pw = lambda shape: rng.choice([-1.0, 1.0], shape) * np.exp2(rng.integers(-3, 1, shape))
    X = pw((N, H)); Wg = pw((E, I, H)) * 0.125; Wu = pw((E, I, H)) * 0.125
    Wd = pw((E, H, I)) * 0.125
    L = rng.standard_normal((N, E)).astype(np.float32)
    Wb = mo.Weights(Wg, Wu, Wd, "bf16")
    Wm = mo.Weights(Wg, Wu, Wd, "mxfp8")
    assert np.array_equal(Wm.fwd_gate(), Wg) and np.array_equal(Wm.fwd_up(), Wu)
    assert np.array_equal(Wm.fwd_down(), Wd) and np.array_equal(Wm.bwd_down(), Wd)
    assert np.array_equal(Wm.bwd_gate(), Wg) and np.array_equal(Wm.bwd_up(), Wu)
    fb = mo.forward(lambda r: X[r], L, Wb, K, 0, E, 5)
    idx, p = mo.topk_gating(L, K)
    s = mo.schedule(idx, 0, E, 5)
    xd = mo.dispatch(X[s.perm // K], "mxfp8")
    assert np.array_equal(xd, X[s.perm // K])
    g, u, h, y = mo.expert_ffn(xd, s, Wm)
    # h is generally not exact, so the MX output differs from BF16 only through Q_I(h).
    assert np.array_equal(g, fb.g) and np.array_equal(u, fb.u)
    hq = np.asarray(fb.h, dtype=np.float32).astype(np.float64)
    assert np.array_equal(h, mx.fake_quant(hq, axis=1))
    # Error of Q is at most half a mantissa step, or the clip of values in [448, 512) * 2^e.
    assert np.abs(h - fb.h).max() <= 0.125 * np.abs(fb.h).max()
    for e in range(E):
        r = slice(int(s.offsets[e]), int(s.offsets[e + 1]))
        assert np.allclose(y[r], h[r] @ Wd[e].T, rtol=1e-13, atol=1e-13)


def test_mx_blocking_axes_of_weight_views():
    """Each GEMM's weight operand is blocked along that GEMM's reduction axis. Build weights
    that are exact in E4M3 along one axis (equal magnitudes in a block) but not along the
    other (1.0 next to 1.5 * 2^-20, which falls below the smallest subnormal under the
    block's scale), so a wrong axis changes the values."""
    E, I, H = 1, 64, 64
    i = np.arange(I)[:, None]; h = np.arange(H)[None, :]
    spread_i = np.where(i % 2 == 0, 1.0, 1.5 * 2.0 ** -20) * np.ones((I, H))   # varies along I
    spread_h = np.where(h % 2 == 0, 1.0, 1.5 * 2.0 ** -20) * np.ones((I, H))   # varies along H
    W = mo.Weights(spread_i[None], spread_i[None], spread_h.T[None].copy(), "mxfp8")
    # wg [I][H] varies along I only: exact when blocked along H (forward), not along I.
    assert np.array_equal(W.fwd_gate(), W.wg) and not np.array_equal(W.bwd_gate(), W.wg)
    # wd [H][I] = spread_h^T varies along H only: exact along I (forward), not along H.
    assert np.array_equal(W.fwd_down(), W.wd) and not np.array_equal(W.bwd_down(), W.wd)


def test_mxfp8_backward_close_to_bf16_backward():
    """The MXFP8 layer differs from the BF16 layer only by E4M3 rounding (<= 2^-4 per element
    before accumulation), so every output agrees to a few percent; a transposed operand or a
    dropped term would not."""
    cfg = datagen.CONFIGS["tiny"]
    X = mo.decode_bf16(datagen.x_all(cfg)) * 50.0
    L = datagen.logits(cfg)
    w = datagen.weights(cfg)
    dO = mo.decode_bf16(datagen.dout_all(cfg))
    res = {}
    for dt in ("bf16", "mxfp8"):
        W = mo.weights_from_bits(w, dt)
        fw = mo.forward(lambda r: X[r], L, W, cfg.K, 0, cfg.E_loc, cfg.M,
                        row_align=32 if dt == "mxfp8" else 1)
        bw = mo.backward(fw, lambda r: dO[r], W, cfg.K, 0, cfg.E_loc, cfg.E)
        res[dt] = (fw, bw)
    (fb, bb), (fm, bm) = res["bf16"], res["mxfp8"]
    rel = lambda a, b: np.linalg.norm(a - b) / np.linalg.norm(b)
    assert rel(fm.out, fb.out) < 0.08
    for name in ("dx", "dp", "dwg", "dwu", "dwd"):
        assert rel(getattr(bm, name), getattr(bb, name)) < 0.08, name
    # dlogits = p (dp - sum p dp) subtracts nearly equal terms, which magnifies the error.
    assert rel(bm.dlogits, bb.dlogits) < 0.2


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_expert_wgrad_rows_match_full_backward(dtype):
    """The per-expert sampled weight-gradient rows (used to check full-size runs) equal the
    corresponding rows of the whole backward, for every expert of a multi-expert layer with
    ragged per-expert row counts."""
    cfg = datagen.CONFIGS["tiny"].replace(S=2, T=96, E=8, K=3, e0=2, E_loc=3, x_std=1.0,
                                          dtype=dtype)
    X = mo.decode_bf16(datagen.x_all(cfg))
    dO = mo.decode_bf16(datagen.dout_all(cfg))
    L = datagen.logits(cfg)
    W = mo.weights_from_bits(datagen.weights(cfg), dtype)
    align = 32 if dtype == "mxfp8" else 1
    fw = mo.forward(lambda r: X[r], L, W, cfg.K, cfg.e0, cfg.E_loc, 64, align)
    bw = mo.backward(fw, lambda r: dO[r], W, cfg.K, cfg.e0, cfg.E_loc, cfg.E)
    gi = np.array([0, 5, 77, cfg.I - 1]); hi = np.array([1, 64, cfg.H - 1])
    for e in range(cfg.E_loc):
        lo, c = int(fw.sched.offsets[e]), int(fw.sched.counts[e])
        pairs = fw.sched.perm[lo:lo + c]
        n = pairs // cfg.K
        p_rows = fw.p.reshape(-1)[pairs]
        dwg, dwu, dwd = mo.expert_wgrad_rows(X[n], dO[n], p_rows, W, e, gi, hi, workers=2)
        assert np.allclose(dwg, bw.dwg[e][gi], rtol=1e-12, atol=1e-14)
        assert np.allclose(dwu, bw.dwu[e][gi], rtol=1e-12, atol=1e-14)
        assert np.allclose(dwd, bw.dwd[e][hi], rtol=1e-12, atol=1e-14)


def test_router_projection_gradients_match_finite_differences():
    """With logits = X W_r^T feeding the layer (every expert local, so dlogits is complete), the
    gradients of L = sum <dOut, out> are dW_r = dlogits^T X and dX = dX_layer + dlogits W_r:
    checked by central differences in fp64 on the tiny workload."""
    cfg = datagen.CONFIGS["tiny"]
    X = mo.decode_bf16(datagen.x_all(cfg))
    Wr = mo.decode_bf16(datagen.router_weight(cfg))
    w = datagen.weights(cfg)
    Wg, Wu, Wd = (mo.decode_bf16(w[k]) for k in ("wg", "wu", "wd"))
    dO = mo.decode_bf16(datagen.dout_all(cfg))
    K, E = cfg.K, cfg.E
    L = mo.router_logits(X, Wr)
    assert 0.5 < L.std() < 2.0                         # the spread the workload's logits have
    Ls = np.sort(L, axis=1)[:, ::-1]
    assert (Ls[:, K - 1] - Ls[:, K]).min() > 1e-4      # no near-tie: top-k is locally constant
    fw, bw = _run_oracle(X, L, Wg, Wu, Wd, dO, K, 0, E, E)
    dwr, dxr = mo.router_backward(X, Wr, bw.dlogits)
    assert np.array_equal(fw.sched.touched, np.arange(cfg.N))
    dx_total = bw.dx + dxr
    f = lambda: _loss(X, mo.router_logits(X, Wr), Wg, Wu, Wd, dO, K, 0, E)
    eps = 1e-6
    rng = np.random.default_rng(11)

    def fd(arr, pos):
        old = arr[pos]
        arr[pos] = old + eps; lp = f()
        arr[pos] = old - eps; lm = f()
        arr[pos] = old
        return (lp - lm) / (2 * eps)

    checks = []
    for _ in range(16):
        pos = (int(rng.integers(E)), int(rng.integers(cfg.H)))
        checks.append((fd(Wr, pos), dwr[pos]))
    for _ in range(16):
        pos = (int(rng.integers(cfg.N)), int(rng.integers(cfg.H)))
        checks.append((fd(X, pos), dx_total[pos]))
    for fdv, an in checks:
        assert abs(fdv - an) <= 1e-6 * max(abs(an), 1e-3), (fdv, an)
    # the projection's share matters: without it dX would be off
    assert np.abs(dxr).max() > 1e-3 * np.abs(bw.dx).max()
