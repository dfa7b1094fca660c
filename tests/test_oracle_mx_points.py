"""Pins of the oracle's MXFP8 quantisation points (where the layer quantises, along which axis,
with what padding) and of its BF16 decoding.

The pages state only that activation quantisation is folded into dispatch, the grouped GEMM and
SwiGLU ("把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ③; "Mixture-of-Kittens (MoK)",
benchmark section, MXFP8 forward and backward). The reading both sides implement: every GEMM
operand is quantised in 32-element blocks along that GEMM's reduction axis; the weight-gradient
operands (reduction over tokens) per expert, zero-padded to a multiple of 32 rows; computed
values are rounded to fp32 first.

Each test runs the oracle on a crafted layer (tests/mx_cases.py) in which quantising along the
stated axis flushes known entries to exactly zero and quantising along the other axis (or not at
all) keeps them, so a wrong axis, a skipped point or a lost padding rule fails an exact check.
Each test also confirms that the wrong reading would change the checked value.
"""
import numpy as np
import pytest

import datagen
from oracle import moe_oracle as mo
from oracle import mx
from tests import mx_cases as mc


def _run(c: mc.Crafted):
    W = mo.Weights(c.wg, c.wu, c.wd, "mxfp8")
    E_loc = c.wg.shape[0]
    fw = mo.forward(lambda r: c.x[r], c.logits, W, c.K, 0, E_loc, 64, row_align=32)
    bw = mo.backward(fw, lambda r: c.dout[r], W, c.K, 0, E_loc, c.E)
    return fw, bw


def _out(fw, N):
    """Forward output as [N][H] (every token is touched in these cases)."""
    assert np.array_equal(fw.sched.touched, np.arange(N))
    return fw.out


def test_crafted_values_are_bf16_exact():
    for build in (mc.dispatch_x_along_h, mc.swiglu_h_along_i, mc.backward_d_along_h,
                  mc.backward_dgdu_along_i, mc.wgrad_x_along_tokens, mc.wgrad_h_along_tokens,
                  mc.wgrad_dgdu_pd_along_tokens):
        c = build()
        for a in (c.x, c.dout, c.wg, c.wu, c.wd):
            mc.bf16_bits(a)


def test_weight_views_are_exact_for_the_crafted_weights():
    """The crafted weights lose nothing in any of their six quantised views, so the checks below
    see activation quantisation only."""
    for build in (mc.dispatch_x_along_h, mc.swiglu_h_along_i, mc.backward_d_along_h,
                  mc.backward_dgdu_along_i, mc.wgrad_x_along_tokens, mc.wgrad_h_along_tokens):
        c = build()
        W = mo.Weights(c.wg, c.wu, c.wd, "mxfp8")
        for view, ref in ((W.fwd_gate, c.wg), (W.fwd_up, c.wu), (W.fwd_down, c.wd),
                          (W.bwd_gate, c.wg), (W.bwd_up, c.wu), (W.bwd_down, c.wd)):
            assert np.array_equal(view(), ref), (build.__name__, view.__name__)


def test_dispatch_quantises_x_along_h():
    c = mc.dispatch_x_along_h()
    fw, _ = _run(c)
    odd = ~mc._even(mc.H)
    assert (fw.xd[:, odd] == 0).all() and (fw.xd[:, ~odd] == 1).all()
    assert (_out(fw, c.N)[:, 1] == 0).all() and (fw.out[:, 0] != 0).all()
    # blocked along tokens (the wrong axis) the odd columns would survive
    assert np.array_equal(mx.fake_quant(c.x, axis=0), c.x)


def test_swiglu_quantises_h_along_i():
    c = mc.swiglu_h_along_i()
    fw, _ = _run(c)
    odd = ~mc._even(mc.I)
    assert (fw.h[:, odd] == 0).all() and (fw.h[:, ~odd] != 0).all()
    assert (_out(fw, c.N)[:, 1] == 0).all() and (fw.out[:, 0] != 0).all()
    h32 = np.asarray(mo.silu(fw.g) * fw.u, np.float32).astype(np.float64)
    assert (mx.fake_quant(h32, axis=0)[:, odd] != 0).all()


def test_backward_quantises_dout_along_h():
    c = mc.backward_d_along_h()
    fw, bw = _run(c)
    assert (bw.a[:, 32] == 0).all() and (bw.a[:, 0] == 64).all()
    dx = bw.dx
    assert (dx[:, 2] == 0).all() and (dx[:, 3] != 0).all()
    assert (mx.fake_quant(c.dout, axis=0)[:, 1] != 0).all()


def test_dx_gemm_quantises_dg_du_along_i():
    c = mc.backward_dgdu_along_i()
    fw, bw = _run(c)
    odd = ~mc._even(mc.I)
    assert (bw.dg[:, odd] != 0).all() and (bw.du[:, odd] != 0).all()
    assert (bw.dx[:, 1] == 0).all() and (bw.dx[:, 0] != 0).all()
    # along tokens (every row alike) they would survive, and reach dX column 1
    for v in (bw.dg, bw.du):
        assert (mx.fake_quant(np.asarray(v, np.float32).astype(np.float64), axis=0)[:, odd] != 0).all()


def test_wgrad_quantises_x_along_tokens():
    c = mc.wgrad_x_along_tokens()
    fw, bw = _run(c)
    n_even = int(mc._even(c.N).sum())
    for dw in (bw.dwg[0], bw.dwu[0]):
        assert (dw[:, 32] != 0).all()
        assert np.array_equal(dw[:, 0] * c.N, dw[:, 32] * n_even)
    # blocked along H the odd tokens' column 0 would keep TINY
    assert (mx.fake_quant(c.x, axis=1)[~mc._even(c.N), 0] == mc.TINY).all()


def test_wgrad_quantises_h_along_tokens():
    c = mc.wgrad_h_along_tokens()
    fw, bw = _run(c)
    ev = mc._even(c.N)
    assert (fw.h[~ev, 1] != 0).all() and (fw.h[~ev][:, [0] + list(range(2, mc.I))] == 0).all()
    assert bw.dwd[0, 0, 1] == ev.sum() * fw.h[0, 1]
    assert bw.dwd[0, 0, 1] != fw.h[:, 1].sum()


def test_wgrad_quantises_dg_du_pd_along_tokens_per_expert():
    fw_t, bw_t = _run(mc.wgrad_dgdu_pd_along_tokens(odd_scale=mc.TINY))
    fw_z, bw_z = _run(mc.wgrad_dgdu_pd_along_tokens(odd_scale=0.0))
    # the odd tokens' dg, du and p*D are nonzero before quantisation ...
    odd_rows = fw_t.sched.tokpos[1::2]
    assert (bw_t.dg[odd_rows] != 0).all() and (bw_t.du[odd_rows] != 0).all()
    # ... and flushed inside the expert's token blocks: the weight gradients do not see them
    for name in ("dwg", "dwu", "dwd"):
        assert np.array_equal(getattr(bw_t, name), getattr(bw_z, name)), name
    # the input gradient, blocked along features, does see them
    assert not np.array_equal(bw_t.dx, bw_z.dx)
    # a second expert holding only the odd tokens has blocks of its own: nonzero gradients
    fw_s, bw_s = _run(mc.wgrad_dgdu_pd_along_tokens(odd_scale=mc.TINY, split_experts=True))
    assert list(fw_s.sched.counts) == [32, 32]
    for name in ("dwg", "dwu", "dwd"):
        g = getattr(bw_s, name)
        assert (g[0] != 0).any() and (g[1] != 0).any(), name
    # with the two experts' rows blocked together, expert 1 would flush entirely
    both = np.concatenate([bw_s.dg[:32], bw_s.dg[32:64]])
    mixed = mx.fake_quant(np.asarray(both[16:48], np.float32).astype(np.float64), axis=0)
    assert (mixed[16:] == 0).all()


def test_fake_quant_rows_padded_blocks_from_row_zero_with_zero_padding():
    r = 40
    v = np.zeros((r, 3))
    v[:32, 0] = 1.0; v[32:, 0] = mc.TINY         # last (padded) block holds TINY only: kept
    v[:, 1] = 1.0; v[39, 1] = mc.TINY              # TINY next to 1s in the padded block: flushed
    v[:8, 2] = mc.TINY; v[8:, 2] = 1.0             # blocks counted from the end would keep row 0..7
    q = mx.fake_quant_rows_padded(v)
    assert q.shape == v.shape
    assert (q[32:, 0] == mc.TINY).all() and (q[:32, 0] == 1.0).all()
    assert q[39, 1] == 0.0 and (q[:39, 1] == 1.0).all()
    assert (q[:8, 2] == 0.0).all() and (q[8:, 2] == 1.0).all()
    # row counts that are multiples of 32 need no padding and agree with plain blocking
    w = np.random.default_rng(0).standard_normal((64, 5))
    assert np.array_equal(mx.fake_quant_rows_padded(w), mx.fake_quant(w, axis=0))


def test_decode_bf16_round_trips_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    vals = mo.decode_bf16(bits[finite])
    assert np.array_equal(datagen.f32_to_bf16_bits(vals.astype(np.float32)), bits[finite])
    assert mo.decode_bf16(np.array([0x3F80, 0xC000, 0x0001, 0x8000], np.uint16)).tolist() == \
        [1.0, -2.0, 2.0 ** -133, -0.0]


def test_quantised_operands_come_from_fp32_values():
    """p*D, du and dg are quantised from their fp32 values, not from a BF16 rounding of them:
    at these E4M3 ties the two differ by a whole grid step (0.5625 vs 0.5)."""
    c = mc.precision_ties()
    fw, bw = _run(c)
    assert np.allclose(fw.p[:, 0], mc.P0, atol=1e-7)
    assert (bw.dwd[0][0:2] == 216.0).all() and (bw.dwd[0][2:] == 0).all()
    assert (bw.dwu[0][:, 0] == 36.0).all()
    assert (bw.dwg[1][:, 0] == 36.0).all()
    assert (bw.dx[:, 7] == 72.0).all() and (bw.dx[:, 9] == 72.0).all()
    # the BF16-first reading would give the lower grid point
    bf = lambda v: datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(np.float32(v))).astype(np.float64)
    for v in (mc.P0, bw.du[0, 0], bw.dg[64, 0]):
        assert 272 < v * 512 < 273
        assert mx.fake_quant(np.full(32, bf(v)))[0] == 0.5
        assert mx.fake_quant(np.full(32, np.float32(v)).astype(np.float64))[0] == 0.5625


def test_parallel_quantiser_slices_give_identical_values():
    v = np.random.default_rng(3).standard_normal((100, 96)) * np.exp2(np.arange(96) % 7)
    for axis in (0, 1):
        assert np.array_equal(mx.fake_quant(v[:96 if axis == 0 else 100], axis=axis, workers=5),
                              mx.fake_quant(v[:96 if axis == 0 else 100], axis=axis))
    assert np.array_equal(mx.fake_quant_rows_padded(v, workers=3), mx.fake_quant_rows_padded(v))
