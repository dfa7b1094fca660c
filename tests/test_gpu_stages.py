"""GPU parity of the staged path (mok_schedule -> mok_dispatch -> mok_expert_ffn -> mok_combine)
against the CPU oracle, through the C ABI.

Integer and copy results are compared bit for bit; float results with the tolerances the
layer is specified to: BF16 max|err| <= 1e-2 max|ref|, MXFP8 relative Frobenius <= 3e-2.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen
from oracle import moe_oracle as mo
from oracle import mx as omx

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from tests._gpu import (BF16_TOL, MX_TOL, Case, bf16_to_f64, dev_u16, frob_rel_err, host_u16,
                        max_rel_err)
import combine_router_top_schedule_amd as mok


def _check_schedule(case, row_align=1):
    cfg = case.cfg
    idx_ref, p_ref = mo.topk_gating(case.logits_h, cfg.K)
    s_ref = mo.schedule(idx_ref, cfg.e0, cfg.E_loc, cfg.M, row_align)
    idx, p = case.idx_p()
    assert np.array_equal(idx, idx_ref)
    assert np.abs(p - p_ref).max() <= 1e-6
    hdr, perm, tokpos, touched = case.layer.table()
    hdr = hdr.numpy()
    assert hdr[0] == s_ref.P and hdr[1] == s_ref.rows and hdr[2] == len(s_ref.touched)
    # header word 3: touched tokens with more than one local pair (the fused merges' list)
    local = ((idx_ref >= cfg.e0) & (idx_ref < cfg.e0 + cfg.E_loc)).sum(axis=1)
    assert hdr[3] == int((local > 1).sum())
    assert np.array_equal(hdr[16:16 + cfg.E_loc], s_ref.counts)
    assert np.array_equal(hdr[96:96 + cfg.E_loc + 1], s_ref.offsets)
    assert np.array_equal(perm.numpy()[:s_ref.rows], s_ref.perm)
    assert np.array_equal(tokpos.numpy(), s_ref.tokpos)
    assert np.array_equal(touched.numpy()[:len(s_ref.touched)], s_ref.touched)
    return s_ref


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (2, 3), (7, 1)])
def test_schedule_tiny(e0, E_loc):
    cfg = datagen.CONFIGS["tiny"].replace(e0=e0, E_loc=E_loc)
    case = Case(cfg)
    case.layer.schedule(case.logits)
    _check_schedule(case)
    # run-to-run identical
    first = [t.clone() for t in (case.layer.idx, case.layer.p, case.layer.saved)]
    case.layer.schedule(case.logits)
    for a, b in zip(first, (case.layer.idx, case.layer.p, case.layer.saved)):
        assert torch.equal(a, b)


def test_schedule_ties_and_ragged_blocks():
    # 1000 tokens (three full blocks of 256 and a ragged one), logits from a 5-value set so
    # ties are everywhere, 64 experts, top-8, five local experts in the middle.
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=250, E=64, K=8, e0=20, E_loc=5)
    rng = np.random.default_rng(3)
    L = rng.choice(np.array([-1.0, 0.0, -0.0, 0.5, 2.0], np.float32), (cfg.N, cfg.E))
    case = Case(cfg, logits=L)
    case.layer.schedule(case.logits)
    _check_schedule(case)


def test_schedule_no_local_pairs():
    cfg = datagen.CONFIGS["tiny"].replace(e0=6, E_loc=2)
    L = np.zeros((cfg.N, cfg.E), np.float32)
    L[:, :2] = 5.0                      # every token picks experts 0 and 1 only
    case = Case(cfg, logits=L)
    case.layer.forward_staged(case.x_seg, case.logits, case.out_seg)
    s = _check_schedule(case)
    assert s.P == 0
    assert not case.out.any()            # nothing written


def test_schedule_dsv3_full_size():
    cfg = datagen.CONFIGS["dsv3"]
    case = Case(cfg)
    case.layer.schedule(case.logits)
    s = _check_schedule(case)
    assert 15000 < s.P < 18000


def test_quantize_mx_bit_exact():
    rng = np.random.default_rng(5)
    for (b, r, c) in ((2, 64, 96), (1, 256, 128)):
        v = rng.standard_normal((b, r, c)).astype(np.float32)
        v *= np.exp2(rng.integers(-30, 30, (b, r, 1))).astype(np.float32)
        v[0, 0, :32] = 0.0                                     # an all-zero block
        v[0, 1, 5] = 1e-40                                     # fp32 subnormal input
        bits = datagen.f32_to_bf16_bits(v)
        vals = mo.decode_bf16(bits)
        src = dev_u16(bits)
        for tr in (0, 1):
            orow, ocol = (c, r) if tr else (r, c)
            codes = torch.empty((b, orow, ocol), dtype=torch.uint8, device="cuda")
            scales = torch.empty((b, orow, ocol // 32), dtype=torch.uint8, device="cuda")
            mok.mok_quantize_mx(src, bool(tr), codes, scales)
            ref_in = np.swapaxes(vals, 1, 2) if tr else vals
            c_ref, s_ref = omx.quantize(ref_in, axis=2)
            assert np.array_equal(codes.cpu().numpy(), c_ref), tr
            assert np.array_equal(scales.cpu().numpy(), s_ref), tr


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_dispatch_rows(dtype):
    cfg = datagen.CONFIGS["tiny"].replace(dtype=dtype, S=2, T=300, e0=1, E_loc=5, M=32)
    case = Case(cfg)
    case.layer.schedule(case.logits)
    case.layer.dispatch(case.x_seg)
    s = _check_schedule(case, 32 if dtype == "mxfp8" else 1)
    real = s.perm >= 0
    src = case.x_h[s.perm[real] // cfg.K]
    if dtype == "bf16":
        xd = host_u16(case.layer.xd[:s.rows * cfg.H * 2].view(torch.int16)).reshape(s.rows, cfg.H)
        assert np.array_equal(xd[real], src)
    else:
        rows_max = int(case.layer.sizes.rows_max)
        raw = case.layer.xd.cpu().numpy()
        codes = raw[:rows_max * cfg.H].reshape(rows_max, cfg.H)[:s.rows]
        scales = raw[rows_max * cfg.H:rows_max * cfg.H + rows_max * cfg.H // 32]
        scales = scales.reshape(rows_max, cfg.H // 32)[:s.rows]
        c_ref, s_ref = omx.quantize(mo.decode_bf16(src), axis=1)
        assert np.array_equal(codes[real], c_ref) and np.array_equal(scales[real], s_ref)
        assert not codes[~real].any() and not scales[~real].any()   # pad rows are zero


def _staged_forward_check(cfg, tol_fn, tol):
    case = Case(cfg)
    case.layer.forward_staged(case.x_seg, case.logits, case.out_seg)
    torch.cuda.synchronize()
    fw = case.oracle_forward()
    got = case.out_rows(fw.sched.touched)
    err = tol_fn(got, fw.out)
    assert err <= tol, err
    # untouched tokens are not written
    untouched = np.setdiff1d(np.arange(cfg.N), fw.sched.touched)
    assert not host_u16(case.out)[untouched].any()
    # run-to-run bit-identical
    first = case.out.clone()
    case.out.zero_()
    case.layer.forward_staged(case.x_seg, case.logits, case.out_seg)
    assert torch.equal(first, case.out)
    return case, fw, err


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (3, 4)])
def test_staged_forward_tiny_bf16(e0, E_loc):
    cfg = datagen.CONFIGS["tiny"].replace(e0=e0, E_loc=E_loc)
    _staged_forward_check(cfg, max_rel_err, BF16_TOL)


def test_staged_forward_ragged_tiles_bf16():
    # 600 tokens, top-2 of 4 experts, all local: ~300 rows per expert -> a full 256-row tile
    # and a ragged one per expert; H = 384 gives a partial 256-column tile in the down GEMM.
    cfg = datagen.CONFIGS["tiny"].replace(S=3, T=200, E=4, K=2, E_loc=4, H=384, I=256)
    _staged_forward_check(cfg, max_rel_err, BF16_TOL)


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (2, 5)])
def test_staged_forward_tiny_mxfp8(e0, E_loc):
    cfg = datagen.CONFIGS["tiny"].replace(e0=e0, E_loc=E_loc, dtype="mxfp8", x_std=1.0, M=32)
    _staged_forward_check(cfg, frob_rel_err, MX_TOL)


def test_staged_forward_dsv3_sampled():
    """Full DeepSeek-V3-shaped local share (64 x 2048 tokens, H 7168, I 2048, experts 0..3 of
    256, top-8); 96 sampled touched tokens are recomputed by the oracle one by one."""
    cfg = datagen.CONFIGS["dsv3"]
    case = Case(cfg)
    case.layer.forward_staged(case.x_seg, case.logits, case.out_seg)
    torch.cuda.synchronize()
    hdr, perm, tokpos, touched = case.layer.table()
    U = int(hdr[2])
    rng = np.random.default_rng(0)
    sample = np.sort(rng.choice(touched.numpy()[:U], 96, replace=False))
    fw = case.oracle_forward(tokens=sample)
    assert len(fw.sched.touched) == len(sample)
    got = case.out_rows(sample)
    err = max_rel_err(got, fw.out)
    assert err <= BF16_TOL, err
