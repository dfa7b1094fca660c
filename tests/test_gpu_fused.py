"""GPU tests of the fused forward (mok_layer_fwd): parity with the oracle, bit-identity with
the staged path and across minibatch sizes, ring wrap-around, and the bounded-wait fault path."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_router_top_schedule_amd as mok
from tests._gpu import BF16_TOL, MX_TOL, Case, frob_rel_err, host_u16, max_rel_err


def _fused(case):
    case.out.zero_()
    case.layer.forward(case.x_seg, case.logits, case.out_seg)
    torch.cuda.synchronize()
    assert mok.mok_device_status(case.layer.ws) == 0
    return case.out.clone()


def _staged(case):
    case.out.zero_()
    case.layer.forward_staged(case.x_seg, case.logits, case.out_seg)
    torch.cuda.synchronize()
    return case.out.clone()


def _local_pair_counts(case, fw):
    cfg = case.cfg
    local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
    return local.sum(axis=1)


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (2, 3)])
@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_fused_forward_tiny_matches_oracle_and_staged(dtype, e0, E_loc):
    """With experts 2..4 of 8 local, some tokens have one local pair (their output row is
    written by the down-GEMM epilogue) and some two (merged from the slots); the fused result
    equals the staged path's, which merges every token from the slots, bit for bit."""
    cfg = datagen.CONFIGS["tiny"].replace(dtype=dtype, M=32, e0=e0, E_loc=E_loc,
                                          x_std=1.0 if dtype == "mxfp8" else 0.02)
    case = Case(cfg, fused=True)
    fused = _fused(case)
    fw = case.oracle_forward()
    if E_loc < cfg.E:
        per_token = _local_pair_counts(case, fw)
        assert (per_token == 1).any() and (per_token > 1).any()
    got = case.out_rows(fw.sched.touched)
    if dtype == "bf16":
        assert max_rel_err(got, fw.out) <= BF16_TOL
    else:
        assert frob_rel_err(got, fw.out) <= MX_TOL
    assert torch.equal(fused, _staged(case))
    assert torch.equal(fused, _fused(case))            # run-to-run


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_fused_forward_ring_wraps(dtype):
    # 2048 pairs cut by 64-row minibatches into ~64 row tiles: ~8 tiles per XCD through the
    # smallest ring (3 gather and 2 activation slots per XCD), so every slot is reused several
    # times.
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, dtype=dtype, M=64, x_std=1.0)
    d = mok.desc_from_config(cfg)
    case = Case(cfg, fused=True, ring_bytes=mok.query_sizes(d).ring_min_bytes)
    assert case.layer.sizes.ring_slots == 16
    fused = _fused(case)
    assert torch.equal(fused, _staged(case))
    fw = case.oracle_forward()
    got = case.out_rows(fw.sched.touched)
    tol_fn, tol = (max_rel_err, BF16_TOL) if dtype == "bf16" else (frob_rel_err, MX_TOL)
    assert tol_fn(got, fw.out) <= tol


def test_fused_forward_dsv3_equals_staged_and_is_minibatch_independent():
    """Full DeepSeek-V3-shaped local share: the fused ring forward equals the staged path bit
    for bit (same tile math per row), for two minibatch sizes."""
    cfg = datagen.CONFIGS["dsv3"]
    case = Case(cfg, fused=True)
    staged = _staged(case)
    fused = _fused(case)
    assert torch.equal(fused, staged)
    case2 = Case(cfg.replace(M=512), fused=True)
    assert torch.equal(_fused(case2), staged)


def test_fused_forward_kimi_minibatch_sweep():
    """Kimi-K2-shaped local share (experts 0..5 of 384, top-8, H 7168, I 2048) through the fixed
    256 MiB ring at minibatch sizes 512, 1024, 2368 and 2560: every fused run equals the staged
    path bit for bit, and 64 sampled touched tokens are recomputed by the oracle."""
    from combine_router_top_schedule_amd.layer import MokLayer
    cfg = datagen.CONFIGS["kimi"]
    case = Case(cfg, fused=True)
    staged = _staged(case)
    for M in (512, 1024, 2368, 2560):
        layer = MokLayer(mok.desc_from_config(cfg, M=M), staged=False, fused=True)
        layer.set_weights(case.wg, case.wu, case.wd)
        case.out.zero_()
        layer.forward(case.x_seg, case.logits, case.out_seg)
        torch.cuda.synchronize()
        assert mok.mok_device_status(layer.ws) == 0
        assert torch.equal(case.out, staged), f"minibatch {M}"
        del layer
    hdr, perm, tokpos, touched = case.layer.table()
    U = int(hdr[2])
    sample = np.sort(np.random.default_rng(2).choice(touched.numpy()[:U], 64, replace=False))
    fw = case.oracle_forward(tokens=sample)
    assert len(fw.sched.touched) == len(sample)
    err = max_rel_err(case.out_rows(sample), fw.out)
    assert err <= BF16_TOL, err


def test_fused_forward_ring_too_small_is_rejected():
    cfg = datagen.CONFIGS["tiny"]
    case = Case(cfg, fused=True, ring_bytes=1 << 20)
    with pytest.raises(mok.MokError) as ei:
        case.layer.forward(case.x_seg, case.logits, case.out_seg)
    assert ei.value.code == 6


def test_fused_forward_withheld_signal_times_out():
    """A debug flag withholds one dispatch signal; the bounded waits expire and the kernel
    reports MOK_ERR_DEVICE_TIMEOUT instead of hanging."""
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, M=64)
    case = Case(cfg, fused=True, flags=mok.MOK_FLAG_SKIP_ONE_SIGNAL)
    case.layer.forward(case.x_seg, case.logits, case.out_seg)
    assert mok.mok_device_status(case.layer.ws) == 8
