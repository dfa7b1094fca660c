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
from oracle import moe_oracle as mo
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


def _expected_tiles(sched, M):
    """The oracle's minibatch cut (rows [jM, (j+1)M) of the expert-ordered stream, one ring
    slot each) intersected with each expert's rows, in GEMM tiles of at most 256 rows: tiles
    never straddle an expert or a minibatch. Ordered by minibatch, then expert, then row."""
    out = []
    for j in range(sched.J):
        rows = mo.minibatch_rows(sched, j)
        for e in range(len(sched.counts)):
            lo, hi = int(sched.offsets[e]), int(sched.offsets[e]) + int(sched.counts[e])
            r0, r1 = max(rows.start, lo), min(rows.stop, hi)
            for q in range(r0, r1, 256):
                out.append((j, e, q, min(256, r1 - q)))
    return np.array(out, dtype=np.int64).reshape(-1, 4)


@pytest.mark.parametrize("name,M,dtype", [("tiny4", 64, "bf16"), ("tiny4", 96, "mxfp8"),
                                          ("dsv3", 2368, "bf16")])
def test_tile_table_is_the_oracles_minibatch_cut(name, M, dtype):
    cfg = (datagen.CONFIGS["tiny"].replace(S=4, T=256, x_std=1.0) if name == "tiny4"
           else datagen.CONFIGS[name]).replace(M=M, dtype=dtype)
    case = Case(cfg, fused=True)
    _fused(case)
    got = case.layer.tiles().numpy().astype(np.int64)
    idx, _ = mo.topk_gating(case.logits_h, cfg.K)
    sched = mo.schedule(idx, cfg.e0, cfg.E_loc, M, 32 if dtype == "mxfp8" else 1)
    exp = _expected_tiles(sched, M)
    print(f"  {len(got)} tiles over {sched.J} minibatches")
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_results_do_not_depend_on_the_cu_split(dtype):
    """The share of compute units given to dispatch changes only who does the work: forward and
    backward outputs are bit-identical for every split."""
    from tests._gpu import BwdCase
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=512, H=1024, I=512, M=128, x_std=1.0, dtype=dtype)
    ring = 2 * mok.query_sizes(mok.desc_from_config(cfg)).ring_min_bytes
    ref = None
    for cus in (8, 16, 40, 96):
        case = BwdCase(cfg, fused=True, comm_cus=cus, ring_bytes=ring)
        case.run(fused=True)
        res = case.grads() + [case.out.clone()]
        if ref is None:
            ref = res
        else:
            for a, b in zip(ref, res):
                assert torch.equal(a, b), cus


def test_layer_calls_do_not_synchronise_with_the_host():
    """mok_layer_fwd and mok_layer_bwd only enqueue work: queued behind a long GPU sleep, both
    host calls return while the stream is still busy, and the results are those of an
    unobstructed run."""
    import time
    from tests._gpu import BwdCase
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, M=64, x_std=1.0)
    case = BwdCase(cfg, fused=True)
    case.run(fused=True)
    ref = case.grads() + [case.out.clone()]
    # calibrate torch.cuda._sleep's cycle count to about 0.5 s
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(); torch.cuda._sleep(10_000_000); b.record(); torch.cuda.synchronize()
    cycles = int(10_000_000 * 500.0 / max(a.elapsed_time(b), 1e-3))
    L = case.layer
    torch.cuda._sleep(cycles)
    t0 = time.perf_counter()
    L.forward(case.x_seg, case.logits, case.out_seg)
    mok.mok_layer_bwd(case.d, case.dout_seg, case.x_seg, L.w, L.idx, L.p, L.saved, L.ring,
                      L.slots, case.dx_seg, case.dp, case.dlogits, case.dwg, case.dwu, case.dwd,
                      case.bws)
    host_s = time.perf_counter() - t0
    done = torch.cuda.Event()
    done.record()
    busy = not done.query()
    torch.cuda.synchronize()
    print(f"  host time of both calls {host_s * 1e3:.2f} ms behind a ~500 ms GPU sleep")
    assert busy and host_s < 0.25
    assert mok.mok_device_status(L.ws) == 0
    for x, y in zip(ref, case.grads() + [case.out.clone()]):
        assert torch.equal(x, y)


def test_autotune_measures_every_candidate_and_all_give_the_same_output():
    """mok_autotune times the fused forward over minibatch sizes M, 2M, 4M, all rows and
    dispatch-CU counts 8 .. 48, returns the fastest, and every candidate produces the same output
    bit for bit (the choice changes speed only)."""
    from combine_router_top_schedule_amd.layer import MokLayer
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=512, H=1024, I=512, M=128, x_std=1.0)
    ring = 2 * mok.query_sizes(mok.desc_from_config(cfg)).ring_min_bytes
    case = Case(cfg, fused=True, ring_bytes=ring)
    ref = _fused(case)
    tuned, best, table = case.layer.autotune(case.x_seg, case.logits, case.out_seg, reps=2,
                                             apply=False)
    print(f"  tuned M={tuned.minibatch_tokens} comm_cus={tuned.comm_cus} {best:.3f} ms; {table}")
    Ms = sorted({m for m, _, _ in table})
    assert Ms[0] == 128 and Ms[1:3] == [256, 512] and len(table) == len(Ms) * 5
    assert (tuned.minibatch_tokens, tuned.comm_cus) in {(m, c) for m, c, _ in table}
    assert best == min(t for _, _, t in table)
    for m, c, _ in table:
        layer = MokLayer(mok.desc_from_config(cfg, M=m, ring_bytes=ring, comm_cus=c),
                         staged=False, fused=True)
        layer.set_weights(case.wg, case.wu, case.wd)
        case.out.zero_()
        layer.forward(case.x_seg, case.logits, case.out_seg)
        torch.cuda.synchronize()
        assert mok.mok_device_status(layer.ws) == 0
        assert torch.equal(case.out, ref), (m, c)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_trace_and_poison_flags_leave_results_unchanged(dtype):
    """MOK_FLAG_POISON fills every ring slot with NaN bytes when a new row tile takes it, before
    that tile's rows arrive; MOK_FLAG_TRACE records each item of the fused forward. Neither
    changes a bit of the forward or backward outputs (so no item read a slot before its data was
    there), and the trace holds every item of every row tile exactly once, with times ordered as
    the counters order them: a tile's gate/up items start after its gathers started, its down
    items after all of its gate/up items started."""
    from combine_router_top_schedule_amd import trace
    from tests._gpu import BwdCase
    # ~64 row tiles through the smallest ring: every slot is reused several times
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, M=64, x_std=1.0, dtype=dtype)
    ring = mok.query_sizes(mok.desc_from_config(cfg)).ring_min_bytes
    ref = BwdCase(cfg, fused=True, ring_bytes=ring)
    ref.run(fused=True)
    want = [ref.out.clone()] + ref.grads()
    ngu, ndn = cfg.I // 128, -(-cfg.H // 256)
    for flags in (mok.MOK_FLAG_POISON, mok.MOK_FLAG_TRACE,
                  mok.MOK_FLAG_POISON | mok.MOK_FLAG_TRACE):
        case = BwdCase(cfg, fused=True, ring_bytes=ring, flags=flags)
        case.run(fused=True)
        for a, b in zip(want, [case.out.clone()] + case.grads()):
            assert torch.equal(a, b), flags
        if not flags & mok.MOK_FLAG_TRACE:
            continue
        L = case.layer
        rec, count = trace.read(L.ws, L.sizes)
        assert count == len(rec) > 0
        kind, xcd, macro = trace.fields(rec)
        assert (macro == 0).all()
        assert (rec["t_wait"] <= rec["t_begin"]).all() and (rec["t_begin"] <= rec["t_end"]).all()
        ntiles = len(L.tiles())
        for t in range(ntiles):
            m = rec["tile"] == t
            gathers = m & (kind <= 2)
            gu, dn = m & (kind == 3), m & (kind == 4)
            assert gathers.any() and gu.sum() == ngu and dn.sum() == ndn, t
            assert len(np.unique(xcd[m])) == 1, t          # a row tile stays on one XCD
            assert rec["t_begin"][gu].min() >= rec["t_begin"][gathers].max(), t
            assert rec["t_begin"][dn].min() >= rec["t_begin"][gu].max(), t
        assert set(np.unique(rec["tile"])) == set(range(ntiles))
        s = trace.summarize(rec)
        print(f"  {dtype} flags {flags}: {s['records']} records, {s['span_us']} us, GEMM workers "
              f"busy {s['gemm_busy_frac']:.2f}, waiting {s['gemm_wait_frac']:.2f}")
