"""GPU parity of mok_layer_bwd (input gradient, router-weight gradient, weight gradients and,
with every expert local, dlogits) against the CPU oracle's backward."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen
from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_router_top_schedule_amd as mok
from tests._gpu import BF16_TOL, MX_TOL, BwdCase, frob_rel_err, host_u16, max_rel_err


def _compare(case, fw, bw, tol_fn, tol):
    cfg = case.cfg
    errs = {}
    tok = fw.sched.touched
    errs["dx"] = tol_fn(mo.decode_bf16(host_u16(case.dx)[tok]), bw.dx)
    dp = case.dp.cpu().numpy().reshape(cfg.N, cfg.K)
    local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
    errs["dp"] = tol_fn(dp[local], bw.dp[local])
    for name in ("dwg", "dwu", "dwd"):
        errs[name] = tol_fn(getattr(case, name).cpu().numpy().astype(np.float64), getattr(bw, name))
    if case.dlogits is not None:
        errs["dlogits"] = tol_fn(case.dlogits.cpu().numpy().astype(np.float64), bw.dlogits)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, (errs, tol)
    return errs


def _run(cfg, tol_fn, tol):
    case = BwdCase(cfg)
    case.run()
    fw, bw = case.oracle_backward()
    errs = _compare(case, fw, bw, tol_fn, tol)
    print(f"  {tol_fn.__name__} vs oracle: {errs}")
    # run-to-run bit-identical
    first = [t.clone() for t in (case.dx, case.dp, case.dwg, case.dwu, case.dwd)]
    case.run()
    for a, b in zip(first, (case.dx, case.dp, case.dwg, case.dwu, case.dwd)):
        assert torch.equal(a, b)
    return errs


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (2, 3)])
def test_backward_tiny_bf16(e0, E_loc):
    _run(datagen.CONFIGS["tiny"].replace(e0=e0, E_loc=E_loc), max_rel_err, BF16_TOL)


@pytest.mark.parametrize("e0,E_loc", [(0, 8), (1, 5)])
def test_backward_tiny_mxfp8(e0, E_loc):
    cfg = datagen.CONFIGS["tiny"].replace(e0=e0, E_loc=E_loc, dtype="mxfp8", x_std=1.0, M=32)
    _run(cfg, frob_rel_err, MX_TOL)


def test_backward_multitile_bf16():
    # 1536 tokens, H 1024, I 384 (a partial 256-column tile), 16 experts, top-4, experts 4..7:
    # several row tiles per expert with ragged edges, several weight-gradient K stages.
    cfg = datagen.CONFIGS["tiny"].replace(S=3, T=512, H=1024, E=16, K=4, I=384, e0=4, E_loc=4,
                                          x_std=1.0)
    _run(cfg, max_rel_err, BF16_TOL)


def test_backward_multitile_mxfp8():
    cfg = datagen.CONFIGS["tiny"].replace(S=3, T=512, H=1024, E=16, K=4, I=384, e0=4, E_loc=4,
                                          x_std=1.0, dtype="mxfp8", M=256)
    _run(cfg, frob_rel_err, MX_TOL)


def _expert_rows(case, hdr, perm, e):
    """Token ids and gates of expert e's rows, in schedule order, from the GPU's schedule table
    (bit-exact to the oracle's, checked by the schedule tests)."""
    cfg = case.cfg
    counts = hdr[16:16 + cfg.E_loc].numpy()
    offs = hdr[96:96 + cfg.E_loc + 1].numpy()
    pairs = perm.numpy()[offs[e]:offs[e] + counts[e]]
    return pairs // cfg.K, case.layer.p.cpu().numpy()[pairs].astype(np.float64)


def _check_expert_wgrads(case, hdr, perm, experts, nrows, tol_fn, tol, seed):
    """Sampled rows of dWg, dWu (rows i) and dWd (rows j) of each listed expert, recomputed by
    the oracle from that expert's rows alone (mo.expert_wgrad_rows)."""
    cfg = case.cfg
    W = case.oracle_weights()
    rng = np.random.default_rng(seed)
    errs = {}
    for e in experts:
        n_of, p_rows = _expert_rows(case, hdr, perm, e)
        gi = np.sort(rng.choice(cfg.I, nrows, replace=False))
        hi = np.sort(rng.choice(cfg.H, nrows, replace=False))
        dwg, dwu, dwd = mo.expert_wgrad_rows(mo.decode_bf16(case.x_h[n_of]),
                                             mo.decode_bf16(case.dout_h[n_of]), p_rows, W, e,
                                             gi, hi, workers=16)
        errs[e] = {"dwg": tol_fn(case.dwg[e].cpu().numpy()[gi], dwg),
                   "dwu": tol_fn(case.dwu[e].cpu().numpy()[gi], dwu),
                   "dwd": tol_fn(case.dwd[e].cpu().numpy()[hi], dwd),
                   "rows": len(n_of)}
    print(f"  sampled weight-gradient errors per expert: {errs}")
    for e, d in errs.items():
        for k in ("dwg", "dwu", "dwd"):
            assert d[k] <= tol, (e, k, d)


def test_backward_dsv3_sampled():
    """DeepSeek-V3-shaped local share at full size; dX and dp of 64 sampled touched tokens, and
    4 sampled rows of dWg, dWu and dWd of every local expert, recomputed by the oracle."""
    cfg = datagen.CONFIGS["dsv3"]
    case = BwdCase(cfg)
    case.run()
    hdr, perm, tokpos, touched = case.layer.table()
    U = int(hdr[2])
    rng = np.random.default_rng(1)
    sample = np.sort(rng.choice(touched.numpy()[:U], 64, replace=False))
    fw = case.oracle_forward(tokens=sample)
    W = case.oracle_weights()
    bw = mo.backward(fw, lambda r: mo.decode_bf16(case.dout_h[sample[r]]), W, cfg.K, cfg.e0,
                     cfg.E_loc, cfg.E)
    got = mo.decode_bf16(host_u16(case.dx)[sample])
    errs = {"dx": max_rel_err(got, bw.dx)}
    dp = case.dp.cpu().numpy().reshape(cfg.N, cfg.K)[sample]
    local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
    errs["dp"] = max_rel_err(dp[local], bw.dp[local])
    print(f"  max|err|/max|ref|: {errs}")
    assert all(v <= BF16_TOL for v in errs.values()), errs
    _check_expert_wgrads(case, hdr, perm, range(cfg.E_loc), 4, max_rel_err, BF16_TOL, seed=3)


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_backward_reuses_ring_after_fused_forward(dtype):
    """Reverse ring walk: after a fused forward through the smallest ring (2 activation slots
    per XCD: ~16 of ~64 row tiles stay resident) the backward restores the resident tiles'
    activations and replays the rest. Matches the oracle, and equals bit for bit the backward
    after a staged forward (which leaves nothing resident, so every row is replayed)."""
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, dtype=dtype, M=64, x_std=1.0)
    ring = mok.query_sizes(mok.desc_from_config(cfg)).ring_min_bytes
    case = BwdCase(cfg, fused=True, ring_bytes=ring)
    case.run(fused=True)
    after_fused = case.grads()
    fw, bw = case.oracle_backward()
    tol_fn, tol = (max_rel_err, BF16_TOL) if dtype == "bf16" else (frob_rel_err, MX_TOL)
    _compare(case, fw, bw, tol_fn, tol)
    case.run(fused=False)
    for a, b in zip(after_fused, case.grads()):
        assert torch.equal(a, b)
    case.run(fused=True)
    for a, b in zip(after_fused, case.grads()):
        assert torch.equal(a, b)


def test_backward_dsv3_after_fused_forward_equals_staged():
    """DeepSeek-V3-shaped local share through the 256 MiB ring (the benchmarked launch
    configuration): the backward that reuses the resident tiles equals the full-replay backward
    bit for bit, and a repeated fused forward + backward reproduces every output bit for bit."""
    case = BwdCase(datagen.CONFIGS["dsv3"], fused=True)
    case.run(fused=True)
    after_fused = case.grads() + [case.out.clone()]
    case.run(fused=False)
    for a, b in zip(after_fused, case.grads()):
        assert torch.equal(a, b)
    case.out.zero_()
    case.run(fused=True)
    for a, b in zip(after_fused, case.grads() + [case.out.clone()]):
        assert torch.equal(a, b)


def test_kimi_mxfp8_skew_sampled():
    """Kimi-K2-shaped local share in MXFP8 under Zipf-skewed routing, full size, fused forward
    through the ring and the backward that reuses it: counts bit-exact against the oracle's
    top-k over all tokens; forward outputs, dX and dp of 48 sampled touched tokens recomputed
    by the oracle one token at a time (every quantisation block of these outputs lies inside
    one token's row); sampled rows of dWg, dWu and dWd of the most and the least loaded expert
    recomputed from that expert's rows (their operands are blocked along tokens, so one column
    quantises alone); and a repeated run is bit-identical."""
    cfg = datagen.CONFIGS["kimi_mx_skew"]
    case = BwdCase(cfg, fused=True)
    case.run(fused=True)
    hdr, perm, tokpos, touched = case.layer.table()
    idx_all, _ = mo.topk_gating(case.logits_h, cfg.K)
    sched = mo.schedule(idx_all, cfg.e0, cfg.E_loc, cfg.M, 32)
    assert np.array_equal(hdr[16:16 + cfg.E_loc].numpy(), sched.counts)
    U = int(hdr[2])
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(touched.numpy()[:U], 48, replace=False))
    fw = case.oracle_forward(tokens=sample)
    W = case.oracle_weights()
    bw = mo.backward(fw, lambda r: mo.decode_bf16(case.dout_h[sample[r]]), W, cfg.K, cfg.e0,
                     cfg.E_loc, cfg.E)
    dp = case.dp.cpu().numpy().reshape(cfg.N, cfg.K)[sample]
    local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
    errs = {"out": frob_rel_err(case.out_rows(sample), fw.out),
            "dx": frob_rel_err(mo.decode_bf16(host_u16(case.dx)[sample]), bw.dx),
            "dp": frob_rel_err(dp[local], bw.dp[local])}
    print(f"  rel. Frobenius error of sampled tokens: {errs}")
    assert all(v <= MX_TOL for v in errs.values()), errs
    # weight gradients: sampled rows of the most and the least loaded local expert
    counts = hdr[16:16 + cfg.E_loc].numpy()
    experts = [int(np.argmax(counts)), int(np.argmin(counts))]
    _check_expert_wgrads(case, hdr, perm, experts, 4, frob_rel_err, MX_TOL, seed=6)
    # a second fused forward + backward reproduces every output bit for bit
    first = case.grads() + [case.out.clone()]
    case.out.zero_()
    case.run(fused=True)
    for a, b in zip(first, case.grads() + [case.out.clone()]):
        assert torch.equal(a, b)


def test_backward_after_timed_out_forward_replays_every_row():
    """A fused forward whose bounded wait expired leaves no ring record (only a forward that
    finished without error publishes one), so the backward that follows replays every row and
    equals, bit for bit, the backward after a staged forward."""
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, M=64, x_std=1.0)
    bad = BwdCase(cfg, fused=True, flags=mok.MOK_FLAG_SKIP_ONE_SIGNAL)
    L = bad.layer
    L.forward(bad.x_seg, bad.logits, bad.out_seg)
    assert mok.mok_device_status(L.ws) == 8
    mok.mok_layer_bwd(bad.d, bad.dout_seg, bad.x_seg, L.w, L.idx, L.p, L.saved, L.ring, L.slots,
                      bad.dx_seg, bad.dp, bad.dlogits, bad.dwg, bad.dwu, bad.dwd, bad.bws)
    torch.cuda.synchronize()
    assert mok.mok_device_status(bad.bws) == 0
    good = BwdCase(cfg)
    good.run(fused=False)
    for a, b in zip(bad.grads(), good.grads()):
        assert torch.equal(a, b)


def _packed_reference(wg, wu, wd):
    """The BF16 packed planes as the C header states them, built by rearranging the weights in
    torch: in a plane of R rows and reduction length K, the 1 KB block (n32, k16) holds in lane l
    the elements 16 k16 + 8 (l // 32) .. +7 of row 32 n32 + l % 32; planes in the order gate/up
    (64-row blocks alternating Wg and Wu), Wd, Wd^T, [Wg^T | Wu^T]."""
    E, I, H = wg.shape

    def plane(W):
        e, R, K = W.shape
        t = W.reshape(e, R // 32, 32, K // 16, 2, 8).permute(0, 1, 3, 4, 2, 5)
        return t.contiguous().reshape(-1)

    gu = torch.stack([wg.reshape(E, I // 64, 64, H), wu.reshape(E, I // 64, 64, H)], dim=2)
    dx = torch.cat([wg.transpose(1, 2), wu.transpose(1, 2)], dim=2)
    return torch.cat([plane(gu.reshape(E, 2 * I, H)), plane(wd), plane(wd.transpose(1, 2)),
                      plane(dx)])


def _packed_reference_mx(wg, wu, wd):
    """The MXFP8 packed planes as the C header states them, from mok_quantize_mx's codes and
    scales in both blockings: 2 KB block (n32, k64) holds in lane l of its first 1 KB the codes
    64 k64 + 16 (l // 32) .. +15 of row 32 n32 + l % 32 and in its second 1 KB the 16 codes 32
    further; then the scale planes, 64 bytes per block, byte l the scale of row 32 n32 + l % 32,
    block 2 k64 + l // 32. Code planes first (aligned to 256 bytes), then the scale planes."""
    E, I, H = wg.shape

    def quant(src, transpose):
        b, r, c = src.shape
        orow, ocol = (c, r) if transpose else (r, c)
        q = torch.empty((b, orow, ocol), dtype=torch.uint8, device=src.device)
        sc = torch.empty((b, orow, ocol // 32), dtype=torch.uint8, device=src.device)
        mok.mok_quantize_mx(src, transpose, q, sc)
        return q, sc

    (gq, gs), (uq, us), (dq, ds) = quant(wg, False), quant(wu, False), quant(wd, False)
    (gtq, gts), (utq, uts), (dtq, dts) = quant(wg, True), quant(wu, True), quant(wd, True)

    def codes(W):
        e, R, K = W.shape
        t = W.reshape(e, R // 32, 32, K // 64, 2, 2, 16).permute(0, 1, 3, 4, 5, 2, 6)
        return t.contiguous().reshape(-1)

    def scales(S):
        e, R, KB = S.shape
        t = S.reshape(e, R // 32, 32, KB // 2, 2).permute(0, 1, 3, 4, 2)
        return t.contiguous().reshape(-1)

    def inter(a, b, w):
        return torch.stack([a.reshape(E, I // 64, 64, w), b.reshape(E, I // 64, 64, w)],
                           dim=2).reshape(E, 2 * I, w)

    c = torch.cat([codes(inter(gq, uq, H)), codes(dq), codes(dtq), codes(torch.cat([gtq, utq], 2))])
    pad = torch.zeros((-c.numel()) % 256, dtype=torch.uint8, device=c.device)
    sc = torch.cat([scales(inter(gs, us, H // 32)), scales(ds), scales(dts),
                    scales(torch.cat([gts, uts], 2))])
    return torch.cat([c, pad, sc])


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_packed_weights_match_the_stated_layout_and_per_call_packing(dtype):
    """The planes mok_pack_weights writes (the layer's default) are exactly the layout the C
    header states, byte for byte; and fused and staged forward + backward reading them give bit
    for bit the outputs of calls that pack into their own workspace each time. I = 384 leaves a
    half column tile (128 rows of the packed Wd^T plane) at each expert's end."""
    cfg = datagen.CONFIGS["tiny"].replace(S=3, T=512, H=1024, E=16, K=4, I=384, e0=4, E_loc=4,
                                          M=64, x_std=1.0, dtype=dtype)
    ring = 4 * mok.query_sizes(mok.desc_from_config(cfg)).ring_min_bytes
    case = BwdCase(cfg, fused=True, ring_bytes=ring)
    assert case.layer.w.packed
    n = case.layer.sizes.packed_bytes
    m = cfg.E_loc * cfg.H * cfg.I
    assert n == (12 * m if dtype == "bf16" else (6 * m + 255) // 256 * 256 + 6 * m // 32)
    got = torch.empty(n, dtype=torch.uint8, device="cuda")
    mok.mok_pack_weights(case.d, case.layer.w, got)
    if dtype == "bf16":
        ref = _packed_reference(case.wg, case.wu, case.wd).view(torch.uint8)
    else:
        ref = _packed_reference_mx(case.wg, case.wu, case.wd)
    assert torch.equal(got, ref)
    results = []
    for packed in (True, False):
        case.layer.set_weights(case.wg, case.wu, case.wd, packed=packed)
        assert bool(case.layer.w.packed) == packed
        for fused in (True, False):
            case.out.zero_()
            case.run(fused=fused)
            results.append(case.grads() + [case.out.clone()])
    fw, bw = case.oracle_backward()
    tol_fn, tol = (max_rel_err, BF16_TOL) if dtype == "bf16" else (frob_rel_err, MX_TOL)
    errs = _compare(case, fw, bw, tol_fn, tol)
    print(f"  {tol_fn.__name__} vs oracle: {errs}")
    for other in results[1:]:
        for a, b in zip(results[0], other):
            assert torch.equal(a, b)
