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


def test_backward_dsv3_sampled():
    """DeepSeek-V3-shaped local share at full size; dX and dp of 64 sampled touched tokens and
    8 sampled rows of dWg / dWu are recomputed by the oracle."""
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
    assert max_rel_err(got, bw.dx) <= BF16_TOL
    dp = case.dp.cpu().numpy().reshape(cfg.N, cfg.K)[sample]
    local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
    assert max_rel_err(dp[local], bw.dp[local]) <= BF16_TOL
    # Sampled rows i of dWg_e / dWu_e need only column i of the gate/up and down products
    # over the expert's rows: dWg_e[i] = sum_r dg[r, i] x_r.
    counts = hdr[16:16 + cfg.E_loc].numpy()
    offs = hdr[96:96 + cfg.E_loc + 1].numpy()
    perm = perm.numpy()
    p_all = case.layer.p.cpu().numpy()
    e = 1
    rows = perm[offs[e]:offs[e] + counts[e]]
    n_of = rows // cfg.K
    X = mo.decode_bf16(case.x_h[n_of])
    D = mo.decode_bf16(case.dout_h[n_of])
    p_row = p_all[rows].astype(np.float64)
    dwg = case.dwg[e].cpu().numpy()
    dwu = case.dwu[e].cpu().numpy()
    for i in rng.choice(cfg.I, 8, replace=False):
        g = X @ W.wg[e, i]
        u = X @ W.wu[e, i]
        a = D @ W.wd[e, :, i]
        sg = 1 / (1 + np.exp(-g))
        dh = p_row * a
        dg = dh * u * sg * (1 + g * (1 - sg))
        du = dh * g * sg
        assert max_rel_err(dwg[i], dg @ X) <= BF16_TOL
        assert max_rel_err(dwu[i], du @ X) <= BF16_TOL
    # Sampled rows j of dWd_e = sum_r p_r D_r[j] h_r need the expert's whole h = silu(g) u.
    G = X @ W.wg[e].T
    U_ = X @ W.wu[e].T
    Hh = G / (1 + np.exp(-G)) * U_
    dwd = case.dwd[e].cpu().numpy()
    for j in rng.choice(cfg.H, 8, replace=False):
        assert max_rel_err(dwd[j], (p_row * D[:, j]) @ Hh) <= BF16_TOL


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
    one token's row)."""
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
    assert frob_rel_err(case.out_rows(sample), fw.out) <= MX_TOL
    W = case.oracle_weights()
    bw = mo.backward(fw, lambda r: mo.decode_bf16(case.dout_h[sample[r]]), W, cfg.K, cfg.e0,
                     cfg.E_loc, cfg.E)
    assert frob_rel_err(mo.decode_bf16(host_u16(case.dx)[sample]), bw.dx) <= MX_TOL
    dp = case.dp.cpu().numpy().reshape(cfg.N, cfg.K)[sample]
    local = (fw.idx >= cfg.e0) & (fw.idx < cfg.e0 + cfg.E_loc)
    assert frob_rel_err(dp[local], bw.dp[local]) <= MX_TOL
