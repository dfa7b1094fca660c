"""GPU parity of the router's gate projection (mok_router_fwd) and its backward (mok_router_bwd)
against the oracle: logits = X W_r^T feeding the layer, then dW_r = dlogits^T X and the
projection's share of dX, with every expert local so dlogits is complete."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen
from oracle import moe_oracle as mo

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_router_top_schedule_amd as mok
from tests._gpu import BF16_TOL, BwdCase, dev_u16, host_u16, max_rel_err

CFGS = {
    "tiny": datagen.CONFIGS["tiny"],
    # 2048 tokens, hidden 1024, 64 experts all local, top-4: several token, expert and hidden
    # tiles in each of the three contractions
    "multitile": datagen.CONFIGS["tiny"].replace(S=4, T=512, H=1024, E=64, K=4, I=256, E_loc=64,
                                                 x_std=1.0, ring_bytes=32 << 20),
}


@pytest.mark.parametrize("name", list(CFGS))
def test_router_projection_and_its_gradients(name):
    cfg = CFGS[name]
    wr_h = datagen.router_weight(cfg)
    X = mo.decode_bf16(datagen.x_all(cfg))
    Wr = mo.decode_bf16(wr_h)
    L_o = mo.router_logits(X, Wr)
    # the oracle's top-k has no near-tie here, so both sides must pick the same experts
    Ls = np.sort(L_o, axis=1)[:, ::-1]
    assert (Ls[:, cfg.K - 1] - Ls[:, cfg.K]).min() > 1e-4
    case = BwdCase(cfg, fused=True, logits=np.zeros((cfg.N, cfg.E), np.float32))
    wr = dev_u16(wr_h)
    mok.mok_router_fwd(case.d, case.x_seg, wr, case.logits)
    torch.cuda.synchronize()
    errs = {"logits": max_rel_err(case.logits.cpu().numpy().astype(np.float64), L_o)}
    # layer forward and backward on the projected logits, then the projection's backward
    case.run(fused=True)
    dwr = torch.empty((cfg.E, cfg.H), dtype=torch.float32, device="cuda")
    rws = torch.empty(mok.router_ws_size(case.d), dtype=torch.uint8, device="cuda")
    mok.mok_router_bwd(case.d, case.x_seg, wr, case.dlogits, dwr, case.dx_seg, rws)
    torch.cuda.synchronize()
    idx, _ = case.idx_p()
    fw = mo.forward(lambda r: X[r], L_o, case.oracle_weights(), cfg.K, cfg.e0, cfg.E_loc, cfg.M)
    bw = mo.backward(fw, mo.bf16_rows(case.dout_h), case.oracle_weights(), cfg.K, cfg.e0,
                     cfg.E_loc, cfg.E)
    assert np.array_equal(idx, fw.idx)
    dwr_o, dxr_o = mo.router_backward(X, Wr, bw.dlogits)
    assert np.array_equal(fw.sched.touched, np.arange(cfg.N))
    errs["out"] = max_rel_err(case.out_rows(np.arange(cfg.N)), fw.out)
    errs["dlogits"] = max_rel_err(case.dlogits.cpu().numpy().astype(np.float64), bw.dlogits)
    errs["dwr"] = max_rel_err(dwr.cpu().numpy().astype(np.float64), dwr_o)
    errs["dx"] = max_rel_err(mo.decode_bf16(host_u16(case.dx)), bw.dx + dxr_o)
    print(f"  max|err|/max|ref|: {errs}")
    assert errs["logits"] <= 1e-5
    assert all(v <= BF16_TOL for v in errs.values()), errs
    # run-to-run bit-identical
    first = [dwr.clone(), case.dx.clone()]
    case.run(fused=True)
    mok.mok_router_bwd(case.d, case.x_seg, wr, case.dlogits, dwr, case.dx_seg, rws)
    torch.cuda.synchronize()
    assert torch.equal(first[0], dwr) and torch.equal(first[1], case.dx)


def test_router_projection_dsv3_sampled():
    """The gate projection of all 131,072 tokens of the DeepSeek-V3-shaped share (256 experts,
    hidden 7168) on 256 sampled tokens, and its time."""
    cfg = datagen.CONFIGS["dsv3"]
    x_h = datagen.x_all(cfg)
    wr_h = datagen.router_weight(cfg)
    x = dev_u16(x_h)
    d = mok.desc_from_config(cfg)
    seg = mok.seg_table(x, cfg.S, cfg.T)
    wr = dev_u16(wr_h)
    logits = torch.empty((cfg.N, cfg.E), dtype=torch.float32, device="cuda")
    mok.mok_router_fwd(d, seg, wr, logits)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        mok.mok_router_fwd(d, seg, wr, logits)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 5
    sample = np.sort(np.random.default_rng(4).choice(cfg.N, 256, replace=False))
    ref = mo.router_logits(mo.decode_bf16(x_h[sample]), mo.decode_bf16(wr_h))
    err = max_rel_err(logits.cpu().numpy()[sample].astype(np.float64), ref)
    tflops = 2.0 * cfg.N * cfg.E * cfg.H / (ms * 1e-3) / 1e12
    print(f"  logits max|err|/max|ref| {err:.2e}; {ms:.3f} ms = {tflops:.0f} TFLOP/s")
    assert err <= 1e-5
