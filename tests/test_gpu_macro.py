"""Macrobatch interleave (mok_layer_fwd_macro): several layer calls in one persistent launch.

Every output equals, bit for bit, that of separate mok_layer_fwd calls, and the backward of each
macrobatch after the joint launch (reusing the ring slots its tiles still hold) equals its
backward after a staged forward."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import datagen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import combine_router_top_schedule_amd as mok
from combine_router_top_schedule_amd.layer import MokLayer
from tests._gpu import dev_u16


class Macro:
    """Inputs and outputs of one macrobatch: its own tokens, logits and upstream gradient
    (seeded by `seed`), the shared weights of `cfg` (seed 0)."""

    def __init__(self, cfg, seed, layer):
        c = cfg.replace(seed=seed)
        self.x = dev_u16(datagen.x_all(c))
        self.dout = dev_u16(datagen.dout_all(c))
        self.logits = torch.from_numpy(datagen.logits(c)).cuda()
        s = layer.sizes
        self.saved = torch.zeros(int(s.saved_bytes), dtype=torch.uint8, device="cuda")
        self.slots = torch.empty(int(s.slots_bytes), dtype=torch.uint8, device="cuda")
        N, K = cfg.N, cfg.K
        self.idx = torch.empty(N * K, dtype=torch.int32, device="cuda")
        self.p = torch.empty(N * K, dtype=torch.float32, device="cuda")
        self.out = torch.zeros((N, cfg.H), dtype=torch.int16, device="cuda")
        self.x_seg, self.out_seg, self.dout_seg = (layer.segs(t) for t in (self.x, self.out, self.dout))


def _setup(cfg, B):
    layer = MokLayer(mok.desc_from_config(cfg), staged=True, fused=True)
    w = datagen.weights(cfg)
    layer.set_weights(*(dev_u16(w[k]) for k in ("wg", "wu", "wd")))
    mbs = [Macro(cfg, b, layer) for b in range(B)]
    ws = torch.zeros(mok.macro_ws_size(layer.d, B), dtype=torch.uint8, device="cuda")
    return layer, mbs, ws


def _separate(layer, mbs):
    """Reference: one mok_layer_fwd per macrobatch (the layer's own saved/slots/idx/p), copied."""
    outs = []
    for m in mbs:
        m.out.zero_()
        layer.forward(m.x_seg, m.logits, m.out_seg)
        torch.cuda.synchronize()
        assert mok.mok_device_status(layer.ws) == 0
        outs.append((m.out.clone(), layer.idx.clone(), layer.p.clone()))
    return outs


def _macro(layer, mbs, ws):
    for m in mbs:
        m.out.zero_()
    mok.mok_layer_fwd_macro(layer.d, [m.x_seg for m in mbs], [m.logits for m in mbs], layer.w,
                            [m.out_seg for m in mbs], [m.idx for m in mbs], [m.p for m in mbs],
                            [m.saved for m in mbs], layer.ring, [m.slots for m in mbs], ws)
    torch.cuda.synchronize()
    assert mok.mok_device_status(ws) == 0


def _grads(layer, m, cfg, saved, ring):
    """mok_layer_bwd of macrobatch m with the given schedule table and ring (None: replay)."""
    dx = torch.zeros((cfg.N, cfg.H), dtype=torch.int16, device="cuda")
    dp = torch.zeros(cfg.N * cfg.K, dtype=torch.float32, device="cuda")
    dwg = torch.empty((cfg.E_loc, cfg.I, cfg.H), dtype=torch.float32, device="cuda")
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((cfg.E_loc, cfg.H, cfg.I), dtype=torch.float32, device="cuda")
    dl = (torch.zeros((cfg.N, cfg.E), dtype=torch.float32, device="cuda")
          if cfg.E_loc == cfg.E else None)
    bws = torch.empty(int(layer.sizes.bwd_ws_bytes), dtype=torch.uint8, device="cuda")
    mok.mok_layer_bwd(layer.d, m.dout_seg, m.x_seg, layer.w, m.idx, m.p, saved, ring, m.slots,
                      layer.segs(dx), dp, dl, dwg, dwu, dwd, bws)
    torch.cuda.synchronize()
    return [dx, dp, dwg, dwu, dwd] + ([dl] if dl is not None else [])


@pytest.mark.parametrize("dtype", ["bf16", "mxfp8"])
def test_macro_forward_equals_separate_calls_and_backward_reuses_its_ring(dtype):
    cfg = datagen.CONFIGS["tiny"].replace(S=4, T=256, M=64, x_std=1.0, dtype=dtype)
    layer, mbs, ws = _setup(cfg, 3)
    ref = _separate(layer, mbs)
    _macro(layer, mbs, ws)
    for m, (out, idx, p) in zip(mbs, ref):
        assert torch.equal(m.out, out) and torch.equal(m.idx, idx) and torch.equal(m.p, p)
    # backward of each macrobatch, last one first, reusing the ring slots its tiles still hold
    for m in reversed(mbs):
        got = _grads(layer, m, cfg, m.saved, layer.ring)
        # reference: the staged forward of this macrobatch, then its full-replay backward
        layer.forward_staged(m.x_seg, m.logits, m.out_seg)
        torch.cuda.synchronize()
        ref_g = _grads(layer, m, cfg, layer.saved, None)
        for a, b in zip(got, ref_g):
            assert torch.equal(a, b)


def test_macro_forward_dsv3_equals_separate_calls():
    """Two DeepSeek-V3-shaped layer calls in one launch: bit-identical to two separate calls;
    prints both timings."""
    cfg = datagen.CONFIGS["dsv3"]
    layer, mbs, ws = _setup(cfg, 2)
    ref = _separate(layer, mbs)
    _macro(layer, mbs, ws)
    for m, (out, idx, p) in zip(mbs, ref):
        assert torch.equal(m.out, out) and torch.equal(m.idx, idx) and torch.equal(m.p, p)
    ev = lambda: torch.cuda.Event(enable_timing=True)
    t_sep, t_mac = [], []
    for _ in range(5):
        a, b, c = ev(), ev(), ev()
        a.record()
        for m in mbs:
            layer.forward(m.x_seg, m.logits, m.out_seg)
        b.record()
        mok.mok_layer_fwd_macro(layer.d, [m.x_seg for m in mbs], [m.logits for m in mbs],
                                layer.w, [m.out_seg for m in mbs], [m.idx for m in mbs],
                                [m.p for m in mbs], [m.saved for m in mbs], layer.ring,
                                [m.slots for m in mbs], ws)
        c.record()
        torch.cuda.synchronize()
        t_sep.append(a.elapsed_time(b)); t_mac.append(b.elapsed_time(c))
    print(f"  two DSv3 forward calls: separate {np.median(t_sep):.3f} ms, one macro launch "
          f"{np.median(t_mac):.3f} ms")
