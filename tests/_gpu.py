"""Helpers for the GPU parity tests: move datagen's arrays to the device, run libmok through its
binding, and bring results back as numpy arrays in the oracle's conventions."""
from __future__ import annotations

import numpy as np
import torch

import combine_router_top_schedule_amd as mok
import datagen
from combine_router_top_schedule_amd.layer import MokLayer
from oracle import moe_oracle as mo


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return mo.decode_bf16(a)


class Case:
    """Device inputs and a MokLayer for one datagen config."""

    def __init__(self, cfg: datagen.Config, M=None, ring_bytes=None, staged=True, fused=False,
                 with_dout=False, logits=None, flags=0, comm_cus=0):
        self.cfg = cfg
        self.d = mok.desc_from_config(cfg, M=M, ring_bytes=ring_bytes, flags=flags,
                                      comm_cus=comm_cus)
        self.layer = MokLayer(self.d, staged=staged, fused=fused)
        self.logits_h = datagen.logits(cfg) if logits is None else logits
        self.x_h = datagen.x_all(cfg)
        self.w_h = datagen.weights(cfg)
        self.logits = torch.from_numpy(self.logits_h).cuda()
        self.x = dev_u16(self.x_h)
        self.x_seg = self.layer.segs(self.x)
        self.wg, self.wu, self.wd = (dev_u16(self.w_h[k]) for k in ("wg", "wu", "wd"))
        self.layer.set_weights(self.wg, self.wu, self.wd)
        self.out = torch.zeros((cfg.N, cfg.H), dtype=torch.int16, device="cuda")
        self.out_seg = self.layer.segs(self.out)
        if with_dout:
            self.dout_h = datagen.dout_all(cfg)
            self.dout = dev_u16(self.dout_h)
            self.dout_seg = self.layer.segs(self.dout)

    # ---- oracle --------------------------------------------------------------------------
    def oracle_weights(self):
        return mo.weights_from_bits(self.w_h, self.cfg.dtype)

    def oracle_forward(self, tokens=None):
        """Oracle forward on all tokens, or only on `tokens` (outputs are per token)."""
        cfg = self.cfg
        W = self.oracle_weights()
        if tokens is None:
            return mo.forward(mo.bf16_rows(self.x_h), self.logits_h, W, cfg.K, cfg.e0, cfg.E_loc,
                              cfg.M, 32 if cfg.dtype == "mxfp8" else 1)
        tokens = np.asarray(tokens)
        return mo.forward(lambda r: mo.decode_bf16(self.x_h[tokens[r]]), self.logits_h[tokens], W,
                          cfg.K, cfg.e0, cfg.E_loc, cfg.M, 32 if cfg.dtype == "mxfp8" else 1)

    # ---- results ---------------------------------------------------------------------------
    def idx_p(self):
        K = self.cfg.K
        return (self.layer.idx.cpu().numpy().reshape(-1, K),
                self.layer.p.cpu().numpy().reshape(-1, K))

    def out_rows(self, tokens):
        return bf16_to_f64(host_u16(self.out)[np.asarray(tokens)])


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (the BF16 tolerance metric)."""
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def frob_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F (the MXFP8 tolerance metric)."""
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


BF16_TOL = 1e-2      # max |err| <= 1e-2 * max |ref|
MX_TOL = 3e-2        # relative Frobenius error


class BwdCase(Case):
    """Case with dOut and backward outputs; forward through the staged path (it fills the
    schedule table that mok_layer_bwd reads)."""

    def __init__(self, cfg, **kw):
        super().__init__(cfg, with_dout=True, **kw)
        d = self.d
        sz = self.layer.sizes
        self.bws = torch.empty(int(sz.bwd_ws_bytes), dtype=torch.uint8, device="cuda")
        self.dx = torch.zeros((cfg.N, cfg.H), dtype=torch.int16, device="cuda")
        self.dx_seg = self.layer.segs(self.dx)
        self.dp = torch.zeros(cfg.N * cfg.K, dtype=torch.float32, device="cuda")
        self.dlogits = (torch.zeros((cfg.N, cfg.E), dtype=torch.float32, device="cuda")
                        if cfg.E_loc == cfg.E else None)
        self.dwg = torch.empty((cfg.E_loc, cfg.I, cfg.H), dtype=torch.float32, device="cuda")
        self.dwu = torch.empty_like(self.dwg)
        self.dwd = torch.empty((cfg.E_loc, cfg.H, cfg.I), dtype=torch.float32, device="cuda")

    def run(self, fused: bool = False):
        """Forward (staged, or fused through the ring) then mok_layer_bwd."""
        L = self.layer
        if fused:
            L.forward(self.x_seg, self.logits, self.out_seg)
        else:
            L.forward_staged(self.x_seg, self.logits, self.out_seg)
        mok.mok_layer_bwd(self.d, self.dout_seg, self.x_seg, L.w, L.idx, L.p, L.saved, L.ring,
                          L.slots, self.dx_seg, self.dp, self.dlogits, self.dwg, self.dwu,
                          self.dwd, self.bws)
        torch.cuda.synchronize()
        assert mok.mok_device_status(L.ws) == 0
        # (the backward's workspace starts uninitialised: the call clears its error word)
        assert mok.mok_device_status(self.bws) == 0

    def grads(self):
        """Copies of every backward output."""
        out = [self.dx, self.dp, self.dwg, self.dwu, self.dwd]
        if self.dlogits is not None:
            out.append(self.dlogits)
        return [t.clone() for t in out]

    def oracle_backward(self, fw=None):
        cfg = self.cfg
        fw = fw or self.oracle_forward()
        W = self.oracle_weights()
        return fw, mo.backward(fw, mo.bf16_rows(self.dout_h), W, cfg.K, cfg.e0, cfg.E_loc, cfg.E)


class ArrayCase:
    """A layer on explicit arrays (float64 values exactly representable in BF16): one segment of
    N tokens, all experts [0, E_loc) local. Runs the staged or the fused forward and the
    backward; results come back as float64 arrays."""

    def __init__(self, x, dout, logits, wg, wu, wd, K, dtype="mxfp8", M=64, fused=False):
        from tests import mx_cases as mc
        N, H = x.shape
        E_loc, I, _ = wg.shape
        E = logits.shape[1]
        self.N, self.H, self.I, self.K, self.E, self.E_loc = N, H, I, K, E, E_loc
        d0 = mok.desc(H, E, K, I, 1, N, 0, E_loc, M, 0, dtype)
        ring = mok.query_sizes(d0).ring_min_bytes if fused else 0
        self.d = mok.desc(H, E, K, I, 1, N, 0, E_loc, M, ring, dtype)
        self.fused = fused
        self.layer = MokLayer(self.d, staged=not fused, fused=fused)
        bits = lambda a: dev_u16(mc.bf16_bits(a))
        self.x, self.dout = bits(x), bits(dout)
        self.logits = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).cuda()
        self.wg, self.wu, self.wd = bits(wg), bits(wu), bits(wd)
        self.layer.set_weights(self.wg, self.wu, self.wd)
        self.out = torch.zeros((N, H), dtype=torch.int16, device="cuda")
        self.dx = torch.zeros_like(self.out)
        self.x_seg, self.out_seg, self.dout_seg, self.dx_seg = (
            self.layer.segs(t) for t in (self.x, self.out, self.dout, self.dx))
        self.dp = torch.zeros(N * K, dtype=torch.float32, device="cuda")
        self.dlogits = (torch.zeros((N, E), dtype=torch.float32, device="cuda")
                        if E_loc == E else None)
        self.dwg = torch.zeros((E_loc, I, H), dtype=torch.float32, device="cuda")
        self.dwu = torch.zeros_like(self.dwg)
        self.dwd = torch.zeros((E_loc, H, I), dtype=torch.float32, device="cuda")
        self.bws = torch.empty(int(self.layer.sizes.bwd_ws_bytes), dtype=torch.uint8, device="cuda")

    def run(self):
        L = self.layer
        if self.fused:
            L.forward(self.x_seg, self.logits, self.out_seg)
        else:
            L.forward_staged(self.x_seg, self.logits, self.out_seg)
        mok.mok_layer_bwd(self.d, self.dout_seg, self.x_seg, L.w, L.idx, L.p, L.saved, L.ring,
                          L.slots, self.dx_seg, self.dp, self.dlogits, self.dwg, self.dwu,
                          self.dwd, self.bws)
        torch.cuda.synchronize()
        assert mok.mok_device_status(L.ws) == 0
        # (the backward's workspace starts uninitialised: the call clears its error word)
        assert mok.mok_device_status(self.bws) == 0
        f64 = lambda t: t.cpu().numpy().astype(np.float64)
        return dict(out=bf16_to_f64(host_u16(self.out)), dx=bf16_to_f64(host_u16(self.dx)),
                    dwg=f64(self.dwg), dwu=f64(self.dwu), dwd=f64(self.dwd),
                    dp=f64(self.dp).reshape(self.N, self.K))
