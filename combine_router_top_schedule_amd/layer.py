"""Buffer ownership for one layer instance: allocates every device buffer libmok needs (with
torch, on the current device) and calls the C entry points. Argument marshalling only."""
from __future__ import annotations

from typing import Optional

import torch

from . import (MOK_MXFP8, desc, mok_autotune, mok_combine, mok_dispatch, mok_expert_ffn,
               mok_layer_bwd, mok_layer_fwd, mok_pack_weights, mok_quantize_mx, mok_schedule,
               query_sizes, seg_table, weights_struct)


def _bytes(n, device):
    return torch.empty(int(max(n, 256)), dtype=torch.uint8, device=device)


class MokLayer:
    """One GPU's share of the MoE layer with its workspace, schedule table, ring and slots.

    x, dout: BF16 bit tensors [S*T][H] (int16 / uint16 / bfloat16 storage) on the device.
    Weights: BF16 tensors wg, wu [E_loc][I][H], wd [E_loc][H][I].
    """

    def __init__(self, d, device="cuda", staged: bool = True, fused: bool = True):
        self.d = d
        self.sizes = query_sizes(d)
        s = self.sizes
        self.device = device
        self.N = d.num_segments * d.tokens_per_segment
        self.mx = d.dtype == MOK_MXFP8
        self.saved = _bytes(s.saved_bytes, device)
        self.ws = _bytes(s.ws_bytes, device)
        self.slots = _bytes(s.slots_bytes, device)
        self.idx = torch.empty(self.N * d.top_k, dtype=torch.int32, device=device)
        self.p = torch.empty(self.N * d.top_k, dtype=torch.float32, device=device)
        self.xd = _bytes(s.xd_bytes, device) if staged else None
        self.act = _bytes(s.act_bytes, device) if staged else None
        self.ring = _bytes(d.ring_bytes, device) if fused else None
        self.bws = None
        self.w = None
        self._keep = []

    # ---- weights ---------------------------------------------------------------------------
    def set_weights(self, wg, wu, wd, packed: bool = True):
        """BF16 masters. In MXFP8 mode they are quantised here (forward blocking along each
        GEMM's reduction axis, and the transposed backward blocking). With `packed`, the GEMMs'
        packed weight planes are made here once (else every call packs them into its
        workspace)."""
        d = self.d
        self._keep = [wg, wu, wd]
        E, I, H = d.num_local_experts, d.intermediate, d.hidden
        dev = self.device
        if not self.mx:
            self.w = weights_struct(wg, wu, wd)
        else:
            def q(src, rows, cols, transpose):
                orow, ocol = (cols, rows) if transpose else (rows, cols)
                c = torch.empty((E, orow, ocol), dtype=torch.uint8, device=dev)
                s = torch.empty((E, orow, ocol // 32), dtype=torch.uint8, device=dev)
                mok_quantize_mx(src, transpose, c, s)
                self._keep += [c, s]
                return c, s

            wg_q, wg_s = q(wg, I, H, False)
            wu_q, wu_s = q(wu, I, H, False)
            wd_q, wd_s = q(wd, H, I, False)
            wgt_q, wgt_s = q(wg, I, H, True)
            wut_q, wut_s = q(wu, I, H, True)
            wdt_q, wdt_s = q(wd, H, I, True)
            self.w = weights_struct(wg, wu, wd, wg_q=wg_q, wg_s=wg_s, wu_q=wu_q, wu_s=wu_s,
                                    wd_q=wd_q, wd_s=wd_s, wgt_q=wgt_q, wgt_s=wgt_s, wut_q=wut_q,
                                    wut_s=wut_s, wdt_q=wdt_q, wdt_s=wdt_s)
        if packed:
            buf = _bytes(query_sizes(d).packed_bytes, dev)
            mok_pack_weights(d, self.w, buf)
            self._keep.append(buf)
            self.w.packed = buf.data_ptr()

    # ---- segment pointer tables ---------------------------------------------------------------
    def segs(self, rows):
        t = seg_table(rows, self.d.num_segments, self.d.tokens_per_segment)
        self._keep.append(t)
        return t

    # ---- staged path ------------------------------------------------------------------------
    def schedule(self, logits):
        mok_schedule(self.d, logits, self.idx, self.p, self.saved, self.ws)

    def dispatch(self, x_seg):
        mok_dispatch(self.d, self.saved, x_seg, self.xd, self.ws)

    def expert_ffn(self):
        mok_expert_ffn(self.d, self.saved, self.xd, self.w, self.act, self.slots, self.ws)

    def combine(self, out_seg, weighted: bool = True):
        mok_combine(self.d, self.saved, self.idx, self.p if weighted else None, self.slots,
                    out_seg, self.ws)

    def forward_staged(self, x_seg, logits, out_seg):
        self.schedule(logits)
        self.dispatch(x_seg)
        self.expert_ffn()
        self.combine(out_seg)

    # ---- fused path -------------------------------------------------------------------------
    def forward(self, x_seg, logits, out_seg):
        mok_layer_fwd(self.d, x_seg, logits, self.w, out_seg, self.idx, self.p, self.saved,
                      self.ring, self.slots, self.ws)

    def autotune(self, x_seg, logits, out_seg, reps: int = 3, apply: bool = True):
        """Time the fused forward over candidate minibatch sizes and dispatch-CU counts (this
        layer's buffers fit every candidate) and, with `apply`, use the fastest from now on.
        Returns (tuned descriptor, best ms, all measurements)."""
        tuned, best, table = mok_autotune(self.d, x_seg, logits, self.w, out_seg, self.idx,
                                          self.p, self.saved, self.ring, self.slots, self.ws, reps)
        if apply:
            self.d = tuned
        return tuned, best, table

    def backward(self, dout_seg, x_seg, dx_seg, dp, dlogits, dwg, dwu, dwd):
        """Backward of the last forward (reads the schedule table, ring and slots it left)."""
        if self.bws is None:
            self.bws = _bytes(self.sizes.bwd_ws_bytes, self.device)
        mok_layer_bwd(self.d, dout_seg, x_seg, self.w, self.idx, self.p, self.saved, self.ring,
                      self.slots, dx_seg, dp, dlogits, dwg, dwu, dwd, self.bws)

    # ---- views of the schedule table (tests) ------------------------------------------------
    def header(self):
        return self.saved[:1024].view(torch.int32).cpu()

    def tiles(self):
        """The grouped-GEMM tile table the last forward used: int32 [n][4] rows
        (minibatch, local expert, first row, rows), copied to the host."""
        s = self.sizes
        n = int(self.ws[8:12].view(torch.int32).item())
        off = int(s.tiles_offset)
        return self.ws[off:off + 16 * n].view(torch.int32).reshape(n, 4).cpu()

    def table(self):
        """(header, perm, tokpos, touched) of the schedule table, copied to the host."""
        s = self.sizes
        i32 = lambda off, n: self.saved[off:off + 4 * n].view(torch.int32).cpu()
        hdr = self.header()
        return (hdr, i32(s.perm_offset, int(s.rows_max)),
                i32(s.tokpos_offset, self.N * self.d.top_k), i32(s.touched_offset, self.N))
