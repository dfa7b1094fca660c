// Fused forward: one persistent kernel whose compute units are split into dispatch workers and
// GEMM workers that hand tiles to each other through counters in HBM, with no host
// synchronisation ("把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ②: SMs split into a
// communication group and an expert-FFN group that notify each other with local counters;
// part ③ and "Mixture-of-Kittens (MoK)", ring section: a fixed-size ring reused as soon as a
// batch of tokens has been consumed, no CPU involvement).
//
// MI355X layout of that idea: every XCD (8 per device, each with its own L2) runs its own
// pipeline. Workgroups learn their XCD from the hardware id; per XCD the first `comm` of them
// gather token rows (pull dispatch, MXFP8 quantisation fused) and the others run the gate/up
// and down GEMM tiles of the same row tiles. An XCD takes its next row tile from one global
// counter whenever it has free ring slots, so the row tiles spread over the XCDs by speed. A
// row tile (<= 256 expert-ordered rows of one expert inside one minibatch) is produced and
// consumed inside one XCD, so its ring bytes stay coherent in that XCD's L2: producers complete
// their stores before bumping a counter, and consumers read ring rows with agent-scope loads
// that miss in their CU's L1 (a slot is reused for one row tile after another, so an L1 line
// kept from an earlier tile would be stale). Each XCD owns a fixed share of the ring, cut into
// three kinds of slots used round-robin: gather slots hold a row tile's X rows until its
// gate/up tiles are done; h slots hold its h until its down tiles are done; activation slots
// hold its g|u, which only the backward reads, and after the kernel the last capa of them stay
// for the backward's reverse walk (it recomputes h from g|u). Splitting them lets one ring keep
// the g|u of many more row tiles than whole-tile slots would. A down-GEMM row whose pair is
// its token's only local pair (nearly all rows when a GPU holds a few experts of many) becomes
// the token's output row at once, bf16(p * bf16(y)), the merge over one term; the other rows
// are pushed to the pair slots and the weighted merge of the tokens with several local pairs
// runs as the next kernel on the stream.
//
// Work order and deadlock freedom: all workgroups are co-resident (cooperative launch, one per
// CU). The first `lag` row tiles of an XCD (lag = 2 with at least 3 activation slots per XCD,
// else 1; below the 3 gather slots) are gathered by all of its workgroups together,
// since no GEMM work exists before them; the later ones by the dispatch workers alone. Within an XCD the GEMM items are numbered gu(0) ..
// gu(lag-1), then blocks [gu(q+lag), dn(q)] for q = 0, 1, ... (gu = the gate/up column tiles of
// a row tile, dn = its down column tiles), so the down tiles of a row tile come `lag` blocks
// after its gate/up tiles and rarely wait for them. A GEMM worker that finishes an item takes
// the next number from the XCD's item counter, so items are handed out in increasing order to
// whichever worker is free. Every wait is on a lower-numbered item, already held by a running
// worker: dn(q) on gu(q), and gu(q) on the gather of tile q, whose slots were freed by
// dn(q - capa) and gu(q - capx), both numbered below gu(q) because capa > lag; before storing h,
// gu(q) also waits for dn(q - caph), the last reader of its h slot, numbered below gu(q)
// because caph > lag. Every wait is bounded; an expired wait sets the error word and all
// workers drain.
#include "k_ffn.h"
#include "mok_rows.h"

namespace mok {
namespace {

constexpr int kMaxXcd = kXcds;

// One macrobatch (one layer call) of a launch: its schedule table, tile table, token segments,
// push records and the ring record it leaves for its backward.
struct MacroArgs {
  const int32_t* perm;
  const MTile* tiles;
  const int32_t* ntiles;     // device word: tiles in this macrobatch's table
  const uint16_t* const* x_seg;
  PushTarget push;           // down-GEMM rows: pair slots, or the output row of a token's only
                             // local pair
  int32_t* rhdr;             // ring state for the backward (in saved): header,
  MTile* rtiles;             //   copy of the tile table,
  int32_t* rslot;            //   activation slot id (x * capa + slot) of every tile,
  int32_t* rowner;           //   the tile of this macrobatch that last used every slot (-1:
                             //   the slot's last tile belongs to another macrobatch)
};

struct FusedArgs {
  uint8_t* ring;
  int64_t ring_share;        // bytes of the ring owned by one XCD
  int64_t xsb, hsb, asb;     // bytes of one gather slot / h slot / activation slot
  int capx, caph, capa;      // gather slots / h slots / activation slots per XCD
  FfnShape s;
  FfnWeights w;
  int32_t* cnt;              // [kCntWords + (3 + kXcds) * B * tiles_max]
  int32_t* err;
  int64_t tiles_max;         // per macrobatch
  int B;                     // macrobatches, each a whole layer call; their row tiles form one
                             // list in macrobatch order
  MacroArgs mb[kMaxMacro];
  int comm_per_xcd;
  int K, T, dtype;
  int64_t NK;
  int spin_limit;
  uint32_t flags;
  TraceRec* trace;           // MOK_FLAG_TRACE: phase records (null without it)
  int64_t trace_max;
  int32_t* trace_count;
};

// Counter words: registration, the global row-tile counter, per XCD the number of row tiles it
// ended up with (-1 until known) and per XCD the next GEMM item. After them: landed / gu_done /
// dn_done per tile, then per XCD the tile id of its q-th row tile (-1 until known).
enum CntWords : int {
  kCntArrived = 0, kCntReg = 8, kCntEnd = 16, kCntNext = 24, kCntItem = 32, kCntExit = 40,
  kCntWords = 64
};

__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & (kMaxXcd - 1);  // HW_REG_XCC_ID
}

// After a counter wait no cache maintenance is needed: every read of ring rows is a GEMM
// A-operand stage load, issued at agent scope (sc1), so it misses in the CU's L1 and sees what
// other CUs of the XCD stored to L2. (A workgroup-scope invalidate is not enough: a CU that
// read or stored rows of a ring slot for an earlier tile can keep those lines in its L1; an
// agent-scope acquire after each wait, buffer_inv sc1, is correct but measured 1-2 % slower.)

// Thread 0 waits until *p >= target (bounded); returns false (for the whole workgroup) if the
// wait failed or another worker already reported an error.
__device__ bool wait_geq(const int32_t* p, int target, int32_t* err, int limit) {
  __shared__ int s_ok;
  if (threadIdx.x == 0) {
    int spins = 0, ok = 1;
    while (ld_relaxed(p) < target) {
      if (ld_relaxed(err) != 0) { ok = 0; break; }
      if (++spins > limit) { set_error(err, MOK_ERR_DEVICE_TIMEOUT); ok = 0; break; }
      __builtin_amdgcn_s_sleep(2);
    }
    if (ok && ld_relaxed(err) != 0) ok = 0;
    s_ok = ok;
  }
  __syncthreads();
  const bool ok = s_ok != 0;
  __syncthreads();
  return ok;
}

// The tile id of this XCD's q-th row tile, once its dispatch worker has taken it: >= 0, or
// INT32_MAX when the XCD gets no q-th tile, or -1 if the wait failed (for the whole workgroup).
// xq has tiles_max entries; no XCD can get more tiles than that.
__device__ int tile_of(const int32_t* xq, const int32_t* xend, int q, int64_t tiles_max,
                       int32_t* err, int limit) {
  __shared__ int s_t;
  if (threadIdx.x == 0) {
    int spins = 0, t = -1;
    if (q >= tiles_max) t = 0x7FFFFFFF;
    while (t < 0) {
      const int v = ld_relaxed(xq + q);
      if (v >= 0) { t = v; break; }
      const int e = ld_relaxed(xend);
      if (e >= 0 && q >= e) { t = 0x7FFFFFFF; break; }
      if (ld_relaxed(err) != 0) break;
      if (++spins > limit) { set_error(err, MOK_ERR_DEVICE_TIMEOUT); break; }
      __builtin_amdgcn_s_sleep(2);
    }
    s_t = t;
  }
  __syncthreads();
  const int t = s_t;
  __syncthreads();
  return t;
}

// All stores of this workgroup are complete (in L2), then thread 0 bumps the counter.
__device__ __forceinline__ void signal(int32_t* p) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) add_relaxed(p, 1);
}

// MXFP8 gather of a dispatch worker's rows: row j's source pointer is lane j's `sp`; its codes
// go to codes + j * rstep * H, its scales to scales + j * rstep * H / 32. Not inlined: the
// persistent kernel's GEMM paths hold the register file near its limit, and the quantiser's
// two rows in flight spilled when allocated together with them; as a call it gets its own
// allocation (the caller keeps almost nothing live across it).
__device__ __noinline__ void gather_rows_mx(int nr, int H, int lane, uint64_t sp, uint8_t* codes,
                                            uint8_t* scales, int rstep) {
  auto src_of = [&](int j) {
    const uint32_t lo = __shfl(uint32_t(sp), j, 64), hi = __shfl(uint32_t(sp >> 32), j, 64);
    return reinterpret_cast<const uint16_t*>((uint64_t(hi) << 32) | lo);
  };
  quant_rows_mx_2(
      nr, H, lane, src_of, [&](int j) { return codes + int64_t(j) * rstep * H; },
      [&](int j) { return scales + int64_t(j) * rstep * (H / 32); });
}

// Constant-rate clock for the phase trace (100 MHz on gfx950).
__device__ __forceinline__ uint64_t trace_clock() { return __builtin_amdgcn_s_memrealtime(); }

// Thread 0 appends one phase record (MOK_FLAG_TRACE); records past the capacity are counted
// but dropped.
__device__ __forceinline__ void trace_item(const FusedArgs& a, int kind, int x, int b, int tile,
                                           int item, uint64_t t_wait, uint64_t t_begin) {
  if (a.trace == nullptr || threadIdx.x != 0) return;
  const uint64_t t_end = trace_clock();
  const int i = add_relaxed(a.trace_count, 1);
  if (i < a.trace_max) {
    TraceRec r;
    r.wg = int(blockIdx.x);
    r.info = kind | (x << 8) | (b << 16);
    r.tile = tile;
    r.item = item;
    r.t_wait = t_wait;
    r.t_begin = t_begin;
    r.t_end = t_end;
    r.pad = 0;
    a.trace[i] = r;
  }
}

// MOK_FLAG_POISON: fill rows r0, r0 + rstep, ... (< kTileM) of a gather slot's X plane (and
// its MXFP8 scales), an activation slot's g|u and an h slot's h (and scales) with 0xFF bytes
// (NaN in BF16, E4M3 and UE8M0), so a read of a released slot before its next tile's data is
// written shows up as NaN. Rows are split exactly as the gather splits them, so each row's
// poison precedes its gathered bytes in one wave's program order (with a vmcnt wait between
// them).
__device__ void poison_rows(const ActPlanes& pl, bool gather_slot, bool gu_slot, bool h_slot,
                            int H, int I, bool mx, int r0, int rstep, int lane) {
  auto fill = [&](uint8_t* p, int64_t bytes) {
    uint32_t* w = reinterpret_cast<uint32_t*>(p);
    const int64_t nw = bytes / 4;
    for (int64_t i = lane; i < nw; i += 64) w[i] = 0xFFFFFFFFu;
    for (int64_t i = nw * 4 + lane; i < bytes; i += 64) p[i] = 0xFFu;
  };
  const int64_t xrow = mx ? H : 2 * int64_t(H);
  const int64_t hrow = mx ? I : 2 * int64_t(I);
  for (int r = r0; r < kTileM; r += rstep) {
    if (gather_slot) {
      fill(pl.x + r * xrow, xrow);
      if (mx) fill(pl.xs + int64_t(r) * (H / 32), H / 32);
    }
    if (gu_slot) fill(reinterpret_cast<uint8_t*>(pl.gu) + int64_t(r) * 4 * I, 4 * int64_t(I));
    if (h_slot) {
      fill(pl.h + r * hrow, hrow);
      if (mx) fill(pl.hs + int64_t(r) * (I / 32), I / 32);
    }
  }
}

// The work of one workgroup. Every exit is taken by the whole workgroup (the values deciding
// it come through LDS or from one thread's atomic), so the caller's exit protocol runs once.
template <bool MX>
__device__ __forceinline__ void layer_fwd_body(const FusedArgs& a, GemmLds& sm) {
  __shared__ int s_x, s_local, s_n[kMaxXcd], s_fail;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  // ---- registration: which XCD am I on, and how many workgroups share it ----
  if (tid == 0) {
    const int x = xcc_id();
    s_x = x;
    s_local = add_relaxed(a.cnt + kCntReg + x, 1);
    add_relaxed(a.cnt + kCntArrived, 1);
    int spins = 0;
    while (ld_relaxed(a.cnt + kCntArrived) < int(gridDim.x)) {
      if (++spins > a.spin_limit) { set_error(a.err, MOK_ERR_DEVICE_TIMEOUT); break; }
      __builtin_amdgcn_s_sleep(2);
    }
    for (int i = 0; i < kMaxXcd; ++i) s_n[i] = ld_relaxed(a.cnt + kCntReg + i);
    s_fail = ld_relaxed(a.err) != 0;
  }
  __syncthreads();
  if (s_fail) return;
  const int x = s_x, local = s_local;
  // active XCDs: those with at least one comm and one GEMM worker
  int nact = 0, ax = -1;
  for (int i = 0; i < kMaxXcd; ++i) {
    if (s_n[i] >= 2) {
      if (i == x) ax = nact;
      ++nact;
    }
  }
  if (ax < 0) return;
  const int nx = s_n[x];
  const int C = min(a.comm_per_xcd, nx - 1);
  // Row tiles of all macrobatches form one list: global tile g is tile g - s_first[b] of
  // macrobatch b, for the b with s_first[b] <= g < s_first[b + 1].
  __shared__ int s_first[kMaxMacro + 1];
  if (tid == 0) {
    int f = 0;
    for (int b = 0; b < a.B; ++b) {
      s_first[b] = f;
      f += min(*a.mb[b].ntiles, int(a.tiles_max));
    }
    s_first[a.B] = f;
  }
  __syncthreads();
  const int nt = s_first[a.B];
  const int64_t gmax = a.tiles_max * a.B;           // bound on global tile ids
  auto macro_of = [&](int g) {
    int b = 0;
    while (b + 1 < a.B && s_first[b + 1] <= g) ++b;
    return b;
  };
  const int ngu = a.s.I / 128;
  const int ndn = (a.s.H + kTileN - 1) / kTileN;
  int32_t* landed = a.cnt + kCntWords;
  int32_t* gu_done = landed + gmax;
  int32_t* dn_done = gu_done + gmax;
  int32_t* xq = dn_done + gmax + int64_t(x) * gmax;   // this XCD's tile ids
  int32_t* xend = a.cnt + kCntEnd + x;
  uint8_t* share = a.ring + int64_t(x) * a.ring_share;
  // Planes of this XCD's q-th row tile: X in gather slot q % capx, h in h slot q % caph, g|u in
  // activation slot q % capa.
  auto planes = [&](int q) {
    ActPlanes pl{};
    pl.x = share + int64_t(q % a.capx) * a.xsb;
    pl.xs = a.dtype == MOK_BF16 ? nullptr : pl.x + int64_t(kTileM) * a.s.H;
    pl.h = share + a.capx * a.xsb + int64_t(q % a.caph) * a.hsb;
    pl.hs = a.dtype == MOK_BF16 ? nullptr : pl.h + int64_t(kTileM) * a.s.I;
    pl.gu = reinterpret_cast<uint16_t*>(share + a.capx * a.xsb + a.caph * a.hsb +
                                        int64_t(q % a.capa) * a.asb);
    return pl;
  };

  // The tile id of this XCD's q-th row tile: workgroup 0 takes it from the global counter and
  // publishes it (row tiles are taken when this XCD has a free slot, so faster XCDs take more
  // of them); the others wait for the publication. Returns >= nt when there is none, -1 after
  // an error.
  __shared__ int s_mt;
  auto take_tile = [&](int q) -> int {
    if (local != 0) return tile_of(xq, xend, q, gmax, a.err, a.spin_limit);
    if (tid == 0) {
      int t = add_relaxed(a.cnt + kCntNext, 1);
      if (t >= nt) {
        t = 0x7FFFFFFF;
        __hip_atomic_store(xend, q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        // One thread per XCD records its tiles in order, so each slot's owner ends as the
        // last tile that used it (and only that tile's macrobatch claims the slot).
        const int slot = x * a.capa + q % a.capa;
        const int b = macro_of(t), tb = t - s_first[b];
        const MacroArgs& m = a.mb[b];
        m.rtiles[tb] = m.tiles[tb];
        m.rslot[tb] = slot;
        for (int o = 0; o < a.B; ++o) a.mb[o].rowner[slot] = o == b ? tb : -1;
        __hip_atomic_store(xq + q, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      s_mt = t;
    }
    __syncthreads();
    const int mt = s_mt;
    __syncthreads();
    return mt;
  };
  // Pull the rows r = r0, r0 + rstep, ... of row tile mt into its gather slot, then count this
  // workgroup in landed[mt]. Lane j looks up row j's source first (one round of dependent
  // loads per tile instead of one per row).
  auto gather = [&](int q, int mt, int r0, int rstep) {
    const int b = macro_of(mt);
    const MacroArgs& m = a.mb[b];
    const MTile tl = m.tiles[mt - s_first[b]];
    const ActPlanes pl = planes(q);
    const uint16_t* my_src = nullptr;
    {
      const int r = r0 + lane * rstep;
      if (lane * rstep < kTileM && r < tl.nrows) {
        const int32_t pair = m.perm[tl.row0 + r];
        if (pair >= 0 && pair < a.NK) {      // (a pad row, or a failed schedule: zeros)
          const int64_t n = pair / a.K;
          my_src = m.x_seg[n / a.T] + (n % a.T) * int64_t(a.s.H);
        }
      }
    }
    const uint64_t sp = reinterpret_cast<uint64_t>(my_src);
    auto src_of = [&](int j) {
      const uint32_t lo = __shfl(uint32_t(sp), j, 64), hi = __shfl(uint32_t(sp >> 32), j, 64);
      return reinterpret_cast<const uint16_t*>((uint64_t(hi) << 32) | lo);
    };
    if (!MX && a.s.H <= 8 * kRowBatchChunks) {
      const int nr = r0 < tl.nrows ? (tl.nrows - r0 + rstep - 1) / rstep : 0;
      copy_rows_bf16_2(nr, a.s.H, lane, src_of, [&](int j) {
        return reinterpret_cast<uint16_t*>(pl.x) + int64_t(r0 + j * rstep) * a.s.H;
      });
    } else if (MX && a.s.H <= 8 * kRowBatchChunks) {
      const int nr = r0 < tl.nrows ? (tl.nrows - r0 + rstep - 1) / rstep : 0;
      gather_rows_mx(nr, a.s.H, lane, sp, pl.x + int64_t(r0) * a.s.H,
                     pl.xs + int64_t(r0) * (a.s.H / 32), rstep);
    } else {
      for (int j = 0; r0 + j * rstep < tl.nrows; ++j) {
        const int r = r0 + j * rstep;
        const uint16_t* src = src_of(j);
        if (MX) quant_row_mx(src, pl.x + int64_t(r) * a.s.H, pl.xs + int64_t(r) * (a.s.H / 32), a.s.H, lane);
        else copy_row_bf16(src, reinterpret_cast<uint16_t*>(pl.x) + int64_t(r) * a.s.H, a.s.H, lane);
      }
    }
    const bool skip = (a.flags & MOK_FLAG_SKIP_ONE_SIGNAL) && q == 0 && ax == 0 && local == 0;
    if (!skip) signal(landed + mt);
  };

  // ---- prologue: the first `lag` row tiles are gathered by every workgroup of the XCD ----
  const int lag = a.capa > 2 ? 2 : 1;                 // lag < capx: the prologue never waits
  bool ended = false;
  for (int q = 0; q < lag; ++q) {
    const uint64_t tw = trace_clock();
    const int mt = take_tile(q);
    if (mt < 0) return;
    if (mt >= nt) {
      ended = true;
      break;
    }
    const uint64_t tb = trace_clock();
    if (a.flags & MOK_FLAG_POISON) {
      const ActPlanes pl = planes(q);
      poison_rows(pl, true, true, true, a.s.H, a.s.I, MX, local * 4 + wave, 4 * nx, lane);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    gather(q, mt, local * 4 + wave, 4 * nx);
    const int b = macro_of(mt);
    trace_item(a, kTrPrologueGather, x, b, mt - s_first[b], q, tw, tb);
  }

  if (local < C) {
    // ---- dispatch worker: the later row tiles. Tile q reuses the gather slot of tile q - capx
    // once its gate/up tiles are done, and the activation slot of tile q - capa once its down
    // tiles are done.
    for (int q = lag; !ended; ++q) {
      const uint64_t tw = trace_clock();
      if (q >= a.capx && !wait_geq(gu_done + ld_relaxed(xq + q - a.capx), ngu, a.err, a.spin_limit))
        return;
      if (q >= a.capa && !wait_geq(dn_done + ld_relaxed(xq + q - a.capa), ndn, a.err, a.spin_limit))
        return;
      const int mt = take_tile(q);
      if (mt < 0) return;
      if (mt >= nt) break;
      const uint64_t tb = trace_clock();
      if (a.flags & MOK_FLAG_POISON) {
        // The gather and activation slots' previous tiles are done with them (the waits
        // above); the h slot's once that tile's down items are done (a wait the gate/up items
        // otherwise make themselves, just before they store h). Poison this workgroup's rows
        // of all three before the new tile's bytes arrive.
        if (q >= a.caph &&
            !wait_geq(dn_done + ld_relaxed(xq + q - a.caph), ndn, a.err, a.spin_limit))
          return;
        const ActPlanes pl = planes(q);
        poison_rows(pl, true, q >= a.capa, q >= a.caph, a.s.H, a.s.I, MX, local * 4 + wave,
                    4 * C, lane);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
      }
      gather(q, mt, local * 4 + wave, 4 * C);
      const int b = macro_of(mt);
      trace_item(a, kTrGather, x, b, mt - s_first[b], q, tw, tb);
    }
    return;
  }

  // ---- GEMM worker: takes the XCD's items in order from its item counter ----
  const int per_tile = ngu + ndn;
  int32_t* item_ctr = a.cnt + kCntItem + x;
  __shared__ int s_it;
  for (;;) {
    if (tid == 0) s_it = add_relaxed(item_ctr, 1);
    __syncthreads();
    const int it = s_it;
    __syncthreads();
    // item -> (row tile q, column item k): k < ngu is gate/up column tile k, else down tile
    int q, k;
    if (it < lag * ngu) {
      q = it / ngu;
      k = it % ngu;
    } else {
      const int blk = (it - lag * ngu) / per_tile, off = (it - lag * ngu) % per_tile;
      const int tb = tile_of(xq, xend, blk, gmax, a.err, a.spin_limit);
      if (tb < 0) return;
      if (tb >= nt) break;                            // no down work left: done
      if (off < ngu) {
        q = blk + lag;
        k = off;
      } else {
        q = blk;
        k = off;
      }
    }
    const int mt = tile_of(xq, xend, q, gmax, a.err, a.spin_limit);
    if (mt < 0) return;
    if (mt >= nt) {
      if (q == 0) break;                              // this XCD got no row tile at all
      continue;                                       // no such row tile: nothing to do
    }
    const int b = macro_of(mt);
    const MTile tl = a.mb[b].tiles[mt - s_first[b]];
    const ActPlanes pl = planes(q);
    const uint64_t tw = trace_clock();
    if (k < ngu) {
      if (!wait_geq(landed + mt, q < lag ? nx : C, a.err, a.spin_limit)) return;
      const uint64_t tb = trace_clock();
      // h goes to h slot q % caph once the down items of the tile that used it before are
      // done (that tile is q - caph: its down items are numbered below this item)
      // (the tile id comes through tile_of: this workgroup may never have seen tile q - caph)
      const bool ok = gateup_tile<MX>(sm, a.s, a.w, pl, 0, tl.nrows, tl.e, k * 128, [&]() {
        if (q < a.caph) return true;
        const int tp = tile_of(xq, xend, q - a.caph, gmax, a.err, a.spin_limit);
        if (tp < 0) return false;
        return tp >= nt || wait_geq(dn_done + tp, ndn, a.err, a.spin_limit);
      });
      if (!ok) return;
      signal(gu_done + mt);
      trace_item(a, kTrGateUp, x, b, mt - s_first[b], it, tw, tb);
    } else {
      if (!wait_geq(gu_done + mt, ngu, a.err, a.spin_limit)) return;
      const uint64_t tb = trace_clock();
      down_tile<MX, kPushRec>(sm, a.s, a.w, pl, 0, tl.row0, tl.nrows, tl.e, (k - ngu) * kTileN,
                              a.mb[b].perm, a.mb[b].push);
      signal(dn_done + mt);
      trace_item(a, kTrDown, x, b, mt - s_first[b], it, tw, tb);
    }
  }
}

// Persistent forward kernel: the workgroup's work, then the exit protocol. The ring record the
// backward reads (which row tile each activation slot holds) is published only by the last
// workgroup to finish, and only when no workgroup reported an error: after a failed bounded
// wait the record may name tiles that were never taken, and the backward must not trust it.
template <bool MX>
__global__ __launch_bounds__(256, 1) void k_layer_fwd(FusedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GemmLds& sm = *reinterpret_cast<GemmLds*>(smem);
  layer_fwd_body<MX>(a, sm);
  // The error word is only ever written by device-scope atomics, which have completed once the
  // writer's vmcnt reaches zero; so when the exit count is full, every failure is in the word.
  // (No release is needed: the ring record's plain stores are read by later kernels.)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int done = add_relaxed(a.cnt + kCntExit, 1);
    if (done == int(gridDim.x) - 1 && ld_relaxed(a.err) == 0) {
      for (int b = 0; b < a.B; ++b) {
        a.mb[b].rhdr[kRhCapt] = a.capa;
        a.mb[b].rhdr[kRhTiles] = min(*a.mb[b].ntiles, int(a.tiles_max));
      }
    }
  }
}

template <class F>
hipError_t allow_big_lds(F* f) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kGemmLdsBytes));
}

}  // namespace

int fused_slots_per_xcd(const Layout& L) { return L.ring_capa; }

hipError_t launch_layer_fwd_macro(const Layout& L, const mok_desc& d, int B,
                                  const MacroBuffers* mb, const mok_weights& w, uint8_t* ring,
                                  uint8_t* ws, hipStream_t s) {
  if (B < 1 || B > kMaxMacro) return hipErrorInvalidValue;
  static std::atomic<bool> attr_done[kMaxDevices];
  hipError_t err = once_per_device(attr_done, [] {
    const hipError_t e = allow_big_lds(k_layer_fwd<false>);
    return e != hipSuccess ? e : allow_big_lds(k_layer_fwd<true>);
  });
  if (err != hipSuccess) return err;
  const MacroWs mw = macro_ws(L, B);
  const bool mx = L.dtype == MOK_MXFP8;
  FusedArgs a{};
  a.B = B;
  // Per macrobatch: router and schedule table (errors of earlier routers are kept). All routers
  // run first: each clears the workspace header, where macrobatch 0's tile count lives.
  for (int b = 0; b < B; ++b)
    if ((err = launch_router(L, mb[b].logits, mb[b].idx, mb[b].p, mb[b].saved, ws, s, b == 0)) !=
        hipSuccess)
      return err;
  // Then per macrobatch: tile table and push records (a token's only local pair goes straight
  // to its output row).
  for (int b = 0; b < B; ++b) {
    uint8_t* sv = mb[b].saved;
    MTile* tiles = reinterpret_cast<MTile*>(ws + mw.tiles[b]);
    int32_t* ntiles = reinterpret_cast<int32_t*>(ws + mw.ntiles[b]);
    if ((err = launch_tiles_to(L, L.M, sv, tiles, ntiles, s)) != hipSuccess) return err;
    PushRec* rec = reinterpret_cast<PushRec*>(ws + mw.push[b]);
    if ((err = launch_push_rows(L, sv, mb[b].slots, mb[b].out_seg, mb[b].p, rec, s)) != hipSuccess)
      return err;
    MacroArgs& m = a.mb[b];
    m.perm = reinterpret_cast<const int32_t*>(sv + L.sv_perm);
    m.tiles = tiles;
    m.ntiles = ntiles;
    m.x_seg = reinterpret_cast<const uint16_t* const*>(mb[b].x_seg);
    m.push = PushTarget{mb[b].slots, rec};
    m.rhdr = reinterpret_cast<int32_t*>(sv + L.sv_rhdr);
    m.rtiles = reinterpret_cast<MTile*>(sv + L.sv_rtiles);
    m.rslot = reinterpret_cast<int32_t*>(sv + L.sv_rslot);
    m.rowner = reinterpret_cast<int32_t*>(sv + L.sv_rowner);
  }
  int32_t* cnt = reinterpret_cast<int32_t*>(ws + mw.counters);
  const int64_t gmax = int64_t(B) * L.tiles_max;
  // One launch sets the counters: zero, except the per-XCD tile counts (kCntEnd, -1 until
  // known) and the per-XCD tile ids that follow the per-tile counters (-1 until taken); and no
  // tile of any macrobatch is resident in any activation slot until the kernel records it.
  {
    uint32_t* c = reinterpret_cast<uint32_t*>(cnt);
    FillRange fills[4 + kMaxMacro] = {
        {c, kCntEnd, 0u},
        {c + kCntEnd, kMaxXcd, 0xFFFFFFFFu},
        {c + kCntEnd + kMaxXcd, kCntWords - kCntEnd - kMaxXcd + 3 * gmax, 0u},
        {c + kCntWords + 3 * gmax, int64_t(kMaxXcd) * gmax, 0xFFFFFFFFu},
    };
    for (int b = 0; b < B; ++b)
      fills[4 + b] = FillRange{reinterpret_cast<uint32_t*>(a.mb[b].rowner),
                               int64_t(kXcds) * L.ring_capa, 0xFFFFFFFFu};
    if ((err = launch_fill_ranges(fills, 4 + B, s)) != hipSuccess) return err;
  }
  a.ring = ring;
  a.ring_share = L.ring_share;
  a.xsb = L.xsb;
  a.hsb = L.hsb;
  a.asb = L.asb;
  a.capx = L.ring_capx;
  a.caph = L.ring_caph;
  a.capa = L.ring_capa;
  a.s = FfnShape{L.H, L.I};
  a.w = ffn_weights(L, w);
  a.cnt = cnt;
  a.err = reinterpret_cast<int32_t*>(ws) + kWsError;
  a.tiles_max = L.tiles_max;
  const int cus = device_cus() > 0 ? device_cus() : 256;
  // Dispatch CUs: 2 per XCD for BF16 copies; 3 per XCD for MXFP8, whose dispatch workers
  // also quantise every row (measured on the Kimi-K2 MXFP8 workload: 8.92 ms with 16, 6.83 ms
  // with 24, 6.88 ms with 32, 7.13 ms with 40, 7.36 ms with 48).
  const int comm_total = d.comm_cus > 0 ? d.comm_cus : (mx ? 24 : 16);
  a.comm_per_xcd = comm_total / kMaxXcd > 0 ? comm_total / kMaxXcd : 1;
  a.K = L.K;
  a.T = L.T;
  a.dtype = L.dtype;
  a.NK = L.NK;
  a.flags = d.flags;
  if ((d.flags & MOK_FLAG_TRACE) && L.trace_max > 0) {
    a.trace = reinterpret_cast<TraceRec*>(ws + L.ws_trace);
    a.trace_max = L.trace_max;
    a.trace_count = reinterpret_cast<int32_t*>(ws) + kWsTraceCount;
  }
  a.spin_limit = (d.flags & MOK_FLAG_SKIP_ONE_SIGNAL) ? (1 << 12) : (1 << 24);
  void* args[] = {&a};
  const void* fn = mx ? reinterpret_cast<const void*>(k_layer_fwd<true>)
                      : reinterpret_cast<const void*>(k_layer_fwd<false>);
  trace_before(MOK_TRACE_FUSED_FWD, s);
  err = hipLaunchCooperativeKernel(fn, dim3(cus), dim3(kThreads), args, kGemmLdsBytes, s);
  trace_after(MOK_TRACE_FUSED_FWD, s);
  if (err != hipSuccess) return err;
  // The weighted merge of each macrobatch's tokens with several local pairs (the others' rows
  // were written by the down-GEMM epilogue).
  for (int b = 0; b < B; ++b)
    if ((err = launch_combine(L, mb[b].saved, mb[b].idx, mb[b].p, mb[b].slots, mb[b].out_seg,
                              true, s)) != hipSuccess)
      return err;
  return hipSuccess;
}

}  // namespace mok
