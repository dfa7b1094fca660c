// Backward of the MoE layer for L = sum_n <dOut[n], out[n]>.
//
// Per expert-order row r (pair n*K+k of expert e, gate p = p[n,k]), with D[r] = dOut[n]:
//   a   = D Wd_e                      (the "a" GEMM, reduction over H)
//   dp  = <a, h>                      (router-weight gradient, inside SwiGLU backward)
//   dh  = p a;  dg = dh u s(g) (1 + g (1 - s(g)));  du = dh silu(g)
//   dx  = dg Wg_e + du Wu_e           (the dx GEMM, reduction over 2I), pushed to slots[pair]
//   dWg_e = sum_r dg_r^T x_r, dWu_e = sum_r du_r^T x_r, dWd_e = sum_r (p_r D_r)^T h_r
// The pages fuse the router-weight gradient into SwiGLU backward ("Mixture-of-Kittens (MoK)",
// benchmark section; "Cursor Open-Sources Mixture-of-Kittens (MoK)", Technical Details) and
// run backward as pull reverse-combine + push reverse-dispatch (same pages, pull dispatch).
//
// GEMM operands are staged K-contiguous. BF16 weights come packed in MFMA fragment order, Wd^T
// and [Wg^T | Wu^T] included (made once per weight update, or per call into the workspace);
// MXFP8 weights come pre-quantised in the transposed blocking. Weight-gradient operands are transposed per
// expert into [feature][row] planes whose expert column ranges start at multiples of 128 and
// are zero-padded, so the weight-gradient GEMM reduces over tokens in K-stages of 64 (BF16) or
// 128 (E4M3) rows with no ragged edge. Every reduction has a fixed order.
#include "k_bwd.h"
#include "mok_rows.h"

namespace mok {
namespace {

// ---- transposes -------------------------------------------------------------------------

// Gather-transpose for the weight-gradient operands: T[f][colpad_e + i] = value of feature f of
// row off_e + i of expert e. Sources: a BF16 plane [rows][F] (with column offset), an MXFP8
// plane (dequantised), or the token segments through perm (optionally scaled by p of the
// pair: the p * D operand of dWd). Tiles of 64 padded columns x 64 features.
struct TransposeArgs {
  const int32_t* hdr;
  const int32_t* hdr2;
  const int32_t* perm;
  const float* p;              // non-null: scale rows by p[pair]
  const uint16_t* const* seg;  // non-null: rows come from segments
  const uint8_t* plane;        // else rows come from this plane
  const uint8_t* plane_s;      // MXFP8 scales of the plane (null: BF16 plane)
  int64_t plane_stride;        // elements per plane row
  int plane_col0;              // first feature column inside the plane
  // Rows of the transposed planes are packed at the padded column total `cols` (hdr2, known on
  // the device only), so the bytes in use stay contiguous whatever the host-side bound.
  uint16_t* dst;               // [F][cols] BF16 (when qdst is null)
  uint8_t* qdst;               // else MXFP8 along tokens: codes [F][cols], scales at F * ld
  int64_t ld;                  // host bound on cols (places the MXFP8 scale plane)
  int F, K, T, El;
  // Non-null (BF16 rows from segments): every source row is also copied, unscaled, to
  // rows_out[its expert-ordered row][F] (the dOut gather D of the backward, read once for both).
  uint16_t* rows_out;
  // Non-null (rows from segments, MXFP8): every source row is also quantised along the features,
  // as the dispatch gather does it (the same 32-element blocks and rule), to codes
  // rows_q[row][F] and scales rows_qs[row][F / 32]: the MXFP8 D operand of the a GEMM.
  uint8_t* rows_q;
  uint8_t* rows_qs;
  // from_act: rows are h, recomputed from the g|u of the activations, read where each row
  // lives (ActSource); h is formed as the forward formed it and then taken as the down GEMM
  // used it: rounded to BF16, or (plane_s non-null) quantised to MXFP8 along the features and
  // decoded. (The plane fields are otherwise unused.)
  int from_act;
  ActSource act;
  // store in MFMA fragment order (PackedB / PackedBMX in k_gemm.h: rows = features, K = the
  // padded columns), the layout the weight-gradient GEMMs read their B operand in
  int packed;
};

// One tile = 64 padded columns (source rows) x 128 features. Source rows are read with 16-byte
// loads (8 features per lane; 8 E4M3 codes for an MXFP8 plane) into an LDS tile
// [row][feature] whose 260-byte pitch spreads the column gathers of the store phase over
// distinct banks; the store phase writes 16 bytes (8 consecutive columns of one feature) per
// lane. Per-row source addresses, gates and MX scales are looked up once per tile.
constexpr int kTrCols = 64, kTrFeat = 128, kTrPitch = kTrFeat + 2;   // pitch in BF16 elements

__global__ __launch_bounds__(256) void k_transpose_rows(TransposeArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t t[kTrCols * kTrPitch];
  __shared__ int s_off[kMaxLocalExperts + 1], s_pad[kMaxLocalExperts + 1], s_cnt[kMaxLocalExperts];
  __shared__ const uint8_t* s_src[kTrCols];   // first byte of the row's tile features (null: zero)
  __shared__ float s_gate[kTrCols];           // p of the row's pair (scaled sources)
  __shared__ uint32_t s_sc4[kTrCols];         // MXFP8 plane: the 4 scale codes of the tile's blocks
  __shared__ int s_row[kTrCols];              // expert-ordered row of the tile's column
  const int tid = threadIdx.x;
  if (tid <= a.El) {
    s_pad[tid] = a.hdr2[kB2ColPad + tid];
    s_off[tid] = a.hdr[kHdrOffsets + tid];
    if (tid < a.El) s_cnt[tid] = a.hdr[kHdrCounts + tid];
  }
  __syncthreads();
  const int cols = s_pad[a.El];
  const int tc = cols / kTrCols, tf = a.F / kTrFeat;
  const int64_t total = int64_t(tc) * tf;
  const bool mxp = a.plane_s != nullptr;
  for (int64_t q = blockIdx.x; q < total; q += gridDim.x) {
    const int c0 = int(q / tf) * kTrCols, f0 = int(q % tf) * kTrFeat;
    if (tid < kTrCols) {
      // expert of this column tile (padding keeps tiles inside one expert)
      int e = 0;
      while (e + 1 < a.El && s_pad[e + 1] <= c0) ++e;
      const int li = c0 + tid - s_pad[e];
      const uint8_t* src = nullptr;
      float gate = 1.f;
      uint32_t sc4 = 0;
      if (li < s_cnt[e]) {
        const int64_t row = s_off[e] + li;
        if (a.seg) {
          const int32_t pair = a.perm[row];
          const int64_t n = pair / a.K;
          src = reinterpret_cast<const uint8_t*>(a.seg[n / a.T] + (n % a.T) * int64_t(a.F) + f0);
          if (a.p) gate = a.p[pair];
        } else if (a.from_act) {
          src = reinterpret_cast<const uint8_t*>(act_gu_row(a.act, row, a.act.code[row], a.F) + f0);
        } else if (mxp) {
          src = a.plane + row * a.plane_stride + a.plane_col0 + f0;
          sc4 = *reinterpret_cast<const uint32_t*>(a.plane_s + row * (a.plane_stride / 32) +
                                                   (a.plane_col0 + f0) / 32);
        } else {
          src = a.plane + (row * a.plane_stride + a.plane_col0 + f0) * 2;
        }
      }
      s_src[tid] = src;
      s_gate[tid] = gate;
      s_sc4[tid] = sc4;
      s_row[tid] = li < s_cnt[e] ? s_off[e] + li : -1;
    }
    __syncthreads();
    // load: kTrCols rows x 16 chunks of 8 features
#pragma unroll
    for (int i = 0; i < kTrCols / 16; ++i) {
      const int idx = tid + 256 * i, r = idx >> 4, ch = idx & 15;
      const uint8_t* src = s_src[r];
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      if (a.from_act) {
        // g at src, u F values further; every lane takes part (the MXFP8 block amax is a
        // 4-lane shuffle), rows without a source as zeros
        u32x4 gv = {0u, 0u, 0u, 0u}, uv = {0u, 0u, 0u, 0u};
        if (src) {
          gv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ch * 16));
          uv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + int64_t(a.F) * 2 + ch * 16));
        }
        float hv[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hv[2 * k] = swiglu_bf(bf2f(uint16_t(gv[k])), bf2f(uint16_t(uv[k])));
          hv[2 * k + 1] = swiglu_bf(bf2f(uint16_t(gv[k] >> 16)), bf2f(uint16_t(uv[k] >> 16)));
        }
        if (mxp) {
          uint32_t sc;
          const uint2 cw = mx_quant8_group4_f(hv, &sc);
          const float scale = exp2i(int(sc) - 127);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t c2 = (k < 2 ? cw.x : cw.y) >> ((k & 1) * 16);
            w[k] = pack_bf2(e4m3_value(uint8_t(c2)) * scale, e4m3_value(uint8_t(c2 >> 8)) * scale);
          }
        } else {
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = pack_bf2(hv[2 * k], hv[2 * k + 1]);
        }
      } else if (src || a.rows_q) {
        if (mxp) {
          const uint64_t c64 = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(src + ch * 8));
          const uint2 c8 = make_uint2(uint32_t(c64), uint32_t(c64 >> 32));
          const float sc = exp2i(int((s_sc4[r] >> (8 * (ch >> 2))) & 0xFFu) - 127);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t cw = k < 2 ? c8.x : c8.y;
            const int sh = (k & 1) * 16;
            w[k] = pack_bf2(e4m3_value(uint8_t(cw >> sh)) * sc, e4m3_value(uint8_t(cw >> (sh + 8))) * sc);
          }
        } else {
          const u32x4 v = src ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + ch * 16))
                              : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int k = 0; k < 4; ++k) w[k] = v[k];
          if (a.rows_out && src)
            *reinterpret_cast<u32x4*>(a.rows_out + int64_t(s_row[r]) * a.F + f0 + ch * 8) = v;
          if (a.rows_q) {
            // every lane takes part (the block amax is a 4-lane shuffle: lanes 4b .. 4b+3 of a
            // row's 16 hold its b-th block of 32 features); rows without a source store nothing
            uint32_t sc;
            const uint2 cw = mx_quant8_group4(v, &sc);
            if (src) {
              const int64_t row = s_row[r];
              *reinterpret_cast<uint2*>(a.rows_q + row * a.F + f0 + ch * 8) = cw;
              if ((ch & 3) == 0) a.rows_qs[row * (a.F / 32) + (f0 + ch * 8) / 32] = uint8_t(sc);
            }
          }
          if (a.p && !a.qdst) {   // BF16 operand; MXFP8 applies the gate in fp32 below
            const float g = s_gate[r];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              w[k] = pack_bf2(bf2f(uint16_t(w[k])) * g, bf2f(uint16_t(w[k] >> 16)) * g);
          }
        }
      }
      uint32_t* dst = reinterpret_cast<uint32_t*>(t + r * kTrPitch + ch * 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[k] = w[k];
    }
    __syncthreads();
    // store: 128 features x kTrCols/8 chunks of 8 columns (runs of 2 * kTrCols bytes per row)
#pragma unroll
    for (int i = 0; i < kTrCols / 16; ++i) {
      const int idx = tid + 256 * i, f = idx / (kTrCols / 8), cc = idx % (kTrCols / 8);
      u32x4 out;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        out[k] = uint32_t(t[(cc * 8 + 2 * k) * kTrPitch + f]) |
                 (uint32_t(t[(cc * 8 + 2 * k + 1) * kTrPitch + f]) << 16);
      if (a.qdst) {
        // blocks of 32 padded columns (4 lanes); expert ranges start at multiples of 128. A
        // gated operand (p * D) is formed in fp32 and quantised from there.
        float fv[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          fv[2 * k] = bf2f(uint16_t(out[k]));
          fv[2 * k + 1] = bf2f(uint16_t(out[k] >> 16));
        }
        if (a.p) {
#pragma unroll
          for (int k = 0; k < 8; ++k) fv[k] *= s_gate[cc * 8 + k];
        }
        uint32_t sc;
        const uint2 codes = mx_quant8_group4_f(fv, &sc);
        const int fa = f0 + f, col = c0 + cc * 8;
        uint8_t* qs = a.qdst + int64_t(a.F) * a.ld;   // the scale plane
        if (a.packed) {
          // fragment (feature/32, column/64): half (column%64)/32, lane feature%32 + 32 *
          // ((column%32)/16), byte column%16; the block's scale is byte feature%32 + 32 *
          // ((column/32)%2) of the fragment's 64 scale bytes
          const int64_t frag = int64_t(fa >> 5) * (cols >> 6) + (col >> 6);
          const int q = col & 63;
          *reinterpret_cast<uint2*>(a.qdst + (frag * 2 + (q >> 5)) * 1024 +
                                    ((fa & 31) + 32 * ((q >> 4) & 1)) * 16 + (q & 15)) = codes;
          if ((cc & 3) == 0) qs[frag * 64 + (fa & 31) + 32 * ((q >> 5) & 1)] = uint8_t(sc);
        } else {
          *reinterpret_cast<uint2*>(a.qdst + int64_t(fa) * cols + col) = codes;
          if ((cc & 3) == 0) qs[int64_t(fa) * (cols / 32) + col / 32] = uint8_t(sc);
        }
      } else if (a.packed) {
        // 8 columns of one feature are one lane's 16 bytes of fragment (feature/32, column/16)
        const int fa = f0 + f, col = c0 + cc * 8;
        const int64_t frag = int64_t(fa >> 5) * (cols >> 4) + (col >> 4);
        *reinterpret_cast<u32x4*>(a.dst + (frag * 64 + (fa & 31) + 32 * ((col >> 3) & 1)) * 8) = out;
      } else {
        *reinterpret_cast<u32x4*>(a.dst + int64_t(f0 + f) * cols + c0 + cc * 8) = out;
      }
    }
    __syncthreads();
  }
}

// ---- reverse ring walk: reuse what the forward left resident, replay the rest -------------

// Backward set-up, one wave, no host synchronisation:
//  - split the forward's tiles into those whose ring slot still holds them (their g|u and h are
//    read in place) and those to replay (X gathered again, gate/up recomputed), both in forward
//    tile order (ballot compaction, so the lists are deterministic); without ring state (staged
//    forward, or no ring passed) every row is replayed, in per-expert tiles;
//  - the backward GEMMs' tile table: per-expert tiles of at most kTileM rows (no minibatch cuts);
//  - the padded column layout of the per-expert transposed planes: expert e's rows go to
//    columns [colpad[e], colpad[e] + count[e]), colpad[e] a multiple of kPadRows, the rest of its
//    rounded-up range zero; hdr2[kB2RowsPad] = total padded columns;
//  - zeroed work-queue counters of the two GEMM launches, and a cleared error word.
// El <= 64, so lane e owns expert e. The ring record is used only if it is whole: its slot
// count matches this ring, and every recorded tile has a slot of this ring and lies inside its
// expert's rows; otherwise every row is replayed (the result is the same either way).
__global__ __launch_bounds__(64) void k_bwd_plan(const int32_t* hdr, const int32_t* rhdr,
                                                 const MTile* rtiles, const int32_t* rslot,
                                                 const int32_t* rowner, int have_ring, int capa,
                                                 MTile* restore, int32_t* restore_slot,
                                                 MTile* replay, int32_t* counts, MTile* tiles,
                                                 int32_t* ntiles, int32_t* hdr2, int El,
                                                 int64_t tiles_max, int32_t* err) {
  const int lane = threadIdx.x;
  // the backward's own error word (its workspace is not the forward's)
  if (lane == 0) *err = 0;
  const uint64_t lt = (1ull << lane) - 1;
  // per-expert rows and tile counts, exclusive prefix over experts (lanes)
  const int off = lane < El ? hdr[kHdrOffsets + lane] : 0;
  const int cnt = lane < El ? hdr[kHdrCounts + lane] : 0;
  const int nt_e = (cnt + kTileM - 1) / kTileM;
  const int pad_e = (cnt + kPadRows - 1) / kPadRows * kPadRows;
  int t_ex = nt_e, p_ex = pad_e;                       // inclusive scans, then made exclusive
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int a = __shfl_up(t_ex, d, 64), b = __shfl_up(p_ex, d, 64);
    if (lane >= d) {
      t_ex += a;
      p_ex += b;
    }
  }
  const int t_tot = __shfl(t_ex, 63, 64), p_tot = __shfl(p_ex, 63, 64);
  t_ex -= nt_e;
  p_ex -= pad_e;
  // the forward's ring record, validated
  int nt = have_ring ? rhdr[kRhTiles] : 0;
  if (nt < 0 || nt > tiles_max || (nt > 0 && rhdr[kRhCapt] != capa)) nt = 0;
  {
    const int nslots = kXcds * capa;
    bool bad = false;
    for (int base = 0; base < nt; base += 64) {
      const int mt = base + lane;
      MTile t{0, 0, 0, 0};
      int sl = 0;
      if (mt < nt) {
        t = rtiles[mt];
        sl = rslot[mt];
      }
      // (every lane takes part in the shuffles)
      const bool eok = t.e >= 0 && t.e < El;
      const int eo = __shfl(off, eok ? t.e : 0, 64), ec = __shfl(cnt, eok ? t.e : 0, 64);
      const bool ok = mt >= nt || (eok && sl >= 0 && sl < nslots && t.nrows >= 1 &&
                                   t.nrows <= kTileM && t.row0 >= eo && t.row0 + t.nrows <= eo + ec);
      bad = bad || __ballot(!ok) != 0;
    }
    if (bad) nt = 0;
  }
  // per-expert tiles: the GEMM tile table, and the replay list when there is no ring state
  if (lane < El) {
    for (int q = 0; q < nt_e && t_ex + q < tiles_max; ++q) {
      const MTile t{0, lane, off + q * kTileM, min(kTileM, cnt - q * kTileM)};
      tiles[t_ex + q] = t;
      if (nt <= 0) replay[t_ex + q] = t;
    }
    hdr2[kB2ColPad + lane] = p_ex;
  }
  // forward tiles -> restore / replay lists in tile order
  int64_t nr = 0, np = 0;
  if (nt > 0) {
    for (int base = 0; base < nt && base < tiles_max; base += 64) {
      const int mt = base + lane;
      const bool valid = mt < nt && mt < tiles_max;
      MTile t{0, 0, 0, 0};
      int sl = 0;
      bool res = false;
      if (valid) {
        t = rtiles[mt];
        sl = rslot[mt];
        res = rowner[sl] == mt;
      }
      const uint64_t bres = __ballot(valid && res), brep = __ballot(valid && !res);
      if (valid && res) {
        const int64_t i = nr + __popcll(bres & lt);
        restore[i] = t;
        restore_slot[i] = sl;
      }
      if (valid && !res) replay[np + __popcll(brep & lt)] = t;
      nr += __popcll(bres);
      np += __popcll(brep);
    }
  } else {
    np = min(int64_t(t_tot), tiles_max);
  }
  if (lane == 0) {
    counts[0] = int32_t(nr);
    counts[1] = int32_t(np);
    *ntiles = int32_t(min(int64_t(t_tot), tiles_max));
    hdr2[kB2ColPad + El] = p_tot;
    hdr2[kB2RowsPad] = p_tot;
  }
  if (lane < 2 * kXcds) counts[4 + lane] = 0;          // the two GEMM launches' queue counters
}

// Work item = 16 rows of one listed tile. Every row gets its row-source code: restored tiles
// point at their ring slot (their g|u and h are read there, not copied); replayed rows get -1
// (the replay writes them to the activation planes) and their X is gathered from its segment
// into the dispatch plane (MXFP8: quantised along H). One wave per row.
struct StageArgs {
  const MTile* restore;
  const int32_t* restore_slot;
  const MTile* replay;
  const int32_t* counts;
  const int32_t* perm;
  const uint16_t* const* x_seg;
  uint8_t* xd;          // dispatch plane [rows_max] (codes then scales in MXFP8)
  int32_t* code;        // [rows_max] row-source codes (ActSource), written here
  int64_t rows_max;
  int H, I, K, T, dtype;
  int64_t NK;
};

__global__ __launch_bounds__(256) void k_bwd_stage(StageArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nr = a.counts[0], np = a.counts[1];
  const int64_t items = int64_t(nr + np) * (kTileM / 16);
  const bool mx = a.dtype == MOK_MXFP8;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int t = int(it / (kTileM / 16)), chunk = int(it % (kTileM / 16));
    const bool rest = t < nr;
    const MTile tl = rest ? a.restore[t] : a.replay[t - nr];
    if (threadIdx.x < 16 && chunk * 16 + int(threadIdx.x) < tl.nrows) {
      const int i = chunk * 16 + int(threadIdx.x);
      a.code[tl.row0 + i] = rest ? ((a.restore_slot[t] << 8) | i) : -1;
    }
    if (rest) continue;
    if (mx && a.H <= 8 * kRowBatchChunks) {
      // MXFP8 replay gather: the wave's rows i0, i0 + 4, ... quantised with the next row's
      // loads in flight; lane j looks up the source of the wave's j-th row.
      const int i0 = chunk * 16 + wave, iend = min(tl.nrows, chunk * 16 + 16);
      const int nrw = i0 < iend ? (iend - i0 + 3) / 4 : 0;
      const uint16_t* my_src = nullptr;
      if (lane < nrw) {
        const int32_t pair = a.perm[tl.row0 + i0 + 4 * lane];
        if (pair >= 0 && pair < a.NK) {
          const int64_t n = pair / a.K;
          my_src = a.x_seg[n / a.T] + (n % a.T) * int64_t(a.H);
        }
      }
      const uint64_t sp = reinterpret_cast<uint64_t>(my_src);
      quant_rows_mx_2(
          nrw, a.H, lane,
          [&](int j) {
            const uint32_t lo = __shfl(uint32_t(sp), j, 64), hi = __shfl(uint32_t(sp >> 32), j, 64);
            return reinterpret_cast<const uint16_t*>((uint64_t(hi) << 32) | lo);
          },
          [&](int j) { return a.xd + (tl.row0 + i0 + 4 * j) * int64_t(a.H); },
          [&](int j) { return a.xd + a.rows_max * a.H + (tl.row0 + i0 + 4 * j) * int64_t(a.H / 32); });
      continue;
    }
    for (int i = chunk * 16 + wave; i < min(tl.nrows, chunk * 16 + 16); i += 4) {
      const int64_t row = tl.row0 + i;
      const int32_t pair = a.perm[row];
      const uint16_t* src = nullptr;
      if (pair >= 0 && pair < a.NK) {
        const int64_t n = pair / a.K;
        src = a.x_seg[n / a.T] + (n % a.T) * int64_t(a.H);
      }
      if (mx) quant_row_mx(src, a.xd + row * a.H, a.xd + a.rows_max * a.H + row * (a.H / 32), a.H, lane);
      else copy_row_bf16(src, reinterpret_cast<uint16_t*>(a.xd) + row * a.H, a.H, lane);
    }
  }
}

// ---- backward GEMM kernels ------------------------------------------------------------------

struct WJob {
  const uint8_t* t_a;      // [Fa][ld] BF16 or codes (rows = output rows)
  const uint8_t* t_a_s;    // MXFP8 scales [Fa][ld/32]
  const uint8_t* t_b;      // [Fb][ld]
  const uint8_t* t_b_s;
  int Fa, Fb;              // output rows, output columns
  float* dw;               // [El][Fa][Fb]
};

struct BwdArgs {
  const MTile* tiles;
  const int32_t* ntiles;
  const int32_t* hdr;      // schedule header (expert offsets)
  const int32_t* perm;
  const float* p;
  const int32_t* hdr2;
  FfnShape s;
  // a GEMM
  const uint8_t* d;        // D rows: BF16 [rows][H] or codes
  const uint8_t* d_s;      // MXFP8 scales [rows][H/32]
  const uint8_t* wdt;      // packed Wd^T plane [El][I rows][H] (BF16 values or E4M3 codes)
  const uint8_t* wdt_s;    // MXFP8: its scales
  ActSource act;           // g|u and h of the forward (ring slot or replayed plane, per row)
  uint16_t* dgu;           // out: dg|du BF16 [rows][2I] (BF16 mode)
  uint8_t* q_dgt;          // out (MXFP8): dg^T, du^T blocked along tokens, codes then scales
  uint8_t* q_dut;
  float* dp_part;          // out: [rows][I/256]
  // dx GEMM
  const uint8_t* dgu_a;    // dg|du as the dx GEMM reads it: BF16 or codes [rows][2I]
  const uint8_t* dgu_s;    // MXFP8 scales [rows][2I/32]
  const uint8_t* wgt;      // packed [Wg^T | Wu^T] plane [El][H rows][2I]
  const uint8_t* wgt_s;    // MXFP8: its scales
  PushTarget push;         // dx rows: pair slots, or dX of a token's only local pair
  // weight gradients: up to three jobs dW[e] = Ta[:, cols of e] . Tb[:, cols of e]^T
  WJob jobs[3];
  int njobs;
  int El;
  int64_t ld;              // host bound on the padded columns (places the MXFP8 scale planes;
                           // rows are packed at the device-side total hdr2[kB2RowsPad])
  int32_t* queue;          // [kXcds] work counters of one launch (zeroed before it)
};

// The backward's GEMM work in two persistent launches with no dependencies inside either:
//   phase 0: the a GEMM (with dp / SwiGLU backward) and dWd = (p D)^T h;
//   phase 1: the dx GEMM (pushed to the slots) and dWg = dg^T X, dWu = du^T X.
// Mixing two kinds of tiles fills the last wave of the first kind. Items are numbered primary
// tiles first (the heavier ones), then weight-gradient tiles; blocks of kQBlock consecutive item
// slots belong to the XCDs in turn (consecutive tiles share operands in that XCD's L2). In
// phase 0 slot i is item i; in phase 1 the two kinds' blocks alternate (interleaved_item). A
// workgroup takes slots from its own XCD's counter, then from the others' until all are done.
// Which workgroup computes an item does not change the item's result.
constexpr int kQBlock = 32;

__device__ __forceinline__ int bwd_xcc_id() {
  return __builtin_amdgcn_s_getreg(20 | (0 << 6) | ((4 - 1) << 11)) & (kXcds - 1);   // HW_REG_XCC_ID
}

constexpr int kItemHole = -2;

// Phase 1 item order: item slot i -> work item, with blocks of kQBlock slots alternating
// between dx tiles (items 0 .. n_p-1) and weight-gradient tiles (n_p .. total-1), so that the
// fp32 gradient stores are spread over the launch instead of all coming at its end (measured
// 1-2 % faster; in phase 0 the same order was slower, so phase 0 keeps its primary tiles
// first). The dx surplus blocks come first, the weight-gradient surplus last. Slots past a
// kind's last item are holes (kItemHole); slots past every block give -1.
__device__ __forceinline__ int interleaved_item(int i, int n_p, int total) {
  const int nbp = (n_p + kQBlock - 1) / kQBlock, nbw = (total - n_p + kQBlock - 1) / kQBlock;
  if (i >= (nbp + nbw) * kQBlock) return -1;
  const int mn = min(nbp, nbw), ep = max(0, nbp - nbw);
  const int b = i / kQBlock, o = i % kQBlock;
  bool primary;
  int kb;
  if (b < ep) {
    primary = true;
    kb = b;
  } else if (b < ep + 2 * mn) {
    const int j = b - ep;
    primary = (j & 1) == 0;
    kb = (primary ? ep : 0) + (j >> 1);
  } else {
    primary = false;
    kb = mn + (b - ep - 2 * mn);
  }
  const int t = kb * kQBlock + o;
  if (primary) return t < n_p ? t : kItemHole;
  return n_p + t < total ? n_p + t : kItemHole;
}

template <bool MX, int PHASE>
__global__ __launch_bounds__(256, 1) void k_bwd_gemms(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GemmLds& sm = *reinterpret_cast<GemmLds*>(smem);
  __shared__ int s_item;
  const int mtiles = *a.ntiles;
  const int ntn = int(PHASE == 0 ? cdiv(a.s.I, kTileN) : cdiv(a.s.H, kTileN));
  const int n_p = mtiles * ntn;
  int total = n_p;
  for (int j = 0; j < a.njobs; ++j)
    total += a.El * ((a.jobs[j].Fa + kTileM - 1) / kTileM) * ((a.jobs[j].Fb + kTileN - 1) / kTileN);
  const int x0 = bwd_xcc_id();
  for (int probe = 0; probe < kXcds; ++probe) {
    const int x = (x0 + probe) & (kXcds - 1);
    for (;;) {
      if (threadIdx.x == 0) {
        const int k = add_relaxed(a.queue + x, 1);
        const int i = ((k / kQBlock) * kXcds + x) * kQBlock + k % kQBlock;
        s_item = PHASE == 1 ? interleaved_item(i, n_p, total) : (i < total ? i : -1);
      }
      __syncthreads();
      const int t = s_item;
      __syncthreads();
      if (t == kItemHole) continue;
      if (t < 0) break;
      if (t < n_p) {
        int mt, nt;
        tile_coords(t, mtiles, ntn, mt, nt);
        const MTile tl = a.tiles[mt];
        if (PHASE == 0) {
          TokQuant tq{};
          if (MX) {
            // token column of the tile's first row in the per-expert padded planes
            const int rel = tl.row0 - a.hdr[kHdrOffsets + tl.e];
            const int cp = a.hdr2[kB2ColPad + tl.e];
            tq = TokQuant{a.q_dgt, a.q_dut, a.ld, a.hdr2[kB2RowsPad], int64_t(cp) + rel,
                          a.hdr2[kB2ColPad + tl.e + 1] - cp - rel};
          }
          a_tile<MX>(sm, a.s, tl.row0, tl.nrows, tl.e, nt * kTileN, a.d, a.d_s, a.wdt, a.wdt_s,
                     a.act, a.perm, a.p, a.dgu, const_cast<uint8_t*>(a.dgu_a),
                     const_cast<uint8_t*>(a.dgu_s), tq, a.dp_part);
        } else
          dx_tile<MX>(sm, a.s, tl.row0, tl.nrows, tl.e, nt * kTileN, a.dgu_a, a.dgu_s, a.wgt,
                      a.wgt_s, a.push);
      } else {
        int j = 0, rem = t - n_p;
        for (; j < a.njobs; ++j) {
          const int per = a.El * ((a.jobs[j].Fa + kTileM - 1) / kTileM) * ((a.jobs[j].Fb + kTileN - 1) / kTileN);
          if (rem < per) break;
          rem -= per;
        }
        const WJob& jb = a.jobs[j];
        const int mtn = (jb.Fa + kTileM - 1) / kTileM, ntw = (jb.Fb + kTileN - 1) / kTileN;
        const int e = rem / (mtn * ntw);
        int mt, nt;
        tile_coords(rem % (mtn * ntw), mtn, ntw, mt, nt);
        const int c0 = a.hdr2[kB2ColPad + e];
        const int ncols = a.hdr2[kB2ColPad + e + 1] - c0;
        wgrad_tile<MX>(sm, jb.t_a, jb.t_a_s, jb.t_b, jb.t_b_s, a.hdr2[kB2RowsPad], c0, ncols, mt * kTileM,
                       nt * kTileN, jb.Fa, jb.Fb, jb.dw + int64_t(e) * jb.Fa * jb.Fb);
      }
    }
  }
}

// dp[pair] = sum of the I/256 partials of its row, in column-tile order; then, when every
// expert is local, dlogits[n, idx_k] = p_k (dp_k - sum_j p_j dp_j).
__global__ void k_dp_finalize(const int32_t* hdr, const int32_t* perm, const float* dp_part,
                              int nparts, float* dp, int64_t rows_max) {
  const int64_t rows = min(int64_t(hdr[kHdrRows]), rows_max);
  for (int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; r < rows;
       r += int64_t(gridDim.x) * blockDim.x) {
    const int32_t pair = perm[r];
    if (pair < 0) continue;
    float s = 0.f;
    for (int q = 0; q < nparts; ++q) s += dp_part[r * nparts + q];
    dp[pair] = s;
  }
}

__global__ void k_dlogits(const int32_t* idx, const float* p, const float* dp, float* dl,
                          int64_t N, int K, int E) {
  for (int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; n < N;
       n += int64_t(gridDim.x) * blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < K; ++k) s = fmaf(p[n * K + k], dp[n * K + k], s);
    for (int e = 0; e < E; ++e) dl[n * E + e] = 0.f;
    for (int k = 0; k < K; ++k) dl[n * E + idx[n * K + k]] = p[n * K + k] * (dp[n * K + k] - s);
  }
}

template <class F>
hipError_t allow_big_lds(F* f) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kGemmLdsBytes));
}

int grid_cap(int64_t items, int cap) {
  return int(items < 1 ? 1 : (items > cap ? cap : items));
}

}  // namespace

hipError_t launch_backward(const Layout& L, const BwdBuffers& b, hipStream_t s) {
  static std::atomic<bool> attr_done[kMaxDevices];
  hipError_t err = once_per_device(attr_done, [] {
    hipError_t e;
    if ((e = allow_big_lds(k_bwd_gemms<false, 0>)) != hipSuccess) return e;
    if ((e = allow_big_lds(k_bwd_gemms<true, 0>)) != hipSuccess) return e;
    if ((e = allow_big_lds(k_bwd_gemms<false, 1>)) != hipSuccess) return e;
    return allow_big_lds(k_bwd_gemms<true, 1>);
  });
  if (err != hipSuccess) return err;
  const bool mx = L.dtype == MOK_MXFP8;
  const int G = device_cus() > 0 ? device_cus() : 256;
  const int H = L.H, I = L.I, El = L.El;
  const int32_t* hdr = reinterpret_cast<const int32_t*>(b.saved);
  const int32_t* perm = reinterpret_cast<const int32_t*>(b.saved + L.sv_perm);

  // 1. reverse ring walk: tiles still resident in the ring give back their g|u and h; the
  //    others are replayed (X gathered again, gate/up recomputed by the same tile code, so the
  //    values are bit-identical either way)
  MTile* restore = reinterpret_cast<MTile*>(b.ws + L.b_restore);
  MTile* replay = reinterpret_cast<MTile*>(b.ws + L.b_replay);
  int32_t* rsl = reinterpret_cast<int32_t*>(b.ws + L.b_rsl);
  int32_t* counts = reinterpret_cast<int32_t*>(b.ws + L.b_counts);
  hipLaunchKernelGGL(k_bwd_plan, dim3(1), dim3(64), 0, s, hdr,
                     reinterpret_cast<const int32_t*>(b.saved + L.sv_rhdr),
                     reinterpret_cast<const MTile*>(b.saved + L.sv_rtiles),
                     reinterpret_cast<const int32_t*>(b.saved + L.sv_rslot),
                     reinterpret_cast<const int32_t*>(b.saved + L.sv_rowner),
                     int(b.ring != nullptr && L.ring_capa > 0), L.ring_capa, restore, rsl,
                     replay, counts,
                     reinterpret_cast<MTile*>(b.ws + L.ws_tiles),
                     reinterpret_cast<int32_t*>(b.ws) + kWsNumTiles, b.hdr2, El, L.tiles_max,
                     reinterpret_cast<int32_t*>(b.ws) + kWsError);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  {
    StageArgs st{};
    st.restore = restore;
    st.restore_slot = rsl;
    st.replay = replay;
    st.counts = counts;
    st.perm = perm;
    st.x_seg = reinterpret_cast<const uint16_t* const*>(b.x_seg);
    st.xd = b.xd;
    st.code = b.actsrc;
    st.rows_max = L.rows_max;
    st.H = H; st.I = I; st.K = L.K; st.T = L.T; st.dtype = L.dtype;
    st.NK = L.NK;
    hipLaunchKernelGGL(k_bwd_stage, dim3(grid_cap(L.tiles_max * (kTileM / 16), 4 * G)), dim3(256), 0, s, st);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if ((err = launch_ffn_gateup_list(L, b.saved, b.xd, b.w, b.act, replay, counts + 1, s)) != hipSuccess)
    return err;
  // 2. pull reverse-combine: D[r] = dOut[n(r)] (BF16; MXFP8 quantised along H for the a GEMM
  //    as the forward dispatch quantises X), written by the (p D)^T gather-transpose below,
  //    which reads the same rows
  // 3. the backward GEMMs read packed Wd^T and [Wg^T | Wu^T] (b.w.packed: the caller's, or
  //    packed by the host entry point into the workspace)
  const PackOffsets po = pack_offsets(El, H, I, L.dtype);
  const uint8_t* packed = static_cast<const uint8_t*>(b.w.packed);
  // 4. weight-gradient operand planes that do not need dg|du: per-expert column ranges, X^T,
  //    (p D)^T and h^T (MXFP8: quantised along tokens as they are written)
  const uint16_t* const* xs = reinterpret_cast<const uint16_t* const*>(b.x_seg);
  const uint16_t* const* ds = reinterpret_cast<const uint16_t* const*>(b.dout_seg);
  const int64_t ld = L.rp_max;
  // where the backward reads each row's g|u and h (ring slot or replayed plane)
  const ActPlanes ap = act_planes(b.act, L.rows_max, H, I, L.dtype, false);
  ActSource asrc{};
  asrc.act = ap;
  asrc.ring = b.ring;
  asrc.ring_share = L.ring_share;
  asrc.aofs = int64_t(L.ring_capx) * L.xsb + int64_t(L.ring_caph) * L.hsb;
  asrc.asb = L.asb;
  asrc.capa = L.ring_capa > 0 ? L.ring_capa : 1;
  asrc.code = b.actsrc;
  auto tr = [&](const uint16_t* const* seg, const float* p, const uint8_t* plane, const uint8_t* plane_s,
                int64_t stride, int col0, int F, uint16_t* dst, uint8_t* qdst,
                uint16_t* rows_out = nullptr, bool from_act = false, bool packed = false,
                uint8_t* rows_q = nullptr) {
    TransposeArgs t{hdr, b.hdr2, perm, p, seg, plane, plane_s, stride, col0, dst, mx ? qdst : nullptr,
                    ld, F, L.K, L.T, El, rows_out, rows_q,
                    rows_q ? rows_q + L.rows_max * int64_t(F) : nullptr, int(from_act), asrc,
                    int(packed)};
    hipLaunchKernelGGL(k_transpose_rows, dim3(grid_cap(ld / kTrCols * (F / kTrFeat), 8192)), dim3(256), 0, s, t);
  };
  // (X^T and h^T are the B operands of the weight-gradient GEMMs: stored packed)
  tr(xs, nullptr, nullptr, nullptr, 0, 0, H, b.xt, b.q_xt, nullptr, false, true);   // X^T
  tr(ds, b.topk_p, nullptr, nullptr, 0, 0, H, b.dt, b.q_dt,
     mx ? nullptr : reinterpret_cast<uint16_t*>(b.d), false, false,
     mx ? b.dq : nullptr);                                                           // (p D)^T (+ D)
  tr(nullptr, nullptr, ap.h, mx ? ap.hs : nullptr, I, 0, I, b.ht, b.q_ht, nullptr, true,
     true);                                                                         // h^T
  if ((err = hipGetLastError()) != hipSuccess) return err;

  BwdArgs a{};
  a.tiles = reinterpret_cast<const MTile*>(b.ws + L.ws_tiles);
  a.ntiles = reinterpret_cast<const int32_t*>(b.ws) + kWsNumTiles;
  a.hdr = hdr;
  a.perm = perm;
  a.q_dgt = b.q_dgt;
  a.q_dut = b.q_dut;
  a.p = b.topk_p;
  a.hdr2 = b.hdr2;
  a.s = FfnShape{H, I};
  a.d = mx ? b.dq : b.d;
  a.d_s = mx ? b.dq + L.rows_max * H : nullptr;
  a.wdt = packed + po.wdt;
  a.wdt_s = mx ? packed + po.wdt_s : nullptr;
  a.act = asrc;
  a.dgu = b.dgu;
  a.dp_part = b.dp_part;
  a.dgu_a = mx ? b.dguq : reinterpret_cast<const uint8_t*>(b.dgu);
  a.dgu_s = mx ? b.dguq + L.rows_max * 2 * I : nullptr;
  a.wgt = packed + po.dx;
  a.wgt_s = mx ? packed + po.dx_s : nullptr;
  a.push = PushTarget{b.slots, b.push};
  a.ld = ld;
  a.El = El;
  a.queue = counts + 4;
  auto job = [&](WJob& o, const uint16_t* ta, const uint16_t* tb, uint8_t* qa, uint8_t* qb, int Fa,
                 int Fb, float* dw) {
    o.Fa = Fa;
    o.Fb = Fb;
    o.dw = dw;
    if (mx) {
      o.t_a = qa; o.t_a_s = qa + int64_t(Fa) * ld;
      o.t_b = qb; o.t_b_s = qb + int64_t(Fb) * ld;
    } else {
      o.t_a = reinterpret_cast<const uint8_t*>(ta); o.t_a_s = nullptr;
      o.t_b = reinterpret_cast<const uint8_t*>(tb); o.t_b_s = nullptr;
    }
  };
  // 5. phase 0: a GEMM with fused dp / SwiGLU backward, and dWd
  a.njobs = 1;
  job(a.jobs[0], b.dt, b.ht, b.q_dt, b.q_ht, H, I, b.g.dwd);
  trace_before(MOK_TRACE_BWD_GEMM1, s);
  if (mx) hipLaunchKernelGGL((k_bwd_gemms<true, 0>), dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  else hipLaunchKernelGGL((k_bwd_gemms<false, 0>), dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  trace_after(MOK_TRACE_BWD_GEMM1, s);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 6. dg^T, du^T (BF16; the MXFP8 a-GEMM epilogue wrote them, quantised along tokens from
  //    fp32); phase 1: dx GEMM pushed to the slots (a token's only local pair straight to its
  //    dX row), dWg and dWu
  if ((err = launch_push_rows(L, b.saved, b.slots, b.dx_seg, nullptr, b.push, s)) != hipSuccess)
    return err;
  if (!mx) {
    const uint8_t* dgu8 = reinterpret_cast<const uint8_t*>(b.dgu);
    tr(nullptr, nullptr, dgu8, nullptr, 2 * I, 0, I, b.dgt, nullptr);                 // dg^T
    tr(nullptr, nullptr, dgu8, nullptr, 2 * I, I, I, b.dut, nullptr);                 // du^T
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  a.njobs = 2;
  job(a.jobs[0], b.dgt, b.xt, b.q_dgt, b.q_xt, I, H, b.g.dwg);
  job(a.jobs[1], b.dut, b.xt, b.q_dut, b.q_xt, I, H, b.g.dwu);
  a.queue = counts + 4 + kXcds;
  trace_before(MOK_TRACE_BWD_GEMM2, s);
  if (mx) hipLaunchKernelGGL((k_bwd_gemms<true, 1>), dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  else hipLaunchKernelGGL((k_bwd_gemms<false, 1>), dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  trace_after(MOK_TRACE_BWD_GEMM2, s);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  // 7. the unweighted fixed-order dX merge, the router-weight gradient per pair, and dlogits
  //    when every expert is local
  if ((err = launch_combine(L, b.saved, b.topk_idx, nullptr, b.slots, b.dx_seg, true, s)) != hipSuccess)
    return err;
  hipLaunchKernelGGL(k_dp_finalize, dim3(grid_cap(L.rows_max / 256 + 1, 4096)), dim3(256), 0, s,
                     hdr, perm, b.dp_part, int(cdiv(I, kTileN)), b.dp, L.rows_max);
  if (b.dlogits)
    hipLaunchKernelGGL(k_dlogits, dim3(grid_cap(L.N / 256 + 1, 4096)), dim3(256), 0, s, b.topk_idx,
                       b.topk_p, b.dp, b.dlogits, L.N, L.K, L.E);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  return hipSuccess;
}

}  // namespace mok
