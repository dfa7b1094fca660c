// Internal definitions shared by the host code and the kernels of libmok (not part of the
// ABI). Buffer layouts are computed here once, from host-known bounds only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/mok.h"

namespace mok {

// ---- fixed kernel geometry -------------------------------------------------------------
constexpr int kTileM = 256;         // GEMM tile rows (tokens)
constexpr int kTileN = 256;         // GEMM tile columns
constexpr int kThreads = 256;       // threads per GEMM workgroup (4 waves, 2 x 2)
constexpr int kTopkTokensPerBlock = 256;
constexpr int kMaxLocalExperts = 64;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kXcds = 8;            // XCDs per MI355X device (each with its own L2)
constexpr int kRingXSlots = 3;      // gather slots per XCD share of the fused-forward ring
constexpr int kRingHSlots = 3;      // h slots per XCD share (more than the forward's lag of 2)
constexpr int kMaxMacro = 8;        // macrobatches (layer calls) one fused launch can run

__host__ __device__ inline int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Marks a token's only local pair: set in the rank words the router passes to k_place and in
// the push codes (pair id | flag) it writes per row. Ranks and pair ids stay below it
// (N*K < 2^30).
constexpr int32_t kSoleFlag = 1 << 30;

// Where the push epilogue of the down GEMM or the dx GEMM sends one expert-ordered row (one
// 16-byte load per row): w < 0: the raw BF16 row to dst (the pair's slot); else dst is the
// token's own output row and receives bf16(w * float(bf16 row)), the merge over one term, for
// a token whose only local pair this is.
struct alignas(16) PushRec {
  uint16_t* dst;
  float w;
  int32_t pad;
};

// One phase-trace record (MOK_FLAG_TRACE): which workgroup ran which item of which row tile, and
// when (s_memrealtime ticks, a 100 MHz clock): t_wait when it started waiting for the item's
// inputs, t_begin when they were there, t_end when its results were signalled.
enum TraceKind : int { kTrPrologueGather = 1, kTrGather = 2, kTrGateUp = 3, kTrDown = 4 };
struct TraceRec {
  int32_t wg;        // workgroup (blockIdx.x)
  int32_t info;      // kind | xcd << 8 | macrobatch << 16
  int32_t tile;      // row tile within its macrobatch
  int32_t item;      // the XCD's item number (GEMM items), or its row-tile index (gathers)
  uint64_t t_wait, t_begin, t_end, pad;
};

// ---- saved (schedule table) header, int32 words ----------------------------------------
enum SavedHeader : int {
  kHdrP = 0,        // local pairs
  kHdrRows = 1,     // expert-order rows (P + per-expert padding in MXFP8 mode)
  kHdrU = 2,        // touched tokens
  kHdrUm = 3,       // touched tokens with more than one local pair
  kHdrStatus = 4,   // copy of the router's device-side status (0 if its scan finished)
  kHdrCounts = 16,  // [E_loc]
  kHdrOffsets = 96, // [E_loc + 1]
  kHdrWords = 192,
};

// ---- ws header, int32 words ------------------------------------------------------------
enum WsHeader : int {
  kWsError = 0,     // mok_status of the first device-side failure, 0 if none
  kWsTicket = 1,    // dynamic block id for the router's single-pass scan
  kWsNumTiles = 2,  // m-tiles in the tile table
  kWsTraceCount = 3,  // phase-trace records written (MOK_FLAG_TRACE)
  kWsWords = 64,
};

// Ring state left in `saved` by the fused forward for the backward: the forward's tile table,
// the ring slot of every tile (x * capt + slot), and the last tile written to every slot.
enum RingHeader : int {
  kRhTiles = 0,     // forward tiles (0: the ring holds nothing, e.g. after the staged path)
  kRhCapt = 1,      // tile slots per XCD
  kRhWords = 16,
};

// Backward header (its own 256 words in the backward part of the workspace).
enum Bwd2Header : int {
  kB2RowsPad = 0,   // padded columns of the per-expert transposed planes
  kB2ColPad = 16,   // [E_loc + 1] first padded column of each expert
  kB2Words = 256,
};
// Expert column ranges of the transposed planes start at multiples of this, so the weight-
// gradient GEMM reduces in whole K-stages (64 BF16 or 128 E4M3 rows) with zero padding.
constexpr int kPadRows = 128;

// Packed weights: the B operands of the expert GEMMs in fragment order (PackedB, PackedBMX in
// k_gemm.h), four planes per set of local experts. Made once per weight update with
// mok_pack_weights, or by each call into its workspace. BF16 planes hold 2-byte values; MXFP8
// planes hold E4M3 codes, with their scale planes (one byte per 32 codes) after the four code
// planes.
struct PackOffsets {
  int64_t gu;     // [El][2I rows][H]: Wg and Wu rows in the gate/up tiles' order (64-row blocks
                  // alternate Wg and Wu: packed row n is row (n/128)*64 + n%64 of Wg when
                  // (n/64) is even, of Wu when it is odd)
  int64_t wd;     // [El][H rows][I]: Wd (the down GEMM)
  int64_t wdt;    // [El][I rows][H]: Wd^T (the a GEMM)
  int64_t dx;     // [El][H rows][2I]: Wg^T then Wu^T along K (the dx GEMM)
  int64_t gu_s, wd_s, wdt_s, dx_s;   // MXFP8 scale planes (0 in BF16)
  int64_t bytes;
};
inline PackOffsets pack_offsets(int El, int H, int I, int dtype) {
  const int64_t m = int64_t(El) * H * I;   // elements of one H x I matrix per expert set
  if (dtype == MOK_BF16) return PackOffsets{0, 4 * m, 6 * m, 8 * m, 0, 0, 0, 0, 12 * m};
  const int64_t s0 = (6 * m + 255) / 256 * 256;
  return PackOffsets{0,      2 * m,           3 * m,           4 * m,
                     s0,     s0 + 2 * m / 32, s0 + 3 * m / 32, s0 + 4 * m / 32,
                     s0 + 6 * m / 32};
}
constexpr int kPackGu = 1, kPackWd = 2, kPackWdt = 4, kPackDx = 8, kPackAll = 15;

struct Layout {
  // shapes
  int H, E, K, I, S, T, e0, El, M, dtype;
  int64_t N, NK, rows_max;
  int row_align;
  // saved
  int64_t sv_perm, sv_tokpos, sv_touched, sv_multi, sv_pcode, sv_bytes;
  int64_t sv_rhdr, sv_rtiles, sv_rslot, sv_rowner;
  // fused-forward ring, one share per XCD: gather slots (X of one row tile), h slots (h of
  // one row tile) and activation slots (g|u of one row tile)
  int64_t ring_share, xsb, hsb, asb;
  int ring_capx, ring_caph, ring_capa;
  // ws
  int64_t ws_state, ws_tiles, ws_counters, ws_dp, ws_push, ws_trace, ws_pack, ws_bytes;
  int64_t trace_max;   // phase-trace records (MOK_FLAG_TRACE; 0 without it)
  int topk_blocks;
  int64_t tiles_max, J_max;
  // activation row bytes: X | GU | Hact
  int64_t x_row_bytes, gu_row_bytes, h_row_bytes;
  // staged buffers
  int64_t xd_bytes, act_bytes, slots_bytes, wq_bytes;
  // backward workspace (after the forward ws): byte offsets from the ws start
  int64_t rp_max;
  int64_t b_hdr2, b_xd, b_act, b_d, b_dq, b_dgu, b_dguq, b_dp;
  int64_t b_xt, b_dt, b_dgt, b_dut, b_ht, b_qxt, b_qdt, b_qdgt, b_qdut, b_qht;
  int64_t b_restore, b_replay, b_rsl, b_counts, b_actsrc, b_bytes;
};

// Bytes of an activation row of width `w` elements in the activation format: BF16, or
// MXFP8 codes followed (in a separate plane) by one scale per 32 elements.
__host__ __device__ inline int64_t act_row_bytes(int w, int dtype) {
  return dtype == MOK_BF16 ? int64_t(w) * 2 : int64_t(w) + w / 32;
}

inline Layout make_layout(const mok_desc& d) {
  Layout L{};
  L.H = d.hidden; L.E = d.num_experts; L.K = d.top_k; L.I = d.intermediate;
  L.S = d.num_segments; L.T = d.tokens_per_segment; L.e0 = d.expert_begin;
  L.El = d.num_local_experts; L.dtype = d.dtype;
  L.N = int64_t(L.S) * L.T;
  L.NK = L.N * L.K;
  L.row_align = d.dtype == MOK_MXFP8 ? 32 : 1;
  int kk = L.K < L.El ? L.K : L.El;
  L.rows_max = L.N * kk + int64_t(L.El) * (L.row_align - 1);
  L.M = d.minibatch_tokens;
  L.J_max = L.M > 0 ? cdiv(L.rows_max, L.M) : 1;
  L.tiles_max = cdiv(L.rows_max, kTileM) + L.J_max + L.El + 1;
  // activation rows
  L.x_row_bytes = act_row_bytes(L.H, L.dtype);
  L.gu_row_bytes = int64_t(2) * L.I * 2;
  L.h_row_bytes = act_row_bytes(L.I, L.dtype);
  // fused-forward ring: one share per XCD = kRingXSlots gather slots (the X rows of a row tile,
  // needed until its gate/up tiles are done), kRingHSlots h slots (its h, needed until its down
  // tiles are done), then activation slots (its g|u, written by the gate/up tiles and kept for
  // the backward, which recomputes h from it)
  L.xsb = align_up(int64_t(kTileM) * L.x_row_bytes, 256);
  L.hsb = align_up(int64_t(kTileM) * L.h_row_bytes, 256);
  L.asb = align_up(int64_t(kTileM) * L.gu_row_bytes, 256);
  L.ring_share = d.ring_bytes / kXcds / 256 * 256;
  L.ring_capx = kRingXSlots;
  L.ring_caph = kRingHSlots;
  {
    const int64_t rest = L.ring_share - kRingXSlots * L.xsb - kRingHSlots * L.hsb;
    L.ring_capa = rest > 0 ? int(rest / L.asb) : 0;
  }
  // saved
  int64_t off = 1024;
  L.sv_perm = off; off = align_up(off + 4 * L.rows_max, 256);
  L.sv_tokpos = off; off = align_up(off + 4 * L.NK, 256);
  L.sv_touched = off; off = align_up(off + 4 * L.N, 256);
  L.sv_multi = off; off = align_up(off + 4 * L.N, 256);   // tokens with several local pairs
  L.sv_pcode = off; off = align_up(off + 4 * L.rows_max, 256);   // perm | kSoleFlag, see k_place
  L.sv_rhdr = off; off = align_up(off + 4 * kRhWords, 256);
  L.sv_rtiles = off; off = align_up(off + 16 * L.tiles_max, 256);
  L.sv_rslot = off; off = align_up(off + 4 * L.tiles_max, 256);
  L.sv_rowner = off; off = align_up(off + 4 * int64_t(kXcds) * (L.ring_capa > 0 ? L.ring_capa : 1), 256);
  L.sv_bytes = off;
  // ws
  L.topk_blocks = int(cdiv(L.N, kTopkTokensPerBlock));
  off = 256;
  L.ws_state = off; off = align_up(off + 4 * int64_t(L.topk_blocks) * (L.El + 2), 256);
  // weights packed by the call itself when the caller gives none (after the router's words, so
  // its offset does not depend on the minibatch size)
  L.ws_pack = off;
  off = align_up(off + pack_offsets(L.El, L.H, L.I, L.dtype).bytes, 256);
  L.ws_tiles = off; off = align_up(off + 16 * L.tiles_max, 256);
  L.ws_counters = off; off = align_up(off + 4 * (64 + (3 + kXcds) * L.tiles_max), 256);
  L.ws_dp = off; off = align_up(off + 4 * L.rows_max * (L.I / kTileN), 256);
  L.ws_push = off; off = align_up(off + 16 * L.rows_max, 256);   // PushRec per row
  // phase trace: a record per fused-forward item (gate/up and down tiles, gathers), for up to
  // kMaxMacro macrobatches and 64 gathering workgroups per row tile
  L.trace_max = (d.flags & MOK_FLAG_TRACE)
                    ? int64_t(kMaxMacro) * L.tiles_max * (L.I / 128 + cdiv(L.H, kTileN) + 64)
                    : 0;
  L.ws_trace = off; off = align_up(off + int64_t(sizeof(TraceRec)) * L.trace_max, 256);
  L.ws_bytes = off;
  // staged
  L.xd_bytes = align_up(L.rows_max * L.x_row_bytes, 256);
  L.act_bytes = align_up(L.rows_max * (L.gu_row_bytes + L.h_row_bytes), 256);
  L.slots_bytes = align_up(L.NK * L.H * 2, 256);
  L.wq_bytes = align_up(int64_t(L.El) * L.I * L.H * 33 / 32, 256);
  // backward
  const bool mx = L.dtype == MOK_MXFP8;
  L.rp_max = align_up(L.rows_max + int64_t(kPadRows) * L.El, kPadRows);
  const int64_t rm = L.rows_max, rp = L.rp_max, H = L.H, I = L.I;
  off = align_up(L.ws_bytes, 256);
  auto take = [&](int64_t bytes) { int64_t o = off; off = align_up(off + bytes, 256); return o; };
  L.b_hdr2 = take(4 * kB2Words);
  L.b_xd = take(L.xd_bytes);
  L.b_act = take(L.act_bytes);
  L.b_d = take(mx ? 0 : rm * H * 2);      // BF16 D (in MXFP8 the (p D)^T transpose writes
                                          // the H-quantised D rows into b_dq instead)
  L.b_dq = take(mx ? rm * (H + H / 32) : 0);
  L.b_dgu = take(mx ? 0 : rm * 2 * I * 2);   // BF16 dg|du (MXFP8 writes codes only)
  L.b_dguq = take(mx ? rm * (2 * I + 2 * I / 32) : 0);
  L.b_dp = take(rm * (I / kTileN + 1) * 4);
  // BF16 transposed planes (MXFP8 writes only the quantised planes below)
  L.b_xt = take(mx ? 0 : H * rp * 2);
  L.b_dt = take(mx ? 0 : H * rp * 2);
  L.b_dgt = take(mx ? 0 : I * rp * 2);
  L.b_dut = take(mx ? 0 : I * rp * 2);
  L.b_ht = take(mx ? 0 : I * rp * 2);
  L.b_qxt = take(mx ? H * rp * 33 / 32 : 0);
  L.b_qdt = take(mx ? H * rp * 33 / 32 : 0);
  L.b_qdgt = take(mx ? I * rp * 33 / 32 : 0);
  L.b_qdut = take(mx ? I * rp * 33 / 32 : 0);
  L.b_qht = take(mx ? I * rp * 33 / 32 : 0);
  L.b_restore = take(16 * L.tiles_max);
  L.b_replay = take(16 * L.tiles_max);
  L.b_rsl = take(4 * L.tiles_max);
  L.b_counts = take(4 * (4 + 2 * kXcds));   // plan counts, then two work-queue counter sets
  L.b_actsrc = take(4 * rm);                 // where each row's g|u and h live (ActSource)
  L.b_bytes = off;
  return L;
}

// Activation plane pointers for `rows` rows starting at `base`: X (codes) then X scales, etc.
struct ActPlanes {
  uint8_t* x;      // BF16 [rows][H] or codes [rows][H]
  uint8_t* xs;     // MXFP8 scales [rows][H/32] (null in BF16)
  uint16_t* gu;    // BF16 [rows][2I]: g in [0, I), u in [I, 2I)
  uint8_t* h;      // BF16 [rows][I] or codes [rows][I]
  uint8_t* hs;     // MXFP8 scales [rows][I/32]
};

__host__ __device__ inline ActPlanes act_planes(uint8_t* base, int64_t rows, int H, int I, int dtype,
                                                bool with_x) {
  ActPlanes p{};
  uint8_t* q = base;
  if (with_x) {
    p.x = q;
    if (dtype == MOK_BF16) { q += rows * H * 2; }
    else { q += rows * H; p.xs = q; q += rows * (H / 32); }
  }
  p.gu = reinterpret_cast<uint16_t*>(q); q += rows * 2 * I * 2;
  p.h = q;
  if (dtype == MOK_BF16) { q += rows * I * 2; }
  else { q += rows * I; p.hs = q; }
  return p;
}

// Where the backward reads each expert-ordered row's g|u: rows of a tile the forward left
// resident in a ring activation slot are read there (code = slot << 8 | row inside the tile,
// slot = XCD * capa + slot of that XCD); replayed rows (code < 0) from the backward's own
// activation planes. (h is recomputed from g|u wherever the backward needs it.)
struct ActSource {
  ActPlanes act;             // backward activation planes [rows_max]
  const uint8_t* ring;       // the forward's ring (may be null when every code is < 0)
  int64_t ring_share;        // bytes per XCD share
  int64_t aofs, asb;         // activation slots: offset inside a share, bytes per slot
  int capa;                  // activation slots per share
  const int32_t* code;       // [rows_max]
};

// The g|u row (BF16 [2I]: g in [0, I), u in [I, 2I)) of an expert-ordered row.
__device__ inline const uint16_t* act_gu_row(const ActSource& s, int64_t row, int32_t code, int I) {
  if (code < 0) return s.act.gu + row * 2 * I;
  const int slot = code >> 8, lr = code & 255;
  const uint8_t* base = s.ring + int64_t(slot / s.capa) * s.ring_share + s.aofs +
                        int64_t(slot % s.capa) * s.asb;
  return reinterpret_cast<const uint16_t*>(base) + int64_t(lr) * 2 * I;
}

// One m-tile of a grouped GEMM: rows [row0, row0 + nrows) of expert e, inside minibatch j.
struct MTile {
  int32_t j, e, row0, nrows;
};

// ---- launch wrappers (defined in the .hip files) ----------------------------------------
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s);
// Several disjoint word ranges set in one launch (ranges with n <= 0 are skipped).
struct FillRange {
  uint32_t* p;
  int64_t n;
  uint32_t v;
};
constexpr int kMaxFillRanges = 16;
hipError_t launch_fill_ranges(const FillRange* r, int count, hipStream_t s);
// clear_error = false keeps a failure an earlier call recorded in the error word (the
// routers of several macrobatches of one fused launch).
hipError_t launch_router(const Layout& L, const float* logits, int32_t* idx, float* p,
                         uint8_t* saved, uint8_t* ws, hipStream_t s, bool clear_error = true);
hipError_t launch_tiles(const Layout& L, int M, const uint8_t* saved, uint8_t* ws, hipStream_t s);
// The same into an explicit table and count word.
hipError_t launch_tiles_to(const Layout& L, int M, const uint8_t* saved, MTile* tiles,
                           int32_t* ntiles, hipStream_t s);
// Bytes of the workspace the router alone uses (header and look-back scan state).
inline int64_t router_ws_bytes(const Layout& L) {
  return L.ws_state + align_up(4 * int64_t(L.topk_blocks) * (L.El + 2), 256);
}
// The router with its workspace in the library's static per-device scratch (no allocation):
// MOK_ERR_SCRATCH when router_ws_bytes exceeds it.
mok_status launch_router_noalloc(const Layout& L, const float* logits, int32_t* idx, float* p,
                                 uint8_t* saved, hipStream_t s);
hipError_t launch_dispatch(const Layout& L, const uint8_t* saved, const void* const* x_seg,
                           uint8_t* xd, hipStream_t s);
// skip_sole: leave out tokens with a single local pair (their row was written by the GEMM
// epilogue that produced it).
hipError_t launch_combine(const Layout& L, const uint8_t* saved, const int32_t* idx, const float* p,
                          const uint16_t* slots, void* const* out_seg, bool skip_sole,
                          hipStream_t s);
// Push records of the rows [0, rows): pairs flagged kSoleFlag in the schedule's push codes go
// to their token's row of seg with weight p[pair] (1 when p is null); the others to the slots.
hipError_t launch_push_rows(const Layout& L, const uint8_t* saved, uint16_t* slots,
                            void* const* seg, const float* p, PushRec* rec, hipStream_t s);
hipError_t launch_quantize_mx(int batch, int rows, int cols, const uint16_t* src, int transpose,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_ffn_staged(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                             const mok_weights& w, uint8_t* act, uint16_t* slots, uint8_t* ws,
                             hipStream_t s);
hipError_t launch_ffn_gateup(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                             const mok_weights& w, uint8_t* act, uint8_t* ws, hipStream_t s);
// Gate/up GEMM over an explicit tile list (device array and device count).
hipError_t launch_ffn_gateup_list(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                                  const mok_weights& w, uint8_t* act, const MTile* tiles,
                                  const int32_t* ntiles, hipStream_t s);

// Device buffers of one backward call (carved out of the workspace by the host code).
struct BwdBuffers {
  const uint8_t* saved;
  uint8_t* ws;
  const void* const* x_seg;
  const void* const* dout_seg;
  void* const* dx_seg;
  const int32_t* topk_idx;
  const float* topk_p;
  mok_weights w;
  mok_weight_grads g;
  uint16_t* slots;
  float* dp;
  float* dlogits;
  int32_t* hdr2;
  uint8_t *xd, *act, *d, *dq, *dguq;
  uint16_t* dgu;
  float* dp_part;
  uint16_t *xt, *dt, *dgt, *dut, *ht;
  uint8_t *q_xt, *q_dt, *q_dgt, *q_dut, *q_ht;
  uint8_t* ring;      // the forward's ring (null: replay every row)
  int32_t* actsrc;    // [rows_max] row-source codes of the activations (ActSource)
  PushRec* push;      // [rows_max] dx GEMM push records
};
hipError_t launch_backward(const Layout& L, const BwdBuffers& b, hipStream_t s);
// Packed weights (k_pack.hip): writes the planes selected by `planes` (kPack* bits) of
// pack_offsets(El, H, I, dtype) at dst: BF16 from the row-major weights wg, wu [El][I][H], wd
// [El][H][I]; MXFP8 from the quantised codes and scales of mok_weights (forward and transposed
// blockings).
hipError_t launch_pack_weights(const Layout& L, const mok_weights& w, uint8_t* dst, int planes,
                               hipStream_t s);

// Fused forward (k_fused.hip): the ring is split into one share per XCD, each cut into tile
// slots of 256 expert-ordered rows (X | g,u | h).
int fused_slots_per_xcd(const Layout& L);

// Buffers of one macrobatch (one layer call) of a fused forward launch.
struct MacroBuffers {
  const void* const* x_seg;
  const float* logits;
  void* const* out_seg;
  int32_t* idx;
  float* p;
  uint8_t* saved;
  uint16_t* slots;
};

// Workspace of a fused forward over B macrobatches (byte offsets from the ws start). B = 1 is the
// single-call layout: tile table, push records and counters where Layout puts them.
struct MacroWs {
  int64_t counters;
  int64_t tiles[kMaxMacro], ntiles[kMaxMacro], push[kMaxMacro];
  int64_t bytes;
};
inline MacroWs macro_ws(const Layout& L, int B) {
  MacroWs m{};
  int64_t off = align_up(L.ws_bytes, 256);
  if (B <= 1) {
    m.counters = L.ws_counters;
  } else {
    m.counters = off;
    off = align_up(off + 4 * (64 + (3 + kXcds) * int64_t(B) * L.tiles_max), 256);
  }
  m.tiles[0] = L.ws_tiles;
  m.ntiles[0] = 4 * int64_t(kWsNumTiles);
  m.push[0] = L.ws_push;
  for (int b = 1; b < B; ++b) {
    m.ntiles[b] = off; off += 256;
    m.tiles[b] = off; off = align_up(off + 16 * L.tiles_max, 256);
    m.push[b] = off; off = align_up(off + 16 * L.rows_max, 256);
  }
  m.bytes = B <= 1 ? L.ws_bytes : off;
  return m;
}

// Router, tile tables and push records of every macrobatch, then one persistent launch over all
// of their row tiles, then each macrobatch's merge of tokens with several local pairs.
hipError_t launch_layer_fwd_macro(const Layout& L, const mok_desc& d, int B,
                                  const MacroBuffers* mb, const mok_weights& w, uint8_t* ring,
                                  uint8_t* ws, hipStream_t s);

// Router gate projection (k_routerg.hip): workspace of the backward (byte offsets), with the
// token axis padded to Np and the expert axis to Ep (multiples of a 64-element K stage).
struct RouterWs {
  int64_t Np;
  int Ep;
  int64_t dl16, dlt, xt, wrt, bytes;
};
RouterWs router_ws(const Layout& L);
hipError_t launch_router_fwd(const Layout& L, const void* const* x_seg, const uint16_t* wr,
                             float* logits, hipStream_t s);
hipError_t launch_router_bwd(const Layout& L, const void* const* x_seg, const uint16_t* wr,
                             const float* dlogits, float* dwr, void* const* dx_seg, uint8_t* ws,
                             hipStream_t s);

int device_cus();

// One-time set-up per device (kernel attributes are set for the device that is current when
// the first call on it happens). `done` holds one flag per device id below kMaxDevices; other
// ids run the set-up every time.
constexpr int kMaxDevices = 64;
template <class F>
hipError_t once_per_device(std::atomic<bool> (&done)[kMaxDevices], F&& setup) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  if (dev >= 0 && dev < kMaxDevices && done[dev].load(std::memory_order_acquire)) return hipSuccess;
  const hipError_t e = setup();
  if (e == hipSuccess && dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  return e;
}

// Measurement hook (mok_trace_kernel): events recorded around one kernel group.
struct TraceHook {
  int kernel;
  hipEvent_t before, after;
};
extern TraceHook g_trace;
inline void trace_before(int kernel, hipStream_t s) {
  if (g_trace.kernel == kernel && g_trace.before) (void)hipEventRecord(g_trace.before, s);
}
inline void trace_after(int kernel, hipStream_t s) {
  if (g_trace.kernel == kernel && g_trace.after) (void)hipEventRecord(g_trace.after, s);
}

}  // namespace mok
