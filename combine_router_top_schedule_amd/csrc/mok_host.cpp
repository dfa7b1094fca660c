// Host side of libmok: the C ABI declared in include/mok.h. Validates arguments, derives
// buffer layouts from host-known bounds, and enqueues kernels on the caller's stream. No call
// except mok_device_status synchronises or reads device memory back.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "mok_internal.h"

using namespace mok;

namespace mok {
TraceHook g_trace = {MOK_TRACE_NONE, nullptr, nullptr};
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int default_minibatch(const mok_desc& d) {
  const int cus = device_cus() > 0 ? device_cus() : 256;
  int64_t m = mok_two_wave_floor(cus, kTileM, kTileN, d.intermediate);
  m = align_up(m, 32);
  return int(m);
}

mok_status check_desc(const mok_desc* d) {
  if (!d) return MOK_ERR_NULL;
  if (d->dtype != MOK_BF16 && d->dtype != MOK_MXFP8) return MOK_ERR_DTYPE;
  if (d->hidden <= 0 || d->hidden % 128 || d->intermediate <= 0 || d->intermediate % 128)
    return MOK_ERR_SHAPE;
  if (d->num_experts < 1 || d->num_experts > kMaxExperts) return MOK_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > kMaxTopK || d->top_k > d->num_experts) return MOK_ERR_SHAPE;
  if (d->num_segments < 1 || d->tokens_per_segment < 1) return MOK_ERR_SHAPE;
  if (d->expert_begin < 0 || d->num_local_experts < 1 || d->num_local_experts > kMaxLocalExperts ||
      d->expert_begin + d->num_local_experts > d->num_experts)
    return MOK_ERR_SHAPE;
  // MXFP8 weight gradients quantise along tokens in 32-row blocks, which minibatch cuts must
  // not split; BF16 takes any minibatch size.
  if (d->minibatch_tokens < 0) return MOK_ERR_SHAPE;
  if (d->dtype == MOK_MXFP8 && d->minibatch_tokens % 32) return MOK_ERR_SHAPE;
  if (d->comm_cus < 0 || d->ring_bytes < 0) return MOK_ERR_SHAPE;
  const int64_t N = int64_t(d->num_segments) * d->tokens_per_segment;
  // Look-back words keep counts in 30 bits; pair ids and rows are int32.
  if (N * d->top_k >= (int64_t(1) << 30)) return MOK_ERR_SHAPE;
  return MOK_OK;
}

mok_status check_weights(const mok_desc* d, const mok_weights* w, bool backward) {
  if (w->packed && (reinterpret_cast<uintptr_t>(w->packed) & 255u)) return MOK_ERR_ALIGN;
  if (d->dtype == MOK_BF16) {
    if (!w->wg || !w->wu || !w->wd) return MOK_ERR_NULL;
    if (!aligned16(w->wg) || !aligned16(w->wu) || !aligned16(w->wd)) return MOK_ERR_ALIGN;
  } else {
    if (!w->wg_q || !w->wg_s || !w->wu_q || !w->wu_s || !w->wd_q || !w->wd_s) return MOK_ERR_DTYPE;
    if (!aligned16(w->wg_q) || !aligned16(w->wu_q) || !aligned16(w->wd_q)) return MOK_ERR_ALIGN;
    if (backward) {
      if (!w->wgt_q || !w->wgt_s || !w->wut_q || !w->wut_s || !w->wdt_q || !w->wdt_s) return MOK_ERR_DTYPE;
      if (!aligned16(w->wgt_q) || !aligned16(w->wut_q) || !aligned16(w->wdt_q)) return MOK_ERR_ALIGN;
    }
  }
  return MOK_OK;
}

Layout layout_of(const mok_desc& d) {
  mok_desc e = d;
  if (e.minibatch_tokens == 0) e.minibatch_tokens = default_minibatch(d);
  return make_layout(e);
}

mok_status hip_status(hipError_t e) { return e == hipSuccess ? MOK_OK : MOK_ERR_HIP; }

// The weights as the kernels read them, with packed planes: the caller's (w.packed) or the
// `planes` packed here into the workspace.
mok_status with_packed(const Layout& L, const mok_weights& w, uint8_t* ws, int planes,
                       hipStream_t s, mok_weights* out) {
  *out = w;
  if (w.packed) return MOK_OK;
  uint8_t* dst = ws + L.ws_pack;
  const hipError_t e = launch_pack_weights(L, w, dst, planes, s);
  if (e != hipSuccess) return MOK_ERR_HIP;
  out->packed = dst;
  return MOK_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int mok_abi_version(void) { return MOK_ABI_VERSION; }

const char* mok_status_str(mok_status s) {
  switch (s) {
    case MOK_OK: return "ok";
    case MOK_ERR_NULL: return "null pointer argument";
    case MOK_ERR_SHAPE: return "invalid shape";
    case MOK_ERR_DTYPE: return "invalid dtype or missing dtype-specific field";
    case MOK_ERR_ALIGN: return "misaligned device pointer";
    case MOK_ERR_WORKSPACE: return "workspace error";
    case MOK_ERR_RING: return "ring buffer smaller than mok_sizes.ring_min_bytes";
    case MOK_ERR_HIP: return "HIP runtime or launch failure";
    case MOK_ERR_DEVICE_TIMEOUT: return "device-side bounded wait expired";
    case MOK_ERR_UNSUPPORTED: return "unsupported";
    case MOK_ERR_SCRATCH: return "shape needs more than the static scratch of mok_schedule_noalloc";
  }
  return "unknown status";
}

int64_t mok_two_wave_floor(int32_t cus, int32_t tile_m, int32_t tile_n, int32_t intermediate) {
  if (cus <= 0 || tile_m <= 0 || tile_n <= 0 || intermediate <= 0) return 0;
  const int64_t num = int64_t(2) * cus * tile_m * tile_n;
  const int64_t den = int64_t(2) * intermediate;
  return (num + den - 1) / den;
}

int32_t mok_device_cus(void) { return device_cus(); }

mok_status mok_trace_kernel(int32_t kernel, void* before, void* after) {
  if (kernel < MOK_TRACE_NONE || kernel > MOK_TRACE_COMBINE) return MOK_ERR_SHAPE;
  g_trace.kernel = (before && after) ? kernel : MOK_TRACE_NONE;
  g_trace.before = reinterpret_cast<hipEvent_t>(before);
  g_trace.after = reinterpret_cast<hipEvent_t>(after);
  return MOK_OK;
}

mok_status mok_query_sizes(const mok_desc* desc, mok_sizes* sizes) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!sizes) return MOK_ERR_NULL;
  const Layout L = layout_of(*desc);
  sizes->saved_bytes = size_t(L.sv_bytes);
  sizes->ws_bytes = size_t(L.ws_bytes);
  sizes->bwd_ws_bytes = size_t(L.b_bytes);
  sizes->slots_bytes = size_t(L.slots_bytes);
  sizes->xd_bytes = size_t(L.xd_bytes);
  sizes->act_bytes = size_t(L.act_bytes);
  sizes->wq_bytes = size_t(L.wq_bytes);
  sizes->rows_max = L.rows_max;
  sizes->ring_slots = kXcds * fused_slots_per_xcd(L);
  sizes->minibatch = L.M;
  sizes->slot_bytes = L.asb;
  sizes->perm_offset = L.sv_perm;
  sizes->tokpos_offset = L.sv_tokpos;
  sizes->touched_offset = L.sv_touched;
  sizes->x_slot_bytes = L.xsb;
  sizes->ring_min_bytes = int64_t(kXcds) * (kRingXSlots * L.xsb + kRingHSlots * L.hsb + 2 * L.asb);
  sizes->tiles_offset = L.ws_tiles;
  sizes->tiles_max = L.tiles_max;
  sizes->trace_offset = L.trace_max > 0 ? L.ws_trace : 0;
  sizes->trace_records = L.trace_max;
  sizes->h_slot_bytes = L.hsb;
  sizes->packed_bytes = pack_offsets(L.El, L.H, L.I, L.dtype).bytes;
  return MOK_OK;
}

mok_status mok_workspace_size(const mok_desc* desc, size_t* ws_bytes, size_t* saved_bytes,
                              size_t* slot_bytes) {
  if (!ws_bytes || !saved_bytes || !slot_bytes) return MOK_ERR_NULL;
  mok_sizes sz{};
  const mok_status st = mok_query_sizes(desc, &sz);
  if (st != MOK_OK) return st;
  *ws_bytes = sz.bwd_ws_bytes;
  *saved_bytes = sz.saved_bytes;
  *slot_bytes = sz.slots_bytes;
  return MOK_OK;
}

mok_status mok_schedule(const mok_desc* desc, const float* logits_dev, int32_t* topk_idx_dev,
                        float* topk_p_dev, void* saved_dev, void* ws_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!logits_dev || !topk_idx_dev || !topk_p_dev || !saved_dev || !ws_dev) return MOK_ERR_NULL;
  if (!aligned16(logits_dev) || !aligned16(saved_dev) || !aligned16(ws_dev)) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  hipStream_t s = as_stream(stream);
  // (the router clears the workspace header and the ring record: the staged path leaves
  // nothing in the ring for the backward)
  return hip_status(launch_router(L, logits_dev, topk_idx_dev, topk_p_dev,
                                  static_cast<uint8_t*>(saved_dev), static_cast<uint8_t*>(ws_dev), s));
}

mok_status mok_schedule_noalloc(const mok_desc* desc, const float* logits_dev,
                                int32_t* topk_idx_dev, float* topk_p_dev, void* saved_dev,
                                void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!logits_dev || !topk_idx_dev || !topk_p_dev || !saved_dev) return MOK_ERR_NULL;
  if (!aligned16(logits_dev) || !aligned16(saved_dev)) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  return launch_router_noalloc(L, logits_dev, topk_idx_dev, topk_p_dev,
                               static_cast<uint8_t*>(saved_dev), as_stream(stream));
}

mok_status mok_dispatch(const mok_desc* desc, const void* saved_dev, const void* const* x_seg_dev,
                        void* xd_dev, void* ws_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!saved_dev || !x_seg_dev || !xd_dev || !ws_dev) return MOK_ERR_NULL;
  if (!aligned16(xd_dev) || !aligned16(saved_dev)) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  return hip_status(launch_dispatch(L, static_cast<const uint8_t*>(saved_dev), x_seg_dev,
                                    static_cast<uint8_t*>(xd_dev), as_stream(stream)));
}

mok_status mok_expert_ffn(const mok_desc* desc, const void* saved_dev, const void* xd_dev,
                          const mok_weights* w, void* act_dev, void* slots_dev, void* ws_dev,
                          void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!saved_dev || !xd_dev || !w || !act_dev || !slots_dev || !ws_dev) return MOK_ERR_NULL;
  st = check_weights(desc, w, false);
  if (st != MOK_OK) return st;
  if (!aligned16(xd_dev) || !aligned16(act_dev) || !aligned16(slots_dev)) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  mok_weights wk;
  st = with_packed(L, *w, static_cast<uint8_t*>(ws_dev), kPackGu | kPackWd, as_stream(stream), &wk);
  if (st != MOK_OK) return st;
  return hip_status(launch_ffn_staged(L, static_cast<const uint8_t*>(saved_dev),
                                      static_cast<const uint8_t*>(xd_dev), wk,
                                      static_cast<uint8_t*>(act_dev),
                                      static_cast<uint16_t*>(slots_dev),
                                      static_cast<uint8_t*>(ws_dev), as_stream(stream)));
}

mok_status mok_combine(const mok_desc* desc, const void* saved_dev, const int32_t* topk_idx_dev,
                       const float* topk_p_dev, const void* slots_dev, void* const* out_seg_dev,
                       void* ws_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!saved_dev || !topk_idx_dev || !slots_dev || !out_seg_dev || !ws_dev) return MOK_ERR_NULL;
  if (!aligned16(slots_dev)) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  return hip_status(launch_combine(L, static_cast<const uint8_t*>(saved_dev), topk_idx_dev,
                                   topk_p_dev, static_cast<const uint16_t*>(slots_dev), out_seg_dev,
                                   false, as_stream(stream)));
}

mok_status mok_quantize_mx(int32_t batch, int32_t rows, int32_t cols, const void* src_dev,
                           int32_t transpose, uint8_t* codes_dev, uint8_t* scales_dev,
                           void* stream) {
  if (!src_dev || !codes_dev || !scales_dev) return MOK_ERR_NULL;
  if (batch < 1 || rows < 1 || cols < 1) return MOK_ERR_SHAPE;
  if ((transpose ? rows : cols) % 32) return MOK_ERR_SHAPE;
  if (transpose != 0 && transpose != 1) return MOK_ERR_SHAPE;
  if (!aligned16(codes_dev)) return MOK_ERR_ALIGN;
  return hip_status(launch_quantize_mx(batch, rows, cols, static_cast<const uint16_t*>(src_dev),
                                       transpose, codes_dev, scales_dev, as_stream(stream)));
}

mok_status mok_pack_weights(const mok_desc* desc, const mok_weights* w, void* packed_dev,
                            void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!w || !packed_dev) return MOK_ERR_NULL;
  mok_weights src = *w;
  src.packed = nullptr;
  st = check_weights(desc, &src, desc->dtype == MOK_MXFP8);
  if (st != MOK_OK) return st;
  if (reinterpret_cast<uintptr_t>(packed_dev) & 255u) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  return hip_status(launch_pack_weights(L, src, static_cast<uint8_t*>(packed_dev), kPackAll,
                                        as_stream(stream)));
}

mok_status mok_device_status(const void* ws_dev, void* stream, mok_status* out) {
  if (!ws_dev || !out) return MOK_ERR_NULL;
  if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return MOK_ERR_HIP;
  int32_t word = 0;
  if (hipMemcpy(&word, ws_dev, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess) return MOK_ERR_HIP;
  *out = static_cast<mok_status>(word);
  return MOK_OK;
}

}  // extern "C"

extern "C" {

mok_status mok_layer_fwd(const mok_desc* desc, const void* const* x_seg_dev,
                         const float* logits_dev, const mok_weights* w,
                         void* const* out_seg_dev, int32_t* topk_idx_dev, float* topk_p_dev,
                         void* saved_dev, void* ring_dev, void* slots_dev, void* ws_dev,
                         void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!x_seg_dev || !logits_dev || !w || !out_seg_dev || !topk_idx_dev || !topk_p_dev ||
      !saved_dev || !ring_dev || !slots_dev || !ws_dev)
    return MOK_ERR_NULL;
  st = check_weights(desc, w, false);
  if (st != MOK_OK) return st;
  if (!aligned16(logits_dev) || !aligned16(saved_dev) || !aligned16(ring_dev) ||
      !aligned16(slots_dev) || !aligned16(ws_dev))
    return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  if (fused_slots_per_xcd(L) < 2) return MOK_ERR_RING;
  const MacroBuffers mb{x_seg_dev, logits_dev, out_seg_dev, topk_idx_dev, topk_p_dev,
                        static_cast<uint8_t*>(saved_dev), static_cast<uint16_t*>(slots_dev)};
  mok_weights wk;
  st = with_packed(L, *w, static_cast<uint8_t*>(ws_dev), kPackGu | kPackWd, as_stream(stream), &wk);
  if (st != MOK_OK) return st;
  return hip_status(launch_layer_fwd_macro(L, *desc, 1, &mb, wk, static_cast<uint8_t*>(ring_dev),
                                           static_cast<uint8_t*>(ws_dev), as_stream(stream)));
}

mok_status mok_macro_ws_size(const mok_desc* desc, int32_t num_macro, size_t* ws_bytes) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!ws_bytes) return MOK_ERR_NULL;
  if (num_macro < 1 || num_macro > kMaxMacro) return MOK_ERR_SHAPE;
  *ws_bytes = size_t(macro_ws(layout_of(*desc), num_macro).bytes);
  return MOK_OK;
}

mok_status mok_layer_fwd_macro(const mok_desc* desc, int32_t num_macro,
                               const void* const* const* x_seg_dev, const float* const* logits_dev,
                               const mok_weights* w, void* const* const* out_seg_dev,
                               int32_t* const* topk_idx_dev, float* const* topk_p_dev,
                               void* const* saved_dev, void* ring_dev, void* const* slots_dev,
                               void* ws_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (num_macro < 1 || num_macro > kMaxMacro) return MOK_ERR_SHAPE;
  if (!x_seg_dev || !logits_dev || !w || !out_seg_dev || !topk_idx_dev || !topk_p_dev ||
      !saved_dev || !ring_dev || !slots_dev || !ws_dev)
    return MOK_ERR_NULL;
  st = check_weights(desc, w, false);
  if (st != MOK_OK) return st;
  if (!aligned16(ring_dev) || !aligned16(ws_dev)) return MOK_ERR_ALIGN;
  MacroBuffers mb[kMaxMacro];
  for (int b = 0; b < num_macro; ++b) {
    if (!x_seg_dev[b] || !logits_dev[b] || !out_seg_dev[b] || !topk_idx_dev[b] || !topk_p_dev[b] ||
        !saved_dev[b] || !slots_dev[b])
      return MOK_ERR_NULL;
    if (!aligned16(logits_dev[b]) || !aligned16(saved_dev[b]) || !aligned16(slots_dev[b]))
      return MOK_ERR_ALIGN;
    for (int o = 0; o < b; ++o)
      if (saved_dev[o] == saved_dev[b] || slots_dev[o] == slots_dev[b] ||
          out_seg_dev[o] == out_seg_dev[b] || topk_idx_dev[o] == topk_idx_dev[b])
        return MOK_ERR_SHAPE;   // each macrobatch needs its own outputs
    mb[b] = MacroBuffers{x_seg_dev[b], logits_dev[b], out_seg_dev[b], topk_idx_dev[b],
                         topk_p_dev[b], static_cast<uint8_t*>(saved_dev[b]),
                         static_cast<uint16_t*>(slots_dev[b])};
  }
  const Layout L = layout_of(*desc);
  if (fused_slots_per_xcd(L) < 2) return MOK_ERR_RING;
  mok_weights wk;
  st = with_packed(L, *w, static_cast<uint8_t*>(ws_dev), kPackGu | kPackWd, as_stream(stream), &wk);
  if (st != MOK_OK) return st;
  return hip_status(launch_layer_fwd_macro(L, *desc, num_macro, mb, wk,
                                           static_cast<uint8_t*>(ring_dev),
                                           static_cast<uint8_t*>(ws_dev), as_stream(stream)));
}

mok_status mok_layer_bwd(const mok_desc* desc, const void* const* dout_seg_dev,
                         const void* const* x_seg_dev, const mok_weights* w,
                         const int32_t* topk_idx_dev, const float* topk_p_dev,
                         const void* saved_dev, void* ring_dev, void* slots_dev,
                         void* const* dx_seg_dev, float* dp_dev, float* dlogits_dev,
                         const mok_weight_grads* g, void* ws_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!dout_seg_dev || !x_seg_dev || !w || !topk_idx_dev || !topk_p_dev || !saved_dev ||
      !slots_dev || !dx_seg_dev || !dp_dev || !g || !g->dwg || !g->dwu || !g->dwd || !ws_dev)
    return MOK_ERR_NULL;
  if (dlogits_dev && desc->num_local_experts != desc->num_experts) return MOK_ERR_SHAPE;
  st = check_weights(desc, w, true);
  if (st != MOK_OK) return st;
  if (!aligned16(slots_dev) || !aligned16(ws_dev) || !aligned16(g->dwg) || !aligned16(g->dwu) ||
      !aligned16(g->dwd))
    return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  uint8_t* ws = static_cast<uint8_t*>(ws_dev);
  BwdBuffers b{};
  b.saved = static_cast<const uint8_t*>(saved_dev);
  b.ws = ws;
  b.x_seg = x_seg_dev;
  b.dout_seg = dout_seg_dev;
  b.dx_seg = dx_seg_dev;
  b.topk_idx = topk_idx_dev;
  b.topk_p = topk_p_dev;
  // the backward replays gate/up (packed gate/up plane) and reads Wd^T and [Wg^T | Wu^T]
  st = with_packed(L, *w, ws, kPackGu | kPackWdt | kPackDx, as_stream(stream), &b.w);
  if (st != MOK_OK) return st;
  b.g = *g;
  b.slots = static_cast<uint16_t*>(slots_dev);
  b.dp = dp_dev;
  b.dlogits = dlogits_dev;
  b.hdr2 = reinterpret_cast<int32_t*>(ws + L.b_hdr2);
  b.xd = ws + L.b_xd;
  b.act = ws + L.b_act;
  b.actsrc = reinterpret_cast<int32_t*>(ws + L.b_actsrc);
  b.push = reinterpret_cast<PushRec*>(ws + L.ws_push);
  b.d = ws + L.b_d;
  b.dq = ws + L.b_dq;
  b.dgu = reinterpret_cast<uint16_t*>(ws + L.b_dgu);
  b.dguq = ws + L.b_dguq;
  b.dp_part = reinterpret_cast<float*>(ws + L.b_dp);
  b.xt = reinterpret_cast<uint16_t*>(ws + L.b_xt);
  b.dt = reinterpret_cast<uint16_t*>(ws + L.b_dt);
  b.dgt = reinterpret_cast<uint16_t*>(ws + L.b_dgt);
  b.dut = reinterpret_cast<uint16_t*>(ws + L.b_dut);
  b.ht = reinterpret_cast<uint16_t*>(ws + L.b_ht);
  b.q_xt = ws + L.b_qxt;
  b.q_dt = ws + L.b_qdt;
  b.q_dgt = ws + L.b_qdgt;
  b.q_dut = ws + L.b_qdut;
  b.q_ht = ws + L.b_qht;
  b.ring = static_cast<uint8_t*>(ring_dev);
  return hip_status(launch_backward(L, b, as_stream(stream)));
}

}  // extern "C"

extern "C" mok_status mok_autotune(const mok_desc* desc, const void* const* x_seg_dev,
                                   const float* logits_dev, const mok_weights* w,
                                   void* const* out_seg_dev, int32_t* topk_idx_dev,
                                   float* topk_p_dev, void* saved_dev, void* ring_dev,
                                   void* slots_dev, void* ws_dev, void* stream, int32_t reps,
                                   mok_desc* tuned, float* best_ms, mok_tune_result* results,
                                   int32_t max_results, int32_t* n_results) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!tuned || !best_ms) return MOK_ERR_NULL;
  if (reps < 1 || reps > 1000 || max_results < 0) return MOK_ERR_SHAPE;
  if (results && max_results > 0 && !n_results) return MOK_ERR_NULL;
  const Layout L0 = layout_of(*desc);
  const int M0 = L0.M;
  const int cus = device_cus() > 0 ? device_cus() : 256;
  const int64_t all_rows = align_up(L0.rows_max, 32);
  std::vector<int> ms_cand = {M0};
  for (int64_t m : {int64_t(2) * M0, int64_t(4) * M0, all_rows})
    if (m > ms_cand.back() && m <= (int64_t(1) << 30)) ms_cand.push_back(int(m));
  std::vector<int> cu_cand;
  for (int c : {8, 16, 24, 32, 48})
    if (c < cus / 2) cu_cand.push_back(c);
  if (cu_cand.empty()) cu_cand.push_back(kXcds);
  hipStream_t s = as_stream(stream);
  if (!w || !ws_dev) return MOK_ERR_NULL;
  if (!aligned16(ws_dev)) return MOK_ERR_ALIGN;
  st = check_weights(desc, w, false);
  if (st != MOK_OK) return st;
  // BF16 weights without packed planes are packed once here (the pack region's offset is the
  // same for every minibatch size), so that no timed call includes the packing
  mok_weights wk;
  st = with_packed(L0, *w, static_cast<uint8_t*>(ws_dev), kPackGu | kPackWd, s, &wk);
  if (st != MOK_OK) return st;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return MOK_ERR_HIP;
  }
  mok_status out = MOK_OK;
  float best = -1.f;
  mok_desc best_d = *desc;
  int32_t n = 0;
  for (int m : ms_cand) {
    for (int c : cu_cand) {
      mok_desc d = *desc;
      d.minibatch_tokens = m;
      d.comm_cus = c;
      std::vector<float> times;
      for (int r = 0; r <= reps && out == MOK_OK; ++r) {
        if (hipEventRecord(e0, s) != hipSuccess) { out = MOK_ERR_HIP; break; }
        out = mok_layer_fwd(&d, x_seg_dev, logits_dev, &wk, out_seg_dev, topk_idx_dev, topk_p_dev,
                            saved_dev, ring_dev, slots_dev, ws_dev, stream);
        if (out != MOK_OK) break;
        if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
          out = MOK_ERR_HIP;
          break;
        }
        mok_status dev = MOK_OK;
        if ((out = mok_device_status(ws_dev, stream, &dev)) != MOK_OK) break;
        if (dev != MOK_OK) { out = dev; break; }
        float t = 0.f;
        if (hipEventElapsedTime(&t, e0, e1) != hipSuccess) { out = MOK_ERR_HIP; break; }
        if (r > 0) times.push_back(t);   // the first call is a warm-up
      }
      if (out != MOK_OK) break;
      std::sort(times.begin(), times.end());
      const float med = times[times.size() / 2];
      if (results && n < max_results) results[n] = mok_tune_result{m, c, med};
      ++n;
      if (best < 0.f || med < best) {
        best = med;
        best_d = d;
      }
    }
    if (out != MOK_OK) break;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (out != MOK_OK) return out;
  *tuned = best_d;
  *best_ms = best;
  if (n_results) *n_results = std::min(n, max_results);
  return MOK_OK;
}

extern "C" {

mok_status mok_router_fwd(const mok_desc* desc, const void* const* x_seg_dev, const void* wr_dev,
                          float* logits_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!x_seg_dev || !wr_dev || !logits_dev) return MOK_ERR_NULL;
  if (desc->num_experts % 4) return MOK_ERR_SHAPE;
  if (!aligned16(wr_dev) || !aligned16(logits_dev)) return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  return hip_status(launch_router_fwd(L, x_seg_dev, static_cast<const uint16_t*>(wr_dev),
                                      logits_dev, as_stream(stream)));
}

mok_status mok_router_ws_size(const mok_desc* desc, size_t* ws_bytes) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!ws_bytes) return MOK_ERR_NULL;
  *ws_bytes = size_t(router_ws(layout_of(*desc)).bytes);
  return MOK_OK;
}

mok_status mok_router_bwd(const mok_desc* desc, const void* const* x_seg_dev, const void* wr_dev,
                          const float* dlogits_dev, float* dwr_dev, void* const* dx_seg_dev,
                          void* ws_dev, void* stream) {
  mok_status st = check_desc(desc);
  if (st != MOK_OK) return st;
  if (!x_seg_dev || !wr_dev || !dlogits_dev || !dwr_dev || !dx_seg_dev || !ws_dev)
    return MOK_ERR_NULL;
  if (desc->num_experts % 4) return MOK_ERR_SHAPE;
  if (!aligned16(wr_dev) || !aligned16(dlogits_dev) || !aligned16(dwr_dev) || !aligned16(ws_dev))
    return MOK_ERR_ALIGN;
  const Layout L = layout_of(*desc);
  return hip_status(launch_router_bwd(L, x_seg_dev, static_cast<const uint16_t*>(wr_dev),
                                      dlogits_dev, dwr_dev, dx_seg_dev,
                                      static_cast<uint8_t*>(ws_dev), as_stream(stream)));
}

}  // extern "C"
