// Staged grouped SwiGLU expert FFN: a persistent gate/up kernel over all m-tiles x h-column
// tiles, then a persistent down kernel over all m-tiles x output-column tiles. Workgroups walk
// the tile list with a static stride (no atomics, so the assignment is deterministic).
#include "k_ffn.h"

namespace mok {
namespace {

struct FfnStagedArgs {
  const MTile* tiles;
  const int32_t* ntiles;
  const int32_t* perm;
  FfnShape s;
  FfnWeights w;
  ActPlanes pl;
  uint16_t* slots;
};

template <bool MX>
__global__ __launch_bounds__(256, 1) void k_gateup_staged(FfnStagedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GemmLds& sm = *reinterpret_cast<GemmLds*>(smem);
  const int mtiles = *a.ntiles;
  const int ntn = a.s.I / 128;
  const int total = mtiles * ntn;
  for (int t = xcd_logical_id(); t < total; t += gridDim.x) {
    int mt, nt;
    tile_coords(t, mtiles, ntn, mt, nt);
    const MTile tl = a.tiles[mt];
    gateup_tile<MX>(sm, a.s, a.w, a.pl, tl.row0, tl.nrows, tl.e, nt * 128);
  }
}

template <bool MX>
__global__ __launch_bounds__(256, 1) void k_down_staged(FfnStagedArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GemmLds& sm = *reinterpret_cast<GemmLds*>(smem);
  const int mtiles = *a.ntiles;
  const int ntn = (a.s.H + kTileN - 1) / kTileN;
  const int total = mtiles * ntn;
  for (int t = xcd_logical_id(); t < total; t += gridDim.x) {
    int mt, nt;
    tile_coords(t, mtiles, ntn, mt, nt);
    const MTile tl = a.tiles[mt];
    down_tile<MX, kPushSlots>(sm, a.s, a.w, a.pl, tl.row0, tl.row0, tl.nrows, tl.e,
                              nt * kTileN, a.perm, PushTarget{a.slots, nullptr});
  }
}

template <class F>
hipError_t allow_big_lds(F* f) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kGemmLdsBytes));
}

}  // namespace

namespace {
hipError_t ffn_init() {
  static std::atomic<bool> attr_done[kMaxDevices];
  return once_per_device(attr_done, [] {
    hipError_t e;
    if ((e = allow_big_lds(k_gateup_staged<false>)) != hipSuccess) return e;
    if ((e = allow_big_lds(k_gateup_staged<true>)) != hipSuccess) return e;
    if ((e = allow_big_lds(k_down_staged<false>)) != hipSuccess) return e;
    return allow_big_lds(k_down_staged<true>);
  });
}

FfnStagedArgs staged_args(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                          const mok_weights& w, uint8_t* act, uint16_t* slots, uint8_t* ws) {
  const bool mx = L.dtype == MOK_MXFP8;
  FfnStagedArgs a{};
  if (ws) {
    a.tiles = reinterpret_cast<const MTile*>(ws + L.ws_tiles);
    a.ntiles = reinterpret_cast<const int32_t*>(ws) + kWsNumTiles;
  }
  a.perm = reinterpret_cast<const int32_t*>(saved + L.sv_perm);
  a.s = FfnShape{L.H, L.I};
  a.w = ffn_weights(L, w);
  ActPlanes xp = act_planes(const_cast<uint8_t*>(xd), L.rows_max, L.H, L.I, L.dtype, true);
  a.pl = act_planes(act, L.rows_max, L.H, L.I, L.dtype, false);
  a.pl.x = xp.x;
  a.pl.xs = xp.xs;
  a.slots = slots;
  return a;
}
}  // namespace

hipError_t launch_ffn_gateup(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                             const mok_weights& w, uint8_t* act, uint8_t* ws, hipStream_t s) {
  hipError_t err = ffn_init();
  if (err != hipSuccess) return err;
  if ((err = launch_tiles(L, int(L.rows_max), saved, ws, s)) != hipSuccess) return err;
  const FfnStagedArgs a = staged_args(L, saved, xd, w, act, nullptr, ws);
  const int G = device_cus() > 0 ? device_cus() : 256;
  if (L.dtype == MOK_MXFP8)
    hipLaunchKernelGGL(k_gateup_staged<true>, dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  else
    hipLaunchKernelGGL(k_gateup_staged<false>, dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn_gateup_list(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                                  const mok_weights& w, uint8_t* act, const MTile* tiles,
                                  const int32_t* ntiles, hipStream_t s) {
  hipError_t err = ffn_init();
  if (err != hipSuccess) return err;
  FfnStagedArgs a = staged_args(L, saved, xd, w, act, nullptr, nullptr);
  a.tiles = tiles;
  a.ntiles = ntiles;
  const int G = device_cus() > 0 ? device_cus() : 256;
  if (L.dtype == MOK_MXFP8)
    hipLaunchKernelGGL(k_gateup_staged<true>, dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  else
    hipLaunchKernelGGL(k_gateup_staged<false>, dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  return hipGetLastError();
}

hipError_t launch_ffn_staged(const Layout& L, const uint8_t* saved, const uint8_t* xd,
                             const mok_weights& w, uint8_t* act, uint16_t* slots, uint8_t* ws,
                             hipStream_t s) {
  hipError_t err = launch_ffn_gateup(L, saved, xd, w, act, ws, s);
  if (err != hipSuccess) return err;
  const FfnStagedArgs a = staged_args(L, saved, xd, w, act, slots, ws);
  const int G = device_cus() > 0 ? device_cus() : 256;
  if (L.dtype == MOK_MXFP8)
    hipLaunchKernelGGL(k_down_staged<true>, dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  else
    hipLaunchKernelGGL(k_down_staged<false>, dim3(G), dim3(kThreads), kGemmLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace mok
