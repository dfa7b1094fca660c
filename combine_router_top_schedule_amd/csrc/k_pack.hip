// Packing of the expert weights into the B-operand planes of the expert GEMMs, in MFMA
// fragment order (PackedB and PackedBMX in k_gemm.h; plane offsets in pack_offsets). Run once
// per weight update (mok_pack_weights), or by a layer call into its workspace when the caller
// gives none.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mok_device.h"
#include "mok_internal.h"

namespace mok {
namespace {

struct PackArgs {
  const uint16_t *wg, *wu, *wd;   // BF16, row-major [El][I][H], [El][I][H], [El][H][I]
  // MXFP8 codes and scales: forward blocking wg, wu [El][I][H], wd [El][H][I]; transposed
  // blocking wgt, wut [El][H][I], wdt [El][I][H] (scales: the last axis / 32)
  const uint8_t *wg_q, *wg_s, *wu_q, *wu_s, *wd_q, *wd_s;
  const uint8_t *wgt_q, *wgt_s, *wut_q, *wut_s, *wdt_q, *wdt_s;
  uint8_t* dst;
  PackOffsets po;
  int El, H, I;
};

// One thread per 16-byte piece of plane PLANE (0 gate/up, 1 Wd, 2 Wd^T, 3 [Wg^T | Wu^T]; one
// launch per plane, the plane fixed at compile time). Piece p of a plane with R rows and
// reduction length K per expert is p = e * (R*K/8) + (n32 * (K/16) + k16) * 64 + l: row
// 32 n32 + l % 32, elements 16 k16 + 8 (l / 32) .. +7. Stores are consecutive. The gate/up and
// Wd planes read 16 bytes of one row per piece; the transposed planes read 8 elements of one
// column, 32 consecutive columns per half-wave.
template <int PLANE>
__global__ __launch_bounds__(256) void k_pack_bf16(PackArgs a) {
  const int H = a.H, I = a.I;
  const int R = PLANE == 0 ? 2 * I : (PLANE == 2 ? I : H);
  const int K = PLANE == 0 || PLANE == 2 ? H : (PLANE == 1 ? I : 2 * I);
  const int64_t off = PLANE == 0 ? a.po.gu : (PLANE == 1 ? a.po.wd : (PLANE == 2 ? a.po.wdt : a.po.dx));
  const int k16s = K / 16;
  const int64_t per_e = int64_t(R) * K / 8;
  const int64_t total = per_e * a.El;
  u32x4* out = reinterpret_cast<u32x4*>(a.dst + off);
  for (int64_t p = blockIdx.x * int64_t(blockDim.x) + threadIdx.x; p < total;
       p += int64_t(gridDim.x) * blockDim.x) {
    const int e = int(p / per_e);
    const int64_t q = p - e * per_e;
    const int lane = int(q & 63);
    const int64_t frag = q >> 6;
    const int n32 = int(frag / k16s), k16 = int(frag - int64_t(n32) * k16s);
    const int n = n32 * 32 + (lane & 31);
    const int k = k16 * 16 + (lane >> 5) * 8;
    u32x4 v;
    if constexpr (PLANE <= 1) {
      const uint16_t* row;
      if constexpr (PLANE == 0) {
        const int qb = n >> 6;                        // 64-row block: even Wg, odd Wu
        const int i = (qb >> 1) * 64 + (n & 63);
        row = ((qb & 1) ? a.wu : a.wg) + (int64_t(e) * I + i) * H;
      } else {
        row = a.wd + (int64_t(e) * H + n) * I;
      }
      v = *reinterpret_cast<const u32x4*>(row + k);
    } else {
      const uint16_t* col;
      int64_t stride;
      if constexpr (PLANE == 2) {                      // Wd^T: element t is Wd[e][k + t][n]
        col = a.wd + (int64_t(e) * H + k) * I + n;
        stride = I;
      } else if (k < I) {                              // Wg^T: Wg[e][k + t][n]
        col = a.wg + (int64_t(e) * I + k) * H + n;
        stride = H;
      } else {                                         // Wu^T: Wu[e][k - I + t][n]
        col = a.wu + (int64_t(e) * I + (k - I)) * H + n;
        stride = H;
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
        v[t] = uint32_t(col[2 * t * stride]) | (uint32_t(col[(2 * t + 1) * stride]) << 16);
    }
    out[p] = v;
  }
}

// MXFP8: the codes of plane PLANE in 16-byte pieces, then its scale bytes. Code piece p is
// p = e * (R*K/16) + ((n32 * (K/64) + k64) * 2 + half) * 64 + l: row 32 n32 + l % 32, codes
// 64 k64 + 32 half + 16 (l / 32) .. +15 (16 consecutive bytes of one source row). Scale byte q is
// q = e * (R*K/32) + (n32 * (K/64) + k64) * 64 + l: row 32 n32 + l % 32, block 2 k64 + l / 32.
template <int PLANE>
__global__ __launch_bounds__(256) void k_pack_mx(PackArgs a) {
  const int H = a.H, I = a.I;
  const int R = PLANE == 0 ? 2 * I : (PLANE == 2 ? I : H);
  const int K = PLANE == 0 || PLANE == 2 ? H : (PLANE == 1 ? I : 2 * I);
  const int64_t off = PLANE == 0 ? a.po.gu : (PLANE == 1 ? a.po.wd : (PLANE == 2 ? a.po.wdt : a.po.dx));
  const int64_t off_s =
      PLANE == 0 ? a.po.gu_s : (PLANE == 1 ? a.po.wd_s : (PLANE == 2 ? a.po.wdt_s : a.po.dx_s));
  const int k64s = K / 64;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  const int64_t t0 = blockIdx.x * int64_t(blockDim.x) + threadIdx.x;
  // source row n of expert e: codes (K or, for the dx plane, two halves of I) and scales
  auto src_row = [&](int e, int n, int k, const uint8_t*& c, const uint8_t*& sc, int& kk) {
    kk = k;
    if constexpr (PLANE == 0) {
      const int qb = n >> 6;                          // 64-row block: even Wg, odd Wu
      const int64_t i = int64_t(e) * I + (qb >> 1) * 64 + (n & 63);
      c = ((qb & 1) ? a.wu_q : a.wg_q) + i * H;
      sc = ((qb & 1) ? a.wu_s : a.wg_s) + i * (H / 32);
    } else if constexpr (PLANE == 1) {
      c = a.wd_q + (int64_t(e) * H + n) * I;
      sc = a.wd_s + (int64_t(e) * H + n) * (I / 32);
    } else if constexpr (PLANE == 2) {
      c = a.wdt_q + (int64_t(e) * I + n) * H;
      sc = a.wdt_s + (int64_t(e) * I + n) * (H / 32);
    } else {
      const bool second = k >= I;                     // Wu^T half of K
      c = (second ? a.wut_q : a.wgt_q) + (int64_t(e) * H + n) * I;
      sc = (second ? a.wut_s : a.wgt_s) + (int64_t(e) * H + n) * (I / 32);
      if (second) kk = k - I;
    }
  };
  const int64_t per_e = int64_t(R) * K / 16;
  u32x4* out = reinterpret_cast<u32x4*>(a.dst + off);
  for (int64_t p = t0; p < per_e * a.El; p += stride) {
    const int e = int(p / per_e);
    const int64_t q = p - e * per_e;
    const int lane = int(q & 63);
    const int64_t rest = q >> 6;
    const int half = int(rest & 1);
    const int64_t frag = rest >> 1;
    const int n32 = int(frag / k64s), k64 = int(frag - int64_t(n32) * k64s);
    const uint8_t *c, *sc;
    int kk;
    src_row(e, n32 * 32 + (lane & 31), k64 * 64 + half * 32 + (lane >> 5) * 16, c, sc, kk);
    out[p] = *reinterpret_cast<const u32x4*>(c + kk);
  }
  const int64_t per_e_s = int64_t(R) * K / 32;
  uint8_t* out_s = a.dst + off_s;
  for (int64_t p = t0; p < per_e_s * a.El; p += stride) {
    const int e = int(p / per_e_s);
    const int64_t q = p - e * per_e_s;
    const int lane = int(q & 63);
    const int64_t frag = q >> 6;
    const int n32 = int(frag / k64s), k64 = int(frag - int64_t(n32) * k64s);
    const uint8_t *c, *sc;
    int kk;
    src_row(e, n32 * 32 + (lane & 31), (k64 * 2 + (lane >> 5)) * 32, c, sc, kk);
    out_s[p] = sc[kk / 32];
  }
}

}  // namespace

hipError_t launch_pack_weights(const Layout& L, const mok_weights& w, uint8_t* dst, int planes,
                               hipStream_t s) {
  PackArgs a{};
  a.wg = static_cast<const uint16_t*>(w.wg);
  a.wu = static_cast<const uint16_t*>(w.wu);
  a.wd = static_cast<const uint16_t*>(w.wd);
  a.wg_q = w.wg_q; a.wg_s = w.wg_s; a.wu_q = w.wu_q; a.wu_s = w.wu_s; a.wd_q = w.wd_q; a.wd_s = w.wd_s;
  a.wgt_q = w.wgt_q; a.wgt_s = w.wgt_s; a.wut_q = w.wut_q; a.wut_s = w.wut_s;
  a.wdt_q = w.wdt_q; a.wdt_s = w.wdt_s;
  a.dst = dst;
  a.po = pack_offsets(L.El, L.H, L.I, L.dtype);
  a.El = L.El;
  a.H = L.H;
  a.I = L.I;
  // pieces per plane (16 bytes each): gate/up and dx twice those of Wd and Wd^T
  const bool mx = L.dtype == MOK_MXFP8;
  const int64_t small = int64_t(L.El) * L.H * L.I / (mx ? 16 : 8);
  auto grid = [](int64_t pieces) { return dim3(unsigned(std::min<int64_t>((pieces + 255) / 256, 4096))); };
  if (mx) {
    if (planes & kPackGu) hipLaunchKernelGGL(k_pack_mx<0>, grid(2 * small), dim3(256), 0, s, a);
    if (planes & kPackWd) hipLaunchKernelGGL(k_pack_mx<1>, grid(small), dim3(256), 0, s, a);
    if (planes & kPackWdt) hipLaunchKernelGGL(k_pack_mx<2>, grid(small), dim3(256), 0, s, a);
    if (planes & kPackDx) hipLaunchKernelGGL(k_pack_mx<3>, grid(2 * small), dim3(256), 0, s, a);
  } else {
    if (planes & kPackGu) hipLaunchKernelGGL(k_pack_bf16<0>, grid(2 * small), dim3(256), 0, s, a);
    if (planes & kPackWd) hipLaunchKernelGGL(k_pack_bf16<1>, grid(small), dim3(256), 0, s, a);
    if (planes & kPackWdt) hipLaunchKernelGGL(k_pack_bf16<2>, grid(small), dim3(256), 0, s, a);
    if (planes & kPackDx) hipLaunchKernelGGL(k_pack_bf16<3>, grid(2 * small), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace mok
