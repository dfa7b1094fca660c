// Packing of the BF16 expert weights into the B-operand planes of the expert GEMMs, in MFMA
// fragment order (PackedB in k_gemm.h; plane offsets in pack_offsets). Run once per weight
// update (mok_pack_bf16), or by a layer call into its workspace when the caller gives none.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "mok_device.h"
#include "mok_internal.h"

namespace mok {
namespace {

struct PackArgs {
  const uint16_t *wg, *wu, *wd;   // row-major [El][I][H], [El][I][H], [El][H][I]
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

}  // namespace

hipError_t launch_pack_bf16(const Layout& L, const void* wg, const void* wu, const void* wd,
                            uint8_t* dst, int planes, hipStream_t s) {
  PackArgs a{};
  a.wg = static_cast<const uint16_t*>(wg);
  a.wu = static_cast<const uint16_t*>(wu);
  a.wd = static_cast<const uint16_t*>(wd);
  a.dst = dst;
  a.po = pack_offsets(L.El, L.H, L.I);
  a.El = L.El;
  a.H = L.H;
  a.I = L.I;
  // pieces per plane: gate/up and dx 2 El H I / 8, Wd and Wd^T El H I / 8
  const int64_t small = int64_t(L.El) * L.H * L.I / 8;
  auto grid = [](int64_t pieces) { return dim3(unsigned(std::min<int64_t>((pieces + 255) / 256, 4096))); };
  if (planes & kPackGu) hipLaunchKernelGGL(k_pack_bf16<0>, grid(2 * small), dim3(256), 0, s, a);
  if (planes & kPackWd) hipLaunchKernelGGL(k_pack_bf16<1>, grid(small), dim3(256), 0, s, a);
  if (planes & kPackWdt) hipLaunchKernelGGL(k_pack_bf16<2>, grid(small), dim3(256), 0, s, a);
  if (planes & kPackDx) hipLaunchKernelGGL(k_pack_bf16<3>, grid(2 * small), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace mok
