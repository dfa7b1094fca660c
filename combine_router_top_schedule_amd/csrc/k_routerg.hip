// The router's gate projection and its gradient.
//
// The router scores every token against every expert, logits = X W_r^T, before top-k picks the
// token's experts; in backward the router-weight gradient flows from dlogits (the top-k softmax
// backward of dp, which SwiGLU backward produces) into W_r and into the token rows ("Mixture-
// of-Kittens (MoK)", benchmark section: the router-weight gradient is computed SonicMoE-style
// and fused into SwiGLU backward; "Cursor Open-Sources Mixture-of-Kittens (MoK)", Technical
// Details).
//   forward : logits[n][e] = sum_h X[n][h] W_r[e][h]                 (fp32, [N][E])
//   backward: dW_r[e][h]   = sum_n dlogits[n][e] X[n][h]             (fp32, [E][H])
//             dX[n][h]    += sum_e dlogits[n][e] W_r[e][h]          (BF16 rows, in place)
// All three are dense contractions on the MFMA tile engine (BF16 operands, fp32 accumulation,
// no split-K, so every sum has a fixed order). Token rows are read straight from the segments;
// the backward's token-axis reduction needs X^T and dlogits^T, which are written once into the
// workspace with their token axis zero-padded to a whole K stage.
#include "k_bwd.h"

namespace mok {
namespace {

constexpr int kKStage = kStageRowBytes / 2;   // BF16 elements per K stage

struct RouterFwdArgs {
  const uint16_t* const* x_seg;
  const uint16_t* wr;      // [E][H]
  float* logits;           // [N][E]
  int H, E, T, tiles_t, tiles_e;
};

// One 256-token x 256-expert tile per workgroup; token tiles never cross a segment.
__global__ __launch_bounds__(256, 1) void k_router_logits(RouterFwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GemmLds& sm = *reinterpret_cast<GemmLds*>(smem);
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = blockIdx.x;
  const int te = q % a.tiles_e, tt = q / a.tiles_e;
  const int seg = tt / a.tiles_t, t0 = (tt % a.tiles_t) * kTileM, e0 = te * kTileN;
  const int rows = min(kTileM, a.T - t0), cols = min(kTileN, a.E - e0);
  const int row_bytes = a.H * 2;
  Operand A = operand(make_rsrc(a.x_seg[seg] + int64_t(t0) * a.H, int64_t(rows) * row_bytes),
                      row_bytes);
  Operand B = operand(make_rsrc(a.wr + int64_t(e0) * a.H, int64_t(cols) * row_bytes), row_bytes);
  f32x16 acc[4][4];
  gemm_tile<false>(sm, A, B, row_bytes / kStageRowBytes, acc, wm, wn, lane);
  store_tile_f32(sm, acc, a.logits + (int64_t(seg) * a.T + t0) * a.E + e0, a.E, rows, cols);
}

// dlogits fp32 [N][E] -> dl BF16 [N][Ep] (K = experts, zero-padded to Ep) and dl^T BF16
// [E][Np] (K = tokens, zero-padded to Np). One thread per (n, e) of the padded [Np][Ep] grid.
__global__ __launch_bounds__(256) void k_router_dl(const float* dl, uint16_t* dl16, uint16_t* dlt,
                                                   int64_t N, int E, int64_t Np, int Ep) {
  const int64_t total = Np * Ep;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t n = i / Ep;
    const int e = int(i % Ep);
    const uint16_t v = (n < N && e < E) ? f2bf(dl[n * E + e]) : uint16_t(0);
    if (n < N) dl16[n * Ep + e] = v;
    if (e < E) dlt[int64_t(e) * Np + n] = v;
  }
}

// W_r [E][H] -> W_r^T [H][Ep] (zero-padded experts). One thread per output element.
__global__ __launch_bounds__(256) void k_router_wrt(const uint16_t* wr, uint16_t* wrt, int H, int E,
                                                    int Ep) {
  const int64_t total = int64_t(H) * Ep;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int h = int(i / Ep), e = int(i % Ep);
    wrt[i] = e < E ? wr[int64_t(e) * H + h] : uint16_t(0);
  }
}

// Token rows from the segments -> X^T [H][Np] (zero-padded tokens), stored in MFMA fragment
// order (PackedB in k_gemm.h; K = the tokens), the B operand of the dW_r GEMM. Tiles of 64
// tokens x 128 features through LDS: 16-byte loads along H, 16-byte stores of 8 consecutive
// tokens of one feature (one lane's share of fragment (feature/32, token/16)).
__global__ __launch_bounds__(256) void k_router_xt(const uint16_t* const* x_seg, uint16_t* xt,
                                                   int64_t N, int T, int H, int64_t Np) {
  constexpr int kPitch = 130;
  __shared__ __attribute__((aligned(16))) uint16_t t[64 * kPitch];
  const int tid = threadIdx.x;
  const int64_t tn = Np / 64;
  const int tf = H / 128;
  for (int64_t q = blockIdx.x; q < tn * tf; q += gridDim.x) {
    const int64_t n0 = (q / tf) * 64;
    const int f0 = int(q % tf) * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, r = idx >> 4, ch = idx & 15;
      const int64_t n = n0 + r;
      u32x4 v{0u, 0u, 0u, 0u};
      if (n < N)
        v = *reinterpret_cast<const u32x4*>(x_seg[n / T] + (n % T) * int64_t(H) + f0 + ch * 8);
      uint32_t* w = reinterpret_cast<uint32_t*>(t + r * kPitch + ch * 8);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + 256 * i, c = idx >> 3, rr = idx & 7;
      u32x4 out;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        out[k] = uint32_t(t[(rr * 8 + 2 * k) * kPitch + c]) |
                 (uint32_t(t[(rr * 8 + 2 * k + 1) * kPitch + c]) << 16);
      const int fa = f0 + c;
      const int64_t col = n0 + rr * 8;
      const int64_t frag = int64_t(fa >> 5) * (Np >> 4) + (col >> 4);
      *reinterpret_cast<u32x4*>(xt + (frag * 64 + (fa & 31) + 32 * ((col >> 3) & 1)) * 8) = out;
    }
    __syncthreads();
  }
}

struct RouterBwdArgs {
  const uint16_t* dlt;     // [E][Np]
  const uint16_t* xt;      // [H][Np], fragment order
  float* dwr;              // [E][H]
  const uint16_t* dl16;    // [N][Ep]
  const uint16_t* wrt;     // [H][Ep]
  uint16_t* const* dx_seg;
  int64_t N, Np;
  int H, E, Ep, T;
  int tiles_w;             // dW_r tiles; the dX tiles follow
  int tiles_h;             // 256-column tiles of H
};

// Both backward contractions in one launch: the first tiles_w workgroups compute dW_r tiles
// (reduction over the padded token axis), the others dX tiles (reduction over the padded
// experts), whose epilogue adds the product to the BF16 dX rows in place: one rounding of
// float(dX) + sum, per element.
__global__ __launch_bounds__(256, 1) void k_router_bwd(RouterBwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  GemmLds& sm = *reinterpret_cast<GemmLds*>(smem);
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int q = blockIdx.x;
  f32x16 acc[4][4];
  if (q < a.tiles_w) {
    const int m0 = (q / a.tiles_h) * kTileM, n0 = (q % a.tiles_h) * kTileN;
    wgrad_tile<false>(sm, reinterpret_cast<const uint8_t*>(a.dlt), nullptr,
                      reinterpret_cast<const uint8_t*>(a.xt), nullptr, a.Np, 0, int(a.Np), m0, n0,
                      a.E, a.H, a.dwr);
    return;
  }
  const int r = q - a.tiles_w;
  const int64_t m0 = int64_t(r / a.tiles_h) * kTileM;
  const int n0 = (r % a.tiles_h) * kTileN;
  const int rows = int(min(int64_t(kTileM), a.N - m0)), cols = min(kTileN, a.H - n0);
  const int kb = a.Ep * 2;
  Operand A = operand(make_rsrc(a.dl16 + m0 * a.Ep, int64_t(rows) * kb), kb);
  Operand B = operand(make_rsrc(a.wrt + int64_t(n0) * a.Ep, int64_t(cols) * kb), kb);
  gemm_tile<false>(sm, A, B, kb / kStageRowBytes, acc, wm, wn, lane);
  // stage the fp32 tile in two passes of 128 rows; each lane then adds 4 columns of a row
  float* t = reinterpret_cast<float*>(sm.a[0]);
  for (int pass = 0; pass < 2; ++pass) {
    if (wm == pass) {
      float* tl = t + opaque(4 * (lane >> 5) * 256 + wn * 128 + (lane & 31));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            tl[(i * 32 + 8 * (v >> 2) + (v & 3)) * 256 + j * 32] = acc[i][j][v];
    }
    __syncthreads();
    for (int rr = wave; rr < 128; rr += 4) {
      const int m = pass * 128 + rr;
      if (m < rows && lane * 4 < cols) {
        const int64_t n = m0 + m;
        uint16_t* row = a.dx_seg[n / a.T] + (n % a.T) * int64_t(a.H) + n0 + lane * 4;
        const uint2 old = *reinterpret_cast<const uint2*>(row);
        const f32x4 add = *reinterpret_cast<const f32x4*>(t + rr * 256 + lane * 4);
        *reinterpret_cast<uint2*>(row) =
            uint2{pack_bf2(bf2f(uint16_t(old.x)) + add[0], bf2f(uint16_t(old.x >> 16)) + add[1]),
                  pack_bf2(bf2f(uint16_t(old.y)) + add[2], bf2f(uint16_t(old.y >> 16)) + add[3])};
      }
    }
    __syncthreads();
  }
}

template <class F>
hipError_t allow_big_lds(F* f) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(f),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(kGemmLdsBytes));
}

hipError_t router_init() {
  static std::atomic<bool> attr_done[kMaxDevices];
  return once_per_device(attr_done, [] {
    const hipError_t e = allow_big_lds(k_router_logits);
    return e != hipSuccess ? e : allow_big_lds(k_router_bwd);
  });
}

int grid_of(int64_t items, int per, int cap) {
  const int64_t b = (items + per - 1) / per;
  return int(b < 1 ? 1 : (b > cap ? cap : b));
}

}  // namespace

RouterWs router_ws(const Layout& L) {
  RouterWs r{};
  r.Np = align_up(L.N, kKStage);
  r.Ep = int(align_up(L.E, kKStage));
  int64_t off = 0;
  auto take = [&](int64_t bytes) { const int64_t o = off; off = align_up(off + bytes, 256); return o; };
  r.dl16 = take(L.N * r.Ep * 2);
  r.dlt = take(int64_t(L.E) * r.Np * 2);
  r.xt = take(int64_t(L.H) * r.Np * 2);
  r.wrt = take(int64_t(L.H) * r.Ep * 2);
  r.bytes = off;
  return r;
}

hipError_t launch_router_fwd(const Layout& L, const void* const* x_seg, const uint16_t* wr,
                             float* logits, hipStream_t s) {
  hipError_t err = router_init();
  if (err != hipSuccess) return err;
  RouterFwdArgs a{reinterpret_cast<const uint16_t* const*>(x_seg), wr, logits, L.H, L.E, L.T,
                  int(cdiv(L.T, kTileM)), int(cdiv(L.E, kTileN))};
  const int64_t tiles = int64_t(L.S) * a.tiles_t * a.tiles_e;
  hipLaunchKernelGGL(k_router_logits, dim3(unsigned(tiles)), dim3(kThreads), kGemmLdsBytes, s, a);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const Layout& L, const void* const* x_seg, const uint16_t* wr,
                             const float* dlogits, float* dwr, void* const* dx_seg, uint8_t* ws,
                             hipStream_t s) {
  hipError_t err = router_init();
  if (err != hipSuccess) return err;
  const RouterWs r = router_ws(L);
  uint16_t* dl16 = reinterpret_cast<uint16_t*>(ws + r.dl16);
  uint16_t* dlt = reinterpret_cast<uint16_t*>(ws + r.dlt);
  uint16_t* xt = reinterpret_cast<uint16_t*>(ws + r.xt);
  uint16_t* wrt = reinterpret_cast<uint16_t*>(ws + r.wrt);
  hipLaunchKernelGGL(k_router_dl, dim3(grid_of(r.Np * r.Ep, 256, 8192)), dim3(256), 0, s, dlogits,
                     dl16, dlt, L.N, L.E, r.Np, r.Ep);
  hipLaunchKernelGGL(k_router_wrt, dim3(grid_of(int64_t(L.H) * r.Ep, 256, 8192)), dim3(256), 0, s,
                     wr, wrt, L.H, L.E, r.Ep);
  hipLaunchKernelGGL(k_router_xt, dim3(grid_of(r.Np / 64 * (L.H / 128), 1, 8192)), dim3(256), 0, s,
                     reinterpret_cast<const uint16_t* const*>(x_seg), xt, L.N, L.T, L.H, r.Np);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  RouterBwdArgs a{};
  a.dlt = dlt; a.xt = xt; a.dwr = dwr; a.dl16 = dl16; a.wrt = wrt;
  a.dx_seg = reinterpret_cast<uint16_t* const*>(dx_seg);
  a.N = L.N; a.Np = r.Np; a.H = L.H; a.E = L.E; a.Ep = r.Ep; a.T = L.T;
  a.tiles_h = int(cdiv(L.H, kTileN));
  a.tiles_w = int(cdiv(L.E, kTileM)) * a.tiles_h;
  const int64_t tiles = a.tiles_w + cdiv(L.N, kTileM) * a.tiles_h;
  hipLaunchKernelGGL(k_router_bwd, dim3(unsigned(tiles)), dim3(kThreads), kGemmLdsBytes, s, a);
  return hipGetLastError();
}

}  // namespace mok
