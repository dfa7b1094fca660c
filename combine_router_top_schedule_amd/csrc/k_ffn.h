// Expert FFN tiles: gate/up GEMM with the SwiGLU epilogue, and the down GEMM with the push
// epilogue that writes each result row into its token's receive slot. Used by the staged
// kernels (k_ffn.hip) and by the fused persistent forward.
#pragma once

#include "k_gemm.h"

namespace mok {

// Packed expert weights (pack_offsets): BF16 values, or MXFP8 codes with their scale planes.
struct FfnWeights {
  const uint8_t* pgu;     // gate/up plane
  const uint8_t* pgu_s;   // MXFP8: its scales
  const uint8_t* pwd;     // Wd plane
  const uint8_t* pwd_s;   // MXFP8: its scales
};

// The FFN weights of a call: the packed planes at w.packed.
inline FfnWeights ffn_weights(const Layout& L, const mok_weights& w) {
  const PackOffsets po = pack_offsets(L.El, L.H, L.I, L.dtype);
  const uint8_t* pk = static_cast<const uint8_t*>(w.packed);
  const bool mx = L.dtype == MOK_MXFP8;
  return FfnWeights{pk + po.gu, mx ? pk + po.gu_s : nullptr, pk + po.wd, mx ? pk + po.wd_s : nullptr};
}

struct FfnShape {
  int H, I;
};

// Cross-lane moves without LDS (gfx950): the value of lane l ^ 32 (a permlane32 swap), and a
// DPP read of another lane of the same 16-lane row (CTRL: 0x128 row_ror:8 = lane ^ 8,
// 0x141 row_half_mirror = lane ^ 7 within 8, 0x4E / 0xB1 quad_perm = lane ^ 2 / lane ^ 1).
__device__ __forceinline__ uint32_t xchg32(uint32_t v, int lane) {
  const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return lane < 32 ? s[1] : s[0];
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Reduce-scatter of x over the 32 lanes of a half-wave: lane l holds 16 values x[v] (one per
// accumulator row v, its own column); on return it holds, for the row index
// scatter_row(l) = 8 b4 + 4 b3 + 2 b2 + b1 (b = bits of l), the largest |x| (MAXABS) or the
// sum of x over all 32 lanes of its half-wave, in a fixed order (lanes l and l ^ 1 hold the
// same row and the same bits). Five halving steps, each with the
// lane that differs in that step's bit: l ^ 16 (a permlane16 swap exchanges the two halves in
// one move), l ^ 8, l ^ 7 (its bits 3 and 4 agree with l's, bit 2 differs), l ^ 2, l ^ 1 (DPP);
// together they reach all 32 lanes.
__device__ __forceinline__ int scatter_row(int lane) {
  return ((lane >> 4) & 1) * 8 + ((lane >> 3) & 1) * 4 + ((lane >> 2) & 1) * 2 + ((lane >> 1) & 1);
}
template <bool MAXABS>
__device__ __forceinline__ float half_wave_row_reduce(const float (&x)[16], int lane) {
  auto op = [](float a, float b) { return MAXABS ? fmaxf(a, b) : a + b; };
  float m8[8], m4[4], m2[2];
  const bool b4 = (lane >> 4) & 1, b3 = (lane >> 3) & 1, b2 = (lane >> 2) & 1, b1 = (lane >> 1) & 1;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    // lanes of the lower 16-lane row keep row k and get it from l ^ 16; the upper row keeps k + 8
    const float lo = MAXABS ? fabsf(x[k]) : x[k], hi = MAXABS ? fabsf(x[k + 8]) : x[k + 8];
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi),
                                                    false, false);
    // (own value first, the partner's second, in every lane)
    m8[k] = b4 ? op(__uint_as_float(r[1]), __uint_as_float(r[0]))
               : op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float keep = b3 ? m8[k + 4] : m8[k], send = b3 ? m8[k] : m8[k + 4];
    m4[k] = op(keep, dpp_f<0x128>(send));
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const float keep = b2 ? m4[k + 2] : m4[k], send = b2 ? m4[k] : m4[k + 2];
    m2[k] = op(keep, dpp_f<0x141>(send));
  }
  const float keep = b1 ? m2[1] : m2[0], send = b1 ? m2[0] : m2[1];
  const float m1 = op(keep, dpp_f<0x4E>(send));
  // the pair's two lanes add in the same order (lower lane's value first) so both hold the same
  // bits
  const float other = dpp_f<0xB1>(m1);
  return (lane & 1) ? op(other, m1) : op(m1, other);
}
__device__ __forceinline__ float half_wave_row_amax(const float (&x)[16], int lane) {
  return half_wave_row_reduce<true>(x, lane);
}

// SwiGLU of the stored (BF16-rounded) g and u, h = g s(g) u with s(g) = 1 / (1 + e^-g) from the
// hardware exp and reciprocal: the forward and the backward's recomputation (which needs s(g)
// for dg and du anyway) form h with these same instructions, so they agree bit for bit.
// (Neither has an add fed by a multiply, so no context can fuse two of their operations.)
__device__ __forceinline__ float sigmoid_hw(float g) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-g));
}
__device__ __forceinline__ float swiglu_of(float gb, float sg, float ub) {
  return gb * sg * ub;
}
__device__ __forceinline__ float swiglu_bf(float g, float u) {
  const float gb = bf2f(f2bf(g)), ub = bf2f(f2bf(u));
  return swiglu_of(gb, sigmoid_hw(gb), ub);
}

// g|u = x [Wg;Wu]^T over the 128 h-columns [i0, i0+128) of expert e; SwiGLU h = silu(g) u of
// the BF16-rounded g and u. B tile rows interleave 64-row blocks of Wg and Wu (block q even:
// Wg, odd: Wu, both for i = i0 + (q/2)*64 + row%64), so wave (wm, wn) holds g in column
// blocks 0,1 and the matching u in column blocks 2,3, lane for lane.
// before_h() runs (workgroup-uniform) after g|u is stored and before h is; when it returns
// false the tile stops there and returns false (the fused forward waits there for h's slot).
struct AlwaysReady {
  __device__ bool operator()() const { return true; }
};
template <bool MX, class BeforeH = AlwaysReady>
__device__ __forceinline__ bool gateup_tile(GemmLds& sm, const FfnShape& s, const FfnWeights& w,
                                            const ActPlanes& pl, int64_t prow0, int nrows, int e,
                                            int i0, BeforeH before_h = BeforeH()) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int eb = MX ? 1 : 2;                              // bytes per element
  const int xrow = s.H * eb;
  Operand A;
  A.interleave = 0;
  A.ksplit = 0x7FFFFFFF;
  A.stride = xrow;
  A.sstride = s.H / 32;
  A.r0 = A.r1 = make_rsrc(pl.x + prow0 * xrow, int64_t(nrows) * xrow);
  f32x16 acc[4][4];
  // the packed gate/up plane holds the tile's 256 B rows in this order, from row 2 i0 of the
  // expert's 2I rows
  const int64_t brow0 = int64_t(e) * 2 * s.I + 2 * int64_t(i0);
  if constexpr (MX) {
    A.s0 = A.s1 = make_rsrc(pl.xs + prow0 * A.sstride, int64_t(nrows) * A.sstride);
    gemm_tile_pb_mx(sm, A, packed_b_mx(w.pgu, w.pgu_s, brow0, kTileN, s.H),
                    xrow / kStageRowBytes, acc, wm, wn, lane);
  } else {
    gemm_tile_pb(sm, A, packed_b(w.pgu, brow0, kTileN, s.H), xrow / kStageRowBytes, acc, wm, wn,
                 lane);
  }

  // SwiGLU epilogue. Column blocks (jg, jg+2) = (g, u) of h-column i0 + wn*64 + jg*32 + lane%32.
  // The K loop ended on a barrier, so the whole 128 KB of stage buffers is free: stage the
  // BF16 g|u tile as [256 rows][g 128 | u 128], write it out row by row with 16-byte stores,
  // then do the same for h.
  uint16_t* t = reinterpret_cast<uint16_t*>(sm.a[0]);
  {
    // lane-dependent part of the staging address; the rest are immediate offsets
    uint16_t* tl = t + opaque((wm * 128 + 4 * (lane >> 5)) * 256 + wn * 64 + (lane & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jg = 0; jg < 2; ++jg)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int ro = (i * 32 + 8 * (v >> 2) + (v & 3)) * 256 + jg * 32;
          tl[ro] = f2bf(acc[i][jg][v]);
          tl[ro + 128] = f2bf(acc[i][jg + 2][v]);
        }
  }
  __syncthreads();
  {
    // 32 lanes per row (512 B), two rows per wave per step.
    const int half = lane >> 5, c = lane & 31;
    for (int r = wave * 2 + half; r < nrows; r += 8) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(t + r * 256 + c * 8);
      uint16_t* dst = pl.gu + (prow0 + r) * 2 * s.I + (c < 16 ? i0 + c * 8 : s.I + i0 + (c - 16) * 8);
      *reinterpret_cast<u32x4*>(dst) = val;
    }
  }
  __syncthreads();
  if (!before_h()) return false;
  uint8_t* tb = sm.a[0];
  uint32_t* ts = reinterpret_cast<uint32_t*>(sm.b[0]);   // MXFP8 scales, one word per row
  const int rl = opaque(wm * 128 + 4 * (lane >> 5));
  const int cl = opaque(wn * 64 + (lane & 31));
  // MXFP8: h is quantised along I; the 32 lanes of a half-wave hold one 32-column block of 16
  // rows. The rows' amaxes come from a reduce-scatter over the half-wave, published through
  // 128 bytes of the wave's LDS (in the fourth stage buffer, free in this phase).
  float* lam = reinterpret_cast<float*>(sm.b[1]) + wave * 32;
  const int hw = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int jg = 0; jg < 2; ++jg) {
      const int col = cl + jg * 32;
      float hv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) hv[v] = swiglu_bf(acc[i][jg][v], acc[i][jg + 2][v]);
      if (MX) {
        const float rh = half_wave_row_amax(hv, lane);
        if ((lane & 1) == 0) lam[hw * 16 + scatter_row(lane)] = rh;
        __builtin_amdgcn_wave_barrier();   // (a wave's LDS accesses complete in order)
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = rl + i * 32 + 8 * (v >> 2) + (v & 3);
        if (MX) {
          const int ex = mx_block_exp(lam[hw * 16 + v]);
          tb[r * 128 + col] = uint8_t(e4m3x2(hv[v] * exp2i(-ex), 0.f) & 0xFFu);
          if ((lane & 31) == 0) reinterpret_cast<uint8_t*>(ts)[r * 4 + (col >> 5)] = uint8_t(ex + 127);
        } else {
          t[r * 128 + col] = f2bf(hv[v]);
        }
      }
      if (MX) __builtin_amdgcn_wave_barrier();   // lam is rewritten for the next block
    }
  __syncthreads();
  if (MX) {
    // 8 lanes per row (128 B of codes); the row's 4 scale bytes by lane 0 of the group.
    const int sub = lane >> 3, c = lane & 7;
    for (int r = wave * 8 + sub; r < nrows; r += 32) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(tb + r * 128 + c * 16);
      *reinterpret_cast<u32x4*>(pl.h + (prow0 + r) * s.I + i0 + c * 16) = val;
      if (c == 0)
        *reinterpret_cast<uint32_t*>(pl.hs + (prow0 + r) * (s.I / 32) + i0 / 32) = ts[r];
    }
  } else {
    // 16 lanes per row (256 B).
    const int sub = lane >> 4, c = lane & 15;
    for (int r = wave * 4 + sub; r < nrows; r += 16) {
      const u32x4 val = *reinterpret_cast<const u32x4*>(t + r * 128 + c * 8);
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(pl.h) + (prow0 + r) * s.I + i0 + c * 8) = val;
    }
  }
  __syncthreads();
  return true;
}

// Where the push epilogue sends a tile's rows. kPushSlots: every row raw to slots[pair], the
// pair ids coming from the caller. kPushRec: per the rows' push records (PushRec), which send
// a token's only local pair straight to its output row.
enum PushMode : int { kPushSlots = 0, kPushRec = 1 };

struct PushTarget {
  uint16_t* slots;
  const PushRec* rec;   // [rows], kPushRec
};

// Push epilogue shared by the down GEMM and the dx GEMM: stage the BF16 tile in LDS, then
// write whole rows (512 B, 16 B per lane) to each row's destination (see PushTarget).
// kPushSlots: `my_pair` is the pair id of tile row threadIdx.x, loaded by the caller before the
// K loop so its latency is hidden. kPushRec: the row's record is loaded here, unconditionally
// (clamped row index), and first used after the LDS staging, so its latency is hidden there;
// nothing of it is live across the K loop.
// The epilogue keeps one destination pointer and one weight per thread in the MXFP8 scale
// buffers, and the BF16 tile in the stage buffers.
static_assert(kThreads * sizeof(void*) <= sizeof(GemmLds::as), "push destinations fit as[]");
static_assert(kThreads * sizeof(float) <= sizeof(GemmLds::bs[0]), "push weights fit bs[0]");
static_assert(kTileM * kTileN * 2 <= 4 * kStageBytes, "BF16 tile fits the stage buffers");

template <int MODE>
__device__ __forceinline__ void push_epilogue(GemmLds& sm, const f32x16 (&acc)[4][4], int nrows,
                                              int c0, int H, int32_t my_pair,
                                              const PushTarget& pt, int64_t row0) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  uint16_t* t = reinterpret_cast<uint16_t*>(sm.a[0]);
  uint16_t** s_dst = reinterpret_cast<uint16_t**>(sm.as[0]);
  float* s_w = reinterpret_cast<float*>(sm.bs[0]);
  PushRec rec{};
  if (MODE == kPushRec) rec = pt.rec[row0 + min(tid, nrows - 1)];
  {
    uint16_t* tl = t + opaque((wm * 128 + 4 * (lane >> 5)) * 256 + wn * 128 + (lane & 31));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          tl[(i * 32 + 8 * (v >> 2) + (v & 3)) * 256 + j * 32] = f2bf(acc[i][j][v]);
  }
  s_dst[tid] = MODE == kPushRec ? rec.dst : pt.slots + int64_t(my_pair) * H;
  s_w[tid] = MODE == kPushRec ? rec.w : -1.f;
  __syncthreads();
  {
    const int half = lane >> 5, c = lane & 31;
    const bool colok = c0 + c * 8 < H;
    for (int r = wave * 2 + half; r < nrows; r += 8) {
      uint16_t* d = s_dst[r];
      const float rw = s_w[r];
      u32x4 val = *reinterpret_cast<const u32x4*>(t + r * 256 + c * 8);
      if (rw >= 0.f) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          val[i] = pack_bf2(fmaf(rw, __uint_as_float(val[i] << 16), 0.f),
                            fmaf(rw, __uint_as_float(val[i] & 0xFFFF0000u), 0.f));
      }
      // The pointer came through LDS: name its address space, or the store becomes a flat
      // store, which every later LDS read would wait for.
      typedef __attribute__((address_space(1))) u32x4 global_u32x4;
      if (colok) *(global_u32x4*)(d + c0 + c * 8) = val;
    }
  }
  __syncthreads();
}

// y = h Wd^T over the 256 output columns [c0, c0+256) of expert e; the epilogue pushes each
// row to its token's receive slot, slots[perm[row]][c] = bf16(y), or (kPushRec: a token's only
// local pair) writes the token's output row.
template <bool MX, int MODE>
__device__ __forceinline__ void down_tile(GemmLds& sm, const FfnShape& s, const FfnWeights& w,
                                          const ActPlanes& pl, int64_t prow0, int64_t row0,
                                          int nrows, int e, int c0, const int32_t* perm,
                                          const PushTarget& pt) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int eb = MX ? 1 : 2;
  const int hrow = s.I * eb;
  Operand A;
  A.interleave = 0;
  A.ksplit = 0x7FFFFFFF;
  A.stride = hrow;
  A.sstride = s.I / 32;
  A.r0 = A.r1 = make_rsrc(pl.h + prow0 * hrow, int64_t(nrows) * hrow);
  const int ncols = min(kTileN, s.H - c0);
  const int64_t wrow0 = int64_t(e) * s.H + c0;
  const int32_t my_pair = MODE == kPushSlots && tid < nrows ? perm[row0 + tid] : 0;
  f32x16 acc[4][4];
  if constexpr (MX) {
    A.s0 = A.s1 = make_rsrc(pl.hs + prow0 * A.sstride, int64_t(nrows) * A.sstride);
    gemm_tile_pb_mx(sm, A, packed_b_mx(w.pwd, w.pwd_s, wrow0, ncols, s.I), hrow / kStageRowBytes,
                    acc, wm, wn, lane);
  } else {
    gemm_tile_pb(sm, A, packed_b(w.pwd, wrow0, ncols, s.I), hrow / kStageRowBytes, acc, wm, wn,
                 lane);
  }

  push_epilogue<MODE>(sm, acc, nrows, c0, s.H, my_pair, pt, row0);
}

}  // namespace mok
