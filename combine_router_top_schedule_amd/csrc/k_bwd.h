// Backward GEMM tiles: the "a" GEMM with the router-weight gradient and SwiGLU backward in its
// epilogue, the dx GEMM with the push epilogue, and the weight-gradient GEMM with an fp32
// epilogue. Same tile engine as the forward (k_gemm.h).
#pragma once

#include "k_ffn.h"

namespace mok {

// E4M3 code -> float (finite codes; the quantiser never produces NaN): gfx950's conversion
// instruction, which decodes the OCP E4M3 format (checked against the format's definition for
// all 254 finite codes).
__device__ __forceinline__ float e4m3_value(uint8_t c) {
  return __builtin_amdgcn_cvt_f32_fp8(int(c), 0);
}

// g and u of one 32-row x 128-column block of the a-GEMM epilogue, as loaded from where the
// rows live (ring slot or activation plane): 16 lanes x 16 bytes cover a row, 4 rows per load.
// Held in registers so the next block's loads are in flight while the current block is computed.
struct AStage {
  u32x4 g[8], u[8];
};

// lcode: the row-source codes of the block's 32 rows (LDS). Rows past the tile or columns past
// I load zeros (their values are never stored).
__device__ __forceinline__ void a_stage_load(AStage& st, const FfnShape& s, int64_t row0,
                                             int nrows, int colw, int rbase,
                                             const ActSource& src, const int32_t* lcode, int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rr = q * 4 + (lane >> 4), cc = (lane & 15) * 8;
    const bool ok = rbase + rr < nrows && colw + cc < s.I;
    st.g[q] = st.u[q] = u32x4{0u, 0u, 0u, 0u};
    if (ok) {
      const uint16_t* gu = act_gu_row(src, row0 + rbase + rr, lcode[rr], s.I);
      const int col = colw + cc;
      st.g[q] = *reinterpret_cast<const u32x4*>(gu + col);
      st.u[q] = *reinterpret_cast<const u32x4*>(gu + s.I + col);
    }
  }
}

// Write a loaded block into the wave's LDS region.
__device__ __forceinline__ void a_stage_store(const AStage& st, uint16_t* lg, uint16_t* lu,
                                              int lane) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int rr = q * 4 + (lane >> 4), cc = (lane & 15) * 8;
    *reinterpret_cast<u32x4*>(lg + rr * 128 + cc) = st.g[q];
    *reinterpret_cast<u32x4*>(lu + rr * 128 + cc) = st.u[q];
  }
}

// MXFP8 weight-gradient operands dg^T and du^T, written by the a-GEMM epilogue: codes
// [I][cols] blocked along tokens (32 rows of one expert per block), scales [I][cols / 32] at
// codes + I * ld. An expert's token columns start at a multiple of 128 (zero padding after its
// rows), so a 32-row block of a tile that starts inside the expert's padded range never mixes
// experts.
struct TokQuant {
  uint8_t* dg;          // codes of dg^T (scales at dg + I * ld)
  uint8_t* du;
  int64_t ld;           // host bound on the padded token columns
  int64_t cols;         // padded token columns in use (device-side total)
  int64_t colbase;      // token column of the tile's row 0
  int padlim;           // rows of the tile inside the expert's padded range
};

// Compute one staged 32-row block (i, a template argument so the accumulator stays in
// registers): dg, du, dp partials, then dg | du rows out.
// BF16: dg, du replace g, u in LDS (BF16) and leave as BF16 rows.
// MXFP8: dg and du are quantised from their fp32 values twice, with no BF16 rounding in
// between: along I for the dx GEMM (the 32 lanes of a half-wave hold one 32-column block of a
// row; codes go to the low byte of the g / u LDS slots, the block's scale code to the high
// byte of its first slot) and along tokens for the weight gradients (a column's 32 rows of the
// block sit in lanes l and l ^ 32; codes of 4 consecutive rows leave as one dword).
template <bool MX, int i>
__device__ __forceinline__ void a_epilogue_block(const f32x16 (&acc)[4][4], const FfnShape& s,
                                                 int64_t row0, int nrows, int colw,
                                                 uint16_t* dgu, uint8_t* dgq, uint8_t* dgq_s,
                                                 const TokQuant& tq, float* s_dp,
                                                 uint16_t* lg, uint16_t* lu,
                                                 const float* lpg, float* lam, int wm, int wn,
                                                 int lane) {
    const int rbase = wm * 128 + i * 32;                                // tile row of lg row 0
    float part[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) part[v] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int lc = j * 32 + (lane & 31);
      const int c = colw + lc;
      float dgr[16], dur[16], hv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int lr = acc_row(v, lane);                                // row inside the block
        const float pg = lpg[lr];
        const float av = acc[i][j][v];
        const float g = bf2f(lg[lr * 128 + lc]);
        const float u = bf2f(lu[lr * 128 + lc]);
        const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-g));
        // the forward's h, recomputed from the stored g and u: g and u are BF16 values, so
        // swiglu_bf(g, u) is g * sigmoid_hw(g) * u with sigmoid_hw(g) = sg (the same expression)
        const float hf = swiglu_of(g, sg, u);
        const float dh = pg * av;
        const float dgv = dh * u * sg * (1.f + g * (1.f - sg));
        const float duv = dh * g * sg;
        if (MX) {
          dgr[v] = dgv;
          dur[v] = duv;
          hv[v] = hf;
        } else {
          // dg and du replace g and u in place (each element is read and written by this lane);
          // the dp partial takes h as the down GEMM did, rounded to BF16
          lg[lr * 128 + lc] = f2bf(dgv);
          lu[lr * 128 + lc] = f2bf(duv);
          if (rbase + lr < nrows && c < s.I) part[v] = fmaf(av, bf2f(f2bf(hf)), part[v]);
        }
      }
      const int hw = lane >> 5;
      if (MX) {
        // Along I: the amax of each of the half-wave's 16 rows over its 32 columns (for dg, du
        // and h), by a reduce-scatter over the 32 lanes (16 exchanges per operand instead of 5
        // per element), published through the wave's 384 bytes of LDS and read back by every
        // lane.
        const float rg = half_wave_row_amax(dgr, lane), ru = half_wave_row_amax(dur, lane);
        const float rh = half_wave_row_amax(hv, lane);
        if ((lane & 1) == 0) {
          const int k = scatter_row(lane);
          lam[hw * 48 + k] = rg;
          lam[hw * 48 + 16 + k] = ru;
          lam[hw * 48 + 32 + k] = rh;
        }
        __builtin_amdgcn_wave_barrier();   // (a wave's LDS accesses complete in order)
        const uint32_t lead = (lane & 31) == 0;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = acc_row(v, lane);
          const int eg = mx_block_exp(lam[hw * 48 + v]), eu = mx_block_exp(lam[hw * 48 + 16 + v]);
          lg[lr * 128 + lc] = uint16_t((e4m3x2(dgr[v] * exp2i(-eg), 0.f) & 0xFFu) | (lead * uint32_t(eg + 127) << 8));
          lu[lr * 128 + lc] = uint16_t((e4m3x2(dur[v] * exp2i(-eu), 0.f) & 0xFFu) | (lead * uint32_t(eu + 127) << 8));
        }
      }
      if (MX) {
        // dp partial with h as the down GEMM used it: quantised along I and decoded (exact)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = acc_row(v, lane);
          const int eh = mx_block_exp(lam[hw * 48 + 32 + v]);
          const float hq = e4m3_value(uint8_t(e4m3x2(hv[v] * exp2i(-eh), 0.f) & 0xFFu)) * exp2i(eh);
          if (rbase + lr < nrows && c < s.I) part[v] = fmaf(acc[i][j][v], hq, part[v]);
        }
        __builtin_amdgcn_wave_barrier();   // lam is rewritten for the next j

        // Along tokens: this lane holds rows 8t + 4h + (0..3), t = 0..3, h = lane / 32, of
        // column c; lane ^ 32 the others. Rows past the tile's valid rows hold 0 (zero operand
        // rows, zero gate), which is the padding of the expert's last block.
        float ag = 0.f, au = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          ag = fmaxf(ag, fabsf(dgr[v]));
          au = fmaxf(au, fabsf(dur[v]));
        }
        ag = fmaxf(ag, __uint_as_float(xchg32(__float_as_uint(ag), lane)));
        au = fmaxf(au, __uint_as_float(xchg32(__float_as_uint(au), lane)));
        const int eg = mx_block_exp(ag), eu = mx_block_exp(au);
        const float ig = exp2i(-eg), iu = exp2i(-eu);
        // Codes of rows 8t + 4h .. +3 as dword t; the two lanes of a column swap two dwords so
        // lane h holds rows 16h .. 16h+15 in order and writes them with one 16-byte store.
        uint32_t wg4[4], wu4[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          wg4[t] = e4m3x2(dgr[4 * t] * ig, dgr[4 * t + 1] * ig) | (e4m3x2(dgr[4 * t + 2] * ig, dgr[4 * t + 3] * ig) << 16);
          wu4[t] = e4m3x2(dur[4 * t] * iu, dur[4 * t + 1] * iu) | (e4m3x2(dur[4 * t + 2] * iu, dur[4 * t + 3] * iu) << 16);
        }
        const bool hi = (lane >> 5) != 0;
        const uint32_t g0 = xchg32(hi ? wg4[0] : wg4[2], lane);
        const uint32_t g1 = xchg32(hi ? wg4[1] : wg4[3], lane);
        const uint32_t u0 = xchg32(hi ? wu4[0] : wu4[2], lane);
        const uint32_t u1 = xchg32(hi ? wu4[1] : wu4[3], lane);
        const u32x4 og = hi ? u32x4{g0, wg4[2], g1, wg4[3]} : u32x4{wg4[0], g0, wg4[1], g1};
        const u32x4 ou = hi ? u32x4{u0, wu4[2], u1, wu4[3]} : u32x4{wu4[0], u0, wu4[1], u1};
        if (c < s.I && rbase < tq.padlim) {
          const int64_t col = tq.colbase + rbase;
          *reinterpret_cast<u32x4*>(tq.dg + int64_t(c) * tq.cols + col + 16 * (lane >> 5)) = og;
          *reinterpret_cast<u32x4*>(tq.du + int64_t(c) * tq.cols + col + 16 * (lane >> 5)) = ou;
          if (lane < 32) {
            tq.dg[int64_t(s.I) * tq.ld + int64_t(c) * (tq.cols / 32) + col / 32] = uint8_t(eg + 127);
            tq.du[int64_t(s.I) * tq.ld + int64_t(c) * (tq.cols / 32) + col / 32] = uint8_t(eu + 127);
          }
        }
      }
    }
    // dp partials: sum over the 32 columns of this half-wave, by a reduce-scatter (a fixed
    // order), then the two wn waves' halves are added when the tile's partials leave
    {
      const float pv = half_wave_row_reduce<false>(part, lane);
      if ((lane & 1) == 0) s_dp[wn * 256 + rbase + acc_row(scatter_row(lane), lane)] = pv;
    }
    // (a wave's LDS accesses complete in order: no wait before reading dg | du back)
    __builtin_amdgcn_wave_barrier();
    // dg | du rows out with 16-byte stores (BF16) or 8-byte code stores (MXFP8), 16 lanes per row.
    // BF16 stores go through a buffer resource over the tile's valid rows of this wave's columns
    // (empty when they lie past I), which drops the rest: every wave issues exactly 16 stores, so
    // the compiler's wait before the next block's staged g, u is for those loads alone.
    __amdgpu_buffer_rsrc_t orsrc;
    if (!MX)
      orsrc = make_rsrc(dgu + row0 * 2 * s.I,
                        colw < s.I ? int64_t(nrows) * 2 * s.I * 2 : int64_t(0));
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rr = q * 4 + (lane >> 4), cc = (lane & 15) * 8;
      const bool wr = rbase + rr < nrows && colw + cc < s.I;
      const u32x4 gv = *reinterpret_cast<const u32x4*>(lg + rr * 128 + cc);
      const u32x4 uv = *reinterpret_cast<const u32x4*>(lu + rr * 128 + cc);
      const int64_t row = row0 + rbase + rr;
      if (!MX) {
        const int off = ((rbase + rr) * 2 * s.I + colw + cc) * 2;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, gv), orsrc, off, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, uv), orsrc, off + s.I * 2,
                                               0, 0);
        continue;
      }
      if (!wr) continue;
      if (MX) {
        // low bytes of the 8 slots are the codes; the first slot of a 32-column block also
        // carries the block's scale code in its high byte
        auto codes = [](const u32x4& w) {
          return uint2{(w[0] & 0xFFu) | ((w[0] >> 8) & 0xFF00u) | ((w[1] & 0xFFu) << 16) | ((w[1] & 0xFF0000u) << 8),
                       (w[2] & 0xFFu) | ((w[2] >> 8) & 0xFF00u) | ((w[3] & 0xFFu) << 16) | ((w[3] & 0xFF0000u) << 8)};
        };
        *reinterpret_cast<uint2*>(dgq + row * 2 * s.I + colw + cc) = codes(gv);
        *reinterpret_cast<uint2*>(dgq + row * 2 * s.I + s.I + colw + cc) = codes(uv);
        if ((lane & 3) == 0) {
          dgq_s[row * (2 * s.I / 32) + (colw + cc) / 32] = uint8_t(gv[0] >> 8);
          dgq_s[row * (2 * s.I / 32) + (s.I + colw + cc) / 32] = uint8_t(uv[0] >> 8);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }

// a = D Wd_e for the 256 intermediate columns [c0, c0+256) of expert e, rows [row0, row0+nrows)
// of the expert-ordered stream (plane rows of `act` and of D). Epilogue per element (row, i):
//   dh = p a, dg = dh u s(g) (1 + g (1 - s(g))), du = dh g s(g)     -> dgu[row][i], [I + i]
//     (MXFP8: codes dgq[row][i], [I + i] blocked along I, and dg^T, du^T blocked along tokens)
//   dp partial = sum over this tile's columns of a h (fixed tree)   -> dp_part[row][c0/256]
// The epilogue's LDS carve-out is laid out for exactly 4 waves: 16 KB per wave in the first
// three stage buffers, dp partials, gates, row-source codes and (MXFP8) the row amaxes along I
// in the fourth.
static_assert(kThreads == 256, "a_tile's LDS regions assume 4 waves");
static_assert(4 * 16384 <= 3 * kStageBytes, "per-wave regions must end before the fourth stage buffer");
static_assert(6144 + 4 * 128 * 4 <= 8192, "dp partials, gates and codes end before the amaxes");
static_assert(8192 + 4 * 96 * 4 <= kStageBytes, "the row amaxes fit the fourth stage buffer");
template <bool MX>
__device__ __forceinline__ void a_tile(GemmLds& sm, const FfnShape& s, int64_t row0, int nrows,
                                       int e, int c0, const uint8_t* d, const uint8_t* d_s,
                                       const uint8_t* wdt, const uint8_t* wdt_s,
                                       const ActSource& act, const int32_t* perm, const float* p,
                                       uint16_t* dgu, uint8_t* dgq, uint8_t* dgq_s,
                                       const TokQuant& tq, float* dp_part) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int eb = MX ? 1 : 2;
  const int xrow = s.H * eb;
  const int ncols = min(kTileN, s.I - c0);
  Operand A = operand(make_rsrc(d + row0 * xrow, int64_t(nrows) * xrow), xrow);
  const int64_t wrow0 = int64_t(e) * s.I + c0;
  if (MX) {
    A.sstride = s.H / 32;
    A.s0 = A.s1 = make_rsrc(d_s + row0 * (s.H / 32), int64_t(nrows) * (s.H / 32));
  }
  // B: the packed Wd^T plane (MXFP8: codes wdt, scales wdt_s)
  f32x16 acc[4][4];
  if constexpr (MX)
    gemm_tile_pb_mx(sm, A, packed_b_mx(wdt, wdt_s, wrow0, ncols, s.H), xrow / kStageRowBytes,
                    acc, wm, wn, lane);
  else
    gemm_tile_pb(sm, A, packed_b(wdt, wrow0, ncols, s.H), xrow / kStageRowBytes, acc, wm, wn,
                 lane);

  // Epilogue. For each 32-row block i, every wave first copies the g, u and h values of its
  // 32 rows x 128 columns into its own LDS region with coalesced 16-byte loads (all issued
  // together), then forms dg, du and the dp partials from LDS. h is staged as fp32 (MXFP8 h is
  // decoded on the way).
  const int nparts = (s.I + kTileN - 1) / kTileN;
  float* s_dp = reinterpret_cast<float*>(sm.b[1]);                      // [2][256]
  uint8_t* wreg = sm.a[0] + wave * 16384;                               // 16 KB per wave
  uint16_t* lg = reinterpret_cast<uint16_t*>(wreg);                     // [32][128] BF16
  uint16_t* lu = lg + 32 * 128;
  const int colw = c0 + wn * 128;                                       // wave's first column
  float* lpg = reinterpret_cast<float*>(sm.b[1] + 4096) + wave * 128;    // gates of the wave's rows
  int32_t* lcode = reinterpret_cast<int32_t*>(sm.b[1] + 6144) + wave * 128;  // their sources
  float* lam = reinterpret_cast<float*>(sm.b[1] + 8192) + wave * 96;   // MXFP8 row amaxes along I
  // gates and row-source codes of the wave's 128 rows (lane l: row wm*128 + l, l < 128 over
  // two halves)
  for (int l = lane; l < 128; l += 64) {
    const int r = wm * 128 + l;
    lpg[l] = r < nrows ? p[perm[row0 + r]] : 0.f;
    lcode[l] = r < nrows ? act.code[row0 + r] : -1;
  }
  __builtin_amdgcn_wave_barrier();
  AStage st;
  a_stage_load(st, s, row0, nrows, colw, wm * 128, act, lcode, lane);
#define MOK_A_BLOCK(I_)                                                                          \
  {                                                                                              \
    if (MX) __builtin_amdgcn_s_waitcnt(0);                                                       \
    a_stage_store(st, lg, lu, lane);                                                             \
    if (I_ < 3) a_stage_load(st, s, row0, nrows, colw, wm * 128 + (I_ + 1) * 32, act,             \
                             lcode + (I_ + 1) * 32, lane);                                       \
    __builtin_amdgcn_wave_barrier();                                                             \
    a_epilogue_block<MX, I_>(acc, s, row0, nrows, colw, dgu, dgq, dgq_s, tq, s_dp, lg, lu,        \
                             lpg + I_ * 32, lam, wm, wn, lane);                                  \
  }
  MOK_A_BLOCK(0)
  MOK_A_BLOCK(1)
  MOK_A_BLOCK(2)
  MOK_A_BLOCK(3)
#undef MOK_A_BLOCK
  __syncthreads();
  for (int r = tid; r < nrows; r += blockDim.x)
    dp_part[(row0 + r) * nparts + c0 / kTileN] = s_dp[r] + s_dp[256 + r];
  __syncthreads();
}

// dx = [dg | du] [Wg_e ; Wu_e] for output columns [c0, c0+256) of H: A = dg|du rows (K = 2I),
// B = rows h of Wg_e^T for the first I of K and of Wu_e^T for the second; pushed to the slots.
template <bool MX>
__device__ __forceinline__ void dx_tile(GemmLds& sm, const FfnShape& s, int64_t row0, int nrows,
                                        int e, int c0, const uint8_t* dgu, const uint8_t* dgu_s,
                                        const uint8_t* wgt, const uint8_t* wgt_s,
                                        const PushTarget& pt) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int eb = MX ? 1 : 2;
  const int arow = 2 * s.I * eb;
  const int ncols = min(kTileN, s.H - c0);
  Operand A = operand(make_rsrc(dgu + row0 * arow, int64_t(nrows) * arow), arow);
  const int64_t wrow0 = int64_t(e) * s.H + c0;
  f32x16 acc[4][4];
  // B: the packed [Wg^T | Wu^T] plane (K = 2I; MXFP8: codes wgt, scales wgt_s)
  if constexpr (MX) {
    A.sstride = 2 * s.I / 32;
    A.s0 = A.s1 = make_rsrc(dgu_s + row0 * A.sstride, int64_t(nrows) * A.sstride);
    gemm_tile_pb_mx(sm, A, packed_b_mx(wgt, wgt_s, wrow0, ncols, 2 * s.I), arow / kStageRowBytes,
                    acc, wm, wn, lane);
  } else {
    gemm_tile_pb(sm, A, packed_b(wgt, wrow0, ncols, 2 * s.I), arow / kStageRowBytes, acc, wm, wn,
                 lane);
  }
  push_epilogue<kPushRec>(sm, acc, nrows, c0, s.H, 0, pt, row0);
}

// Write an fp32 tile: out[m * ld + n] = acc for m < ma, n < nb. The tile leaves through LDS in
// two passes of 128 rows: the two waves holding those rows (wm == pass) stage their 128 x 128
// blocks in the stage buffers ([128][256] fp32, 128 KB), then every wave writes whole 1 KB rows
// with 16-byte stores (storing 4 bytes per lane straight from the accumulators is many times
// slower when many tiles end together). nb and ld are multiples of 4, so a lane's 4 columns
// are all in range or all out. The caller's K loop has ended (stage buffers free).
__device__ __forceinline__ void store_tile_f32(GemmLds& sm, const f32x16 (&acc)[4][4], float* out,
                                               int64_t ld, int ma, int nb) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
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
    for (int r = wave; r < 128; r += 4) {
      const int m = pass * 128 + r;
      if (m < ma && lane * 4 < nb)
        *reinterpret_cast<f32x4*>(out + int64_t(m) * ld + lane * 4) =
            *reinterpret_cast<const f32x4*>(t + r * 256 + lane * 4);
    }
    __syncthreads();
  }
}

// Weight-gradient tile: out[m0 + m][n0 + n] = sum over the expert's padded columns c of
// Ta[m0 + m][c] Tb[n0 + n][c]; fp32 output [Fa][Fb] (fully overwritten). ld = row pitch of Ta
// and Tb (elements; the MXFP8 scale rows of Ta have ld / 32 bytes). Tb is packed in fragment
// order with ld columns (K = the padded columns; MXFP8: its scale plane at tb_s), read straight
// into registers.
template <bool MX>
__device__ __forceinline__ void wgrad_tile(GemmLds& sm, const uint8_t* ta, const uint8_t* ta_s,
                                           const uint8_t* tb, const uint8_t* tb_s, int64_t ld,
                                           int c0, int ncols, int m0, int n0, int Fa, int Fb,
                                           float* out) {
  const int tid = tile_tid(), lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int eb = MX ? 1 : 2;
  const int64_t stride = ld * eb;
  const int ma = min(kTileM, Fa - m0), nb = min(kTileN, Fb - n0);
  f32x16 acc[4][4];
  if (ncols > 0) {
    Operand A = operand(make_rsrc(ta + int64_t(m0) * stride + int64_t(c0) * eb, int64_t(ma) * stride),
                        int(stride));
    if (MX) {
      A.sstride = int(ld / 32);
      A.s0 = A.s1 = make_rsrc(ta_s + int64_t(m0) * (ld / 32) + c0 / 32, int64_t(ma) * (ld / 32));
    }
    if constexpr (MX) {
      // packed codes: fragment (n32, k64) at (n32 * ld/64 + k64) * 2 KB; scales 64 bytes each
      const int k64s = int(ld / 64);
      const int64_t f0 = int64_t(n0 / 32) * k64s + c0 / 64;
      const int64_t nf = int64_t(nb / 32 - 1) * k64s + ncols / 64;
      PackedBMX P;
      P.r = make_rsrc(tb + f0 * 2048, nf * 2048);
      P.s = make_rsrc(tb_s + f0 * 64, nf * 64);
      P.k64s = k64s;
      gemm_tile_pb_mx(sm, A, P, ncols * eb / kStageRowBytes, acc, wm, wn, lane);
    } else {
      // fragment (n32, k16) of the packed plane at (n32 * ld/16 + k16) KB; the resource covers
      // the tile's nb rows over the expert's columns [c0, c0 + ncols)
      const int k16s = int(ld / 16);
      PackedB P;
      P.r = make_rsrc(tb + (int64_t(n0 / 32) * k16s + c0 / 16) * 1024,
                      (int64_t(nb / 32 - 1) * k16s + ncols / 16) * 1024);
      P.k16s = k16s;
      gemm_tile_pb(sm, A, P, ncols * eb / kStageRowBytes, acc, wm, wn, lane);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  }
  store_tile_f32(sm, acc, out + int64_t(m0) * Fb + n0, Fb, ma, nb);
}

}  // namespace mok
