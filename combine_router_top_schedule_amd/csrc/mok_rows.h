// Per-row device routines shared by the staged kernels and the fused persistent kernels.
// A whole wave (64 lanes) works on one row; lanes take consecutive 16-byte chunks. Source rows
// are read once, so they are loaded non-temporally: on MI355X a row gather runs at ~6.3 TB/s
// that way against ~4.8 TB/s with default loads (measured with 14 KB rows, 16 K rows).
#pragma once

#include "mok_device.h"
#include "mok_internal.h"

namespace mok {

// Copy one BF16 row of H elements (src == nullptr writes zeros). Up to 16 chunks of 16 bytes
// per lane are loaded before any is stored, so a wave keeps a whole 16 KB row in flight.
__device__ __forceinline__ void copy_row_bf16(const uint16_t* src, uint16_t* dst, int H, int lane) {
  const int nch = H / 8;
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  for (int c0 = 0; c0 < nch; c0 += 64 * 16) {
    u32x4 v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int c = c0 + q * 64 + lane;
      v[q] = (src && c < nch) ? __builtin_nontemporal_load(s + c) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int c = c0 + q * 64 + lane;
      if (c < nch) d[c] = v[q];
    }
  }
}

// Rows of at most 64 x 16 chunks of 16 bytes (H <= 8192 BF16) fit one register batch per lane.
constexpr int kRowBatchChunks = 64 * 16;

// (src == nullptr loads zeros)
__device__ __forceinline__ void load_row16(const uint16_t* src, u32x4 (&v)[16], int nch, int lane) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int c = q * 64 + lane;
    v[q] = (src && c < nch) ? __builtin_nontemporal_load(s + c) : u32x4{0, 0, 0, 0};
  }
}

__device__ __forceinline__ void store_row16(uint16_t* dst, const u32x4 (&v)[16], int nch, int lane) {
  u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int c = q * 64 + lane;
    if (c < nch) d[c] = v[q];
  }
}

// Copy rows j = 0 .. nrows-1 of BF16 (H <= 8192 elements) from src_of(j) to dst_of(j), keeping
// two rows in flight per wave: row j+1 is loaded before row j is stored.
template <class Src, class Dst>
__device__ __forceinline__ void copy_rows_bf16_2(int nrows, int H, int lane, Src src_of, Dst dst_of) {
  const int nch = H / 8;
  u32x4 va[16], vb[16];
  if (nrows <= 0) return;
  load_row16(src_of(0), va, nch, lane);
  for (int j = 0;; j += 2) {
    const bool has1 = j + 1 < nrows;
    if (has1) load_row16(src_of(j + 1), vb, nch, lane);
    store_row16(dst_of(j), va, nch, lane);
    if (!has1) break;
    const bool has2 = j + 2 < nrows;
    if (has2) load_row16(src_of(j + 2), va, nch, lane);
    store_row16(dst_of(j + 1), vb, nch, lane);
    if (!has2) break;
  }
}

// Quantise one BF16 row of H elements to MXFP8 along H: codes [H], scales [H/32]. Each lane
// loads the 64 bytes of up to 4 blocks before quantising any, to keep loads in flight.
__device__ __forceinline__ void quant_row_mx(const uint16_t* src, uint8_t* codes, uint8_t* scales,
                                             int H, int lane) {
  const int nblk = H / 32;
  for (int b0 = 0; b0 < nblk; b0 += 64 * 4) {
    u32x4 raw[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = b0 + j * 64 + lane;
      const u32x4* s = reinterpret_cast<const u32x4*>(src + int64_t(b) * 32);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        raw[j][q] = (src && b < nblk) ? __builtin_nontemporal_load(s + q) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = b0 + j * 64 + lane;
      if (b >= nblk) continue;
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[q * 8 + 2 * i] = __uint_as_float(raw[j][q][i] << 16);
          v[q * 8 + 2 * i + 1] = __uint_as_float(raw[j][q][i] & 0xFFFF0000u);
        }
      uint32_t c8[8];
      const uint32_t sc = mx_quant32(v, c8);
      u32x4* d = reinterpret_cast<u32x4*>(codes + b * 32);
      d[0] = u32x4{c8[0], c8[1], c8[2], c8[3]};
      d[1] = u32x4{c8[4], c8[5], c8[6], c8[7]};
      scales[b] = uint8_t(sc);
    }
  }
}

// Rows of at most 8192 BF16 values, MXFP8 along the row: lane l loads the 16-byte chunks
// l, l + 64, ... (as load_row16), so every load instruction reads 1 KB of consecutive bytes,
// and an aligned group of 4 lanes holds one 32-element MX block (src == nullptr loads zeros).
// The codes leave as 8 bytes per lane (512 consecutive bytes per instruction), the scale from
// the group's first lane. Same rule as quant_row_mx.
__device__ __forceinline__ void mx_row_load(const uint16_t* src, u32x4 (&raw)[16], int nch,
                                            int lane) {
  load_row16(src, raw, nch, lane);
}

__device__ __forceinline__ void mx_row_store(const u32x4 (&raw)[16], uint8_t* codes,
                                             uint8_t* scales, int nch, int lane) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q * 64 >= nch) break;                     // (uniform)
    const int c = q * 64 + lane;
    uint32_t sc;
    const uint2 cw = mx_quant8_group4(raw[q], &sc);   // every lane: the block amax shuffles
    if (c < nch) {
      *reinterpret_cast<uint2*>(codes + int64_t(c) * 8) = cw;
      if ((lane & 3) == 0) scales[c >> 2] = uint8_t(sc);
    }
    // one chunk at a time: interleaving the 16 chunks' arithmetic would hold all of their
    // temporaries at once (spills in the fused forward kernel, which inlines this)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Quantise rows j = 0 .. nrows-1 (H <= 8192) from src_of(j) to codes_of(j) / scales_of(j),
// keeping two rows in flight per wave: row j+1 is loaded before row j is quantised, so the
// quantiser's arithmetic runs under the next row's load latency.
template <class Src, class Codes, class Scales>
__device__ __forceinline__ void quant_rows_mx_2(int nrows, int H, int lane, Src src_of,
                                                Codes codes_of, Scales scales_of) {
  const int nch = H / 8;
  u32x4 ra[16], rb[16];
  if (nrows <= 0) return;
  mx_row_load(src_of(0), ra, nch, lane);
  for (int j = 0;; j += 2) {
    const bool has1 = j + 1 < nrows;
    if (has1) mx_row_load(src_of(j + 1), rb, nch, lane);
    mx_row_store(ra, codes_of(j), scales_of(j), nch, lane);
    if (!has1) break;
    const bool has2 = j + 2 < nrows;
    if (has2) mx_row_load(src_of(j + 2), ra, nch, lane);
    mx_row_store(rb, codes_of(j + 1), scales_of(j + 1), nch, lane);
    if (!has2) break;
  }
}

// Fixed-order merge of token n's local pairs: dst = bf16( sum over k ascending, idx[n,k]
// local, of w_k * slots[n*K+k] ), w_k = p[n,k] (or 1 when p == nullptr). fp32 accumulation,
// one fused multiply-add per term in k order, so the result is bit-reproducible. The token's
// K indices and weights are read once (lane k), and a pass keeps 16 chunks of 16 bytes per
// lane of every term in flight.
__device__ __forceinline__ void merge_row(int64_t n, const int32_t* idx, const float* p,
                                         const uint16_t* slots, uint16_t* dst, int H, int K, int e0,
                                         int El, int lane) {
  int my_le = -1;
  float my_w = 0.f;
  if (lane < K) {
    my_le = idx[n * K + lane] - e0;
    my_w = p ? p[n * K + lane] : 1.f;
  }
  const uint64_t local = __ballot(my_le >= 0 && my_le < El);
  const int nch = H / 8;
  for (int c0 = 0; c0 < nch; c0 += 64 * 16) {
    float acc[16][8];
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[q][i] = 0.f;
    for (uint64_t m = local; m; m &= m - 1) {
      const int k = __builtin_ctzll(m);
      const float w = __shfl(my_w, k, 64);
      const u32x4* z = reinterpret_cast<const u32x4*>(slots + (n * K + k) * int64_t(H));
      u32x4 v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int c = c0 + q * 64 + lane;
        v[q] = c < nch ? __builtin_nontemporal_load(z + c) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          acc[q][2 * i] = fmaf(w, __uint_as_float(v[q][i] << 16), acc[q][2 * i]);
          acc[q][2 * i + 1] = fmaf(w, __uint_as_float(v[q][i] & 0xFFFF0000u), acc[q][2 * i + 1]);
        }
    }
    u32x4* d = reinterpret_cast<u32x4*>(dst);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int c = c0 + q * 64 + lane;
      if (c < nch)
        d[c] = u32x4{pack_bf2(acc[q][0], acc[q][1]), pack_bf2(acc[q][2], acc[q][3]),
                     pack_bf2(acc[q][4], acc[q][5]), pack_bf2(acc[q][6], acc[q][7])};
    }
  }
}

}  // namespace mok
