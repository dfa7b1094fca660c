// Grouped-GEMM tile engine for gfx950: one 256 x 256 output tile per workgroup of 4 waves
// (2 x 2, each wave 128 x 128 = 4 x 4 MFMA 32x32 blocks), K consumed in stages of 128 bytes
// per row (64 BF16 or 128 E4M3 values), double-buffered in LDS.
//
// Both operands are staged "K-contiguous": LDS holds [256 rows][128 bytes] per stage, 16-byte
// chunks XOR-swizzled per row (swz) so the MFMA fragment reads (32 rows at one chunk per
// half-wave) are free of bank conflicts. Stages are filled by buffer loads that write LDS
// directly, issued one stage ahead of the MFMA work.
//
// MFMA result layout (v_mfma_f32_32x32x16_bf16 and v_mfma_scale_f32_32x32x64_f8f6f4, checked
// on gfx950): accumulator register v of lane l holds row 8*(v/4) + 4*(l/32) + (v%4), column
// l%32. Lanes 0-31 and 32-63 carry the two K-halves of each BF16 operand fragment; the fp8
// layout is described at mma_stage_mx.
#pragma once

#include <type_traits>

#include "mok_device.h"
#include "mok_internal.h"

namespace mok {

constexpr int kStageRowBytes = 128;
constexpr int kStageBytes = kTileM * kStageRowBytes;   // 32 KB per operand per stage

struct GemmLds {
  uint8_t a[2][kStageBytes];
  uint8_t b[2][kStageBytes];
  uint32_t as[2][kTileM];   // MXFP8: the 4 scale bytes of each row for the stage
  uint32_t bs[2][kTileN];
};
constexpr size_t kGemmLdsBytes = sizeof(GemmLds);

// Physical chunk of logical 16-byte chunk `chunk` in row `row`: chunk ^ f(row) with
// f(row) = (row & 7) ^ ((row >> 3) & 1). Any 8 consecutive rows, and the 8 even (or odd) rows
// of any aligned 16-row group, then occupy 8 different chunk positions, so a half-wave reading
// one chunk of 32 consecutive rows is free of bank conflicts whether the LDS serves 8 or 16
// lanes of a 16-byte read per cycle (measured: 2-way conflicts with f(row) = row & 7).
__device__ __forceinline__ int swz_f(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kStageRowBytes + ((chunk ^ swz_f(row)) << 4);
}

// Hide a value from loop-invariant code motion: persistent kernels would otherwise hoist
// hundreds of per-row epilogue addresses out of the tile loop and spill them.
template <class T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Thread index for per-tile code. Laundered through opaque() so that lane-dependent epilogue
// addresses are recomputed per tile instead of being hoisted out of the persistent tile loop
// and kept live (in VGPRs, or spilled) across the K loop.
__device__ __forceinline__ int tile_tid() { return opaque(int(threadIdx.x)); }

// Accumulator row of register v for this lane, inside a 32 x 32 block.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

// ---- operand source: rows with the reduction axis contiguous in memory -------------------
// Staged straight from global memory into LDS with buffer loads (no registers in between).
// A buffer resource covers exactly the valid rows of the tile, so rows past a ragged edge
// read as zeros. With `interleave`, 64-row blocks of the tile alternate between two matrices
// (r0/s0 for even blocks, r1/s1 for odd), block q reading rows (q/2)*64 .. of its matrix; a
// 64-row block is exactly one wave's share of a stage, so every load has one resource.
typedef __attribute__((address_space(3))) void lds_void;

struct Operand {
  __amdgpu_buffer_rsrc_t r0, r1;    // codes / BF16 values
  __amdgpu_buffer_rsrc_t s0, s1;    // MXFP8 scales
  int stride;                       // bytes per row
  int sstride;                      // scale bytes per row
  int interleave;                   // 64-row blocks alternate r0 / r1
  int ksplit;                       // stages kt >= ksplit read r1/s1 at stage kt - ksplit
};

__device__ __forceinline__ Operand operand(__amdgpu_buffer_rsrc_t r, int stride) {
  Operand o;
  o.r0 = o.r1 = r;
  o.s0 = o.s1 = r;
  o.stride = stride;
  o.sstride = 0;
  o.interleave = 0;
  o.ksplit = 0x7FFFFFFF;
  return o;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // Raw buffer: stride 0, num_records = bytes (clamped to the 32-bit field).
  const int nrec = int(bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0ll : (bytes < 0 ? 0 : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nrec, 0x00020000);
}

__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
}

// Cache policy of a stage load. kLoadAgent (sc1): agent scope, the load misses in the CU's L1
// and is served by the XCD's L2. A-operand rows can be rows another CU of the XCD stored
// during the same launch (ring slots of the fused forward, reused for one row tile after
// another), and an L1 line kept from an earlier read of the same address would be stale;
// the A tile of a workgroup is read once per stage, so bypassing L1 costs nothing (measured).
constexpr int kLoadDefault = 0, kLoadAgent = 16;

// Issue the loads of stage kt (128 bytes of every row, and in MXFP8 mode the 4 scale bytes of
// every row) into one LDS stage. Wave w covers rows 64w .. 64w+63: 8 loads of 8 rows x 128
// bytes. Lane L of load c lands at LDS offset 16*L: row 64w + 8c + L/8, physical chunk L%8,
// which holds the logical chunk (L%8) ^ f(row) of the swizzled layout, where
// f(row) = (L/8) ^ (c & 1) because 64w + 8c is a multiple of 8.
template <int POLICY>
__device__ __forceinline__ void issue_stage(const Operand& op, uint8_t* lds, uint32_t* lds_s, int kt,
                                            bool mx, int w) {
  // The lane's offsets are recomputed per stage (a few VALU operations) rather than hoisted out
  // of the K loop, where 8 per operand would stay live and, in MXFP8, be spilled. `w` is the
  // wave index, computed once by the caller (a uniform value).
  const int L = opaque(int(threadIdx.x) & 63);
  const int lchunk0 = (L & 7) ^ (L >> 3);
  const bool second = kt >= op.ksplit;                 // K split across two sources
  if (second) kt -= op.ksplit;
  const bool odd = (op.interleave && (w & 1)) || second;
  const __amdgpu_buffer_rsrc_t r = odd ? op.r1 : op.r0;
  const int rbase = op.interleave ? (w >> 1) * 64 : w * 64;   // first row inside the matrix
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int lrow = rbase + 8 * c + (L >> 3);
    const int lchunk = lchunk0 ^ (c & 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds + (w * 64 + 8 * c) * kStageRowBytes),
                                             16, lrow * op.stride + kt * kStageRowBytes + lchunk * 16,
                                             0, 0, POLICY);
  }
  if (mx) {
    const __amdgpu_buffer_rsrc_t rs = odd ? op.s1 : op.s0;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds_s + w * 64), 4,
                                             (rbase + L) * op.sstride + kt * 4, 0, 0, POLICY);
  }
}

// ---- MFMA fragments ------------------------------------------------------------------------
// One "kk" step is one MFMA K-slice: 16 BF16 (32x32x16) or 64 E4M3 (32x32x64). A stage of 128
// bytes per row holds 4 BF16 slices or 2 E4M3 slices. Fragments of slice kk+1 are loaded from
// LDS while the 16 MFMAs of slice kk run, so LDS latency hides under matrix work.
struct FragBF16 {
  bf16x8 a[4], b[4];
};
struct FragMX {
  i32x8 a[4], b[4];
  int sa[4], sb[4];
};

__device__ __forceinline__ void load_frag(FragBF16& f, const uint8_t* A, const uint8_t* B,
                                          const uint32_t*, const uint32_t*, int kk, int wm, int wn,
                                          int lane) {
  const int ch = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.a[i] = *reinterpret_cast<const bf16x8*>(A + swz(wm * 128 + i * 32 + (lane & 31), ch));
    f.b[i] = *reinterpret_cast<const bf16x8*>(B + swz(wn * 128 + i * 32 + (lane & 31), ch));
  }
}

// E4M3 slice kk covers MX blocks 2kk and 2kk+1. Lane half h carries elements 16h..16h+15 of
// block 2kk in bytes 0-15 and of block 2kk+1 in bytes 16-31, and its scale byte is that of
// block 2kk+h (checked on gfx950).
__device__ __forceinline__ void load_frag(FragMX& f, const uint8_t* A, const uint8_t* B,
                                          const uint32_t* As, const uint32_t* Bs, int kk, int wm,
                                          int wn, int lane) {
  const int h = lane >> 5;
  const int blk = kk * 2 + h;
  const int ch0 = kk * 4 + h, ch1 = kk * 4 + 2 + h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + (lane & 31);
    const int rb = wn * 128 + i * 32 + (lane & 31);
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(A + swz(ra, ch0));
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(A + swz(ra, ch1));
    const u32x4 b0 = *reinterpret_cast<const u32x4*>(B + swz(rb, ch0));
    const u32x4 b1 = *reinterpret_cast<const u32x4*>(B + swz(rb, ch1));
    f.a[i] = i32x8{int(a0[0]), int(a0[1]), int(a0[2]), int(a0[3]),
                   int(a1[0]), int(a1[1]), int(a1[2]), int(a1[3])};
    f.b[i] = i32x8{int(b0[0]), int(b0[1]), int(b0[2]), int(b0[3]),
                   int(b1[0]), int(b1[1]), int(b1[2]), int(b1[3])};
    f.sa[i] = int((As[ra] >> (8 * blk)) & 0xFFu);
    f.sb[i] = int((Bs[rb] >> (8 * blk)) & 0xFFu);
  }
}

__device__ __forceinline__ void mma(const FragBF16& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ void mma(const FragMX& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], 0, 0,
                                                                  0, f.sa[i], 0, f.sb[j]);
}

// s_waitcnt with only the vector-memory counter at zero (gfx9 encoding: expcnt and lgkmcnt
// fields left at their maxima), so fragment reads from LDS stay in flight.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- the tile loop -----------------------------------------------------------------------
// Runs the K loop of one output tile; on return acc holds the fp32 tile (no split-K, slices
// in ascending K order, so the result depends only on the operands). Per stage: issue the
// next stage's buffer loads, then for each slice load the next slice's fragments and run the
// current slice's MFMAs; the stage barrier sits before the last slice, so the first fragments
// of the next stage also load under MFMA work. After return every LDS read of the stage
// buffers has completed (the last barrier precedes the last slice's MFMAs, whose fragments
// are already in registers), so the caller may reuse the LDS.
template <bool MX>
__device__ __forceinline__ void gemm_tile(GemmLds& sm, const Operand& A, const Operand& B,
                                          int ksteps, f32x16 (&acc)[4][4], int wm, int wn,
                                          int lane) {
  using Frag = typename std::conditional<MX, FragMX, FragBF16>::type;
  constexpr int KK = MX ? 2 : 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if (ksteps <= 0) return;
  const int w = wave_id();
  issue_stage<kLoadAgent>(A, sm.a[0], sm.as[0], 0, MX, w);
  issue_stage<kLoadDefault>(B, sm.b[0], sm.bs[0], 0, MX, w);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  Frag f[2];
  load_frag(f[0], sm.a[0], sm.b[0], sm.as[0], sm.bs[0], 0, wm, wn, lane);
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < ksteps;
    // BF16 (4 slices per stage): the next stage's A loads go out before slice 0 and its B loads
    // before slice 1, so the DMA writes into LDS are spread over the stage instead of
    // competing with one slice's fragment reads (measured +9 %). E4M3 (2 slices): both before
    // slice 0, which leaves the whole stage to cover their latency.
    if (more && MX) {
      issue_stage<kLoadAgent>(A, sm.a[cur ^ 1], sm.as[cur ^ 1], kt + 1, MX, w);
      issue_stage<kLoadDefault>(B, sm.b[cur ^ 1], sm.bs[cur ^ 1], kt + 1, MX, w);
    }
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (!MX && more && kk == 0) issue_stage<kLoadAgent>(A, sm.a[cur ^ 1], sm.as[cur ^ 1], kt + 1, MX, w);
      if (!MX && more && kk == 1) issue_stage<kLoadDefault>(B, sm.b[cur ^ 1], sm.bs[cur ^ 1], kt + 1, MX, w);
      // Scheduling fences keep each phase whole: the compiler would otherwise interleave the
      // MFMAs of slice kk with the fragment reads of slice kk+1 and wait on those reads.
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < KK) {
        load_frag(f[(kk + 1) & 1], sm.a[cur], sm.b[cur], sm.as[cur], sm.bs[cur], kk + 1, wm, wn,
                  lane);
      } else {
        wait_vmem();
        __syncthreads();
        if (more)
          load_frag(f[(kk + 1) & 1], sm.a[cur ^ 1], sm.b[cur ^ 1], sm.as[cur ^ 1], sm.bs[cur ^ 1],
                    0, wm, wn, lane);
      }
      mma(f[kk & 1], acc);
      if (!MX) {
        // BF16: one fragment read between consecutive MFMAs of the slice
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      } else {
        // E4M3: the 24 LDS reads of the next slice (16 code fragments, 8 scale words), two
        // between consecutive MFMAs (measured 3-8 % faster than issuing them all first)
#pragma unroll
        for (int q = 0; q < 12; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- B operand in fragment order (BF16) -----------------------------------------------------
// A packed matrix with R rows (a multiple of 32) and reduction length K (a multiple of 16) is
// stored as R/32 x K/16 fragments of 1 KB: fragment (n32, k16) at byte (n32 * K/16 + k16) * 1024,
// where lane l's 16 bytes hold row 32 n32 + l % 32, elements 16 k16 + 8 (l / 32) .. +7 -- the
// register contents of a v_mfma_f32_32x32x16_bf16 fragment. One load per lane then fills a
// fragment from 1 KB of consecutive bytes (8 whole cache lines), where row-major rows would
// touch 32 lines per load. The first r rows (r a multiple of 32) take the first r * K * 2 bytes,
// as in a row-major matrix, so a row offset converts to a byte offset the same way.
struct PackedB {
  __amdgpu_buffer_rsrc_t r;   // from the tile's first row; rows past the valid ones read as 0
  int k16s;                   // K / 16: fragments per 32-row block
};

__device__ __forceinline__ PackedB packed_b(const uint8_t* plane, int64_t row0, int nrows, int K) {
  PackedB p;
  p.r = make_rsrc(plane + row0 * K * 2, int64_t(nrows) * K * 2);
  p.k16s = K / 16;
  return p;
}

// Slice kk of stage kt: the wave's 4 B fragments (column blocks j of its 128 tile columns).
__device__ __forceinline__ void load_b_packed(bf16x8 (&b)[4], const PackedB& B, int kt, int kk,
                                              int wn, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 v = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   B.r, ((wn * 4 + j) * B.k16s + kt * 4 + kk) * 1024 + lane * 16, 0, 0));
    b[j] = __builtin_bit_cast(bf16x8, v);
  }
}

__device__ __forceinline__ void load_a_frag(bf16x8 (&a)[4], const uint8_t* A, int kk, int wm,
                                            int lane) {
  const int ch = kk * 2 + (lane >> 5);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(A + swz(wm * 128 + i * 32 + (lane & 31), ch));
}

// The K loop of one BF16 output tile with a packed B operand. A is staged through LDS as in
// gemm_tile; B fragments go from global memory straight into registers one stage ahead: once
// the MFMAs of slice kk have read B(kt, kk), the same registers are loaded with B(kt+1, kk). That
// halves the LDS traffic per stage (the DMA writes and fragment reads of B are gone), the
// largest cost of the LDS-staged loop. The stage barrier waits only for the A stage; the 12 B
// loads issued after it stay in flight. Slices run in the same order as gemm_tile, so the
// result is bit-identical to it. On return no load is in flight and every LDS read of the stage
// buffers has completed.
__device__ __forceinline__ void gemm_tile_pb(GemmLds& sm, const Operand& A, const PackedB& B,
                                             int ksteps, f32x16 (&acc)[4][4], int wm, int wn,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if (ksteps <= 0) return;
  const int w = wave_id();
  const int last = ksteps - 1;
  bf16x8 b[4][4];   // [slice][column block]
  bf16x8 fa[2][4];
  issue_stage<kLoadAgent>(A, sm.a[0], sm.as[0], 0, false, w);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) load_b_packed(b[kk], B, 0, kk, wn, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  load_a_frag(fa[0], sm.a[0], 0, wm, lane);
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    const bool more = kt < last;
    // Issued in every stage (in the last one a harmless reload of the same stage): with a
    // conditional issue the compiler counts the stage's loads as absent on the merged path and
    // its waits for each B slice would also wait for 8 younger B loads.
    issue_stage<kLoadAgent>(A, sm.a[cur ^ 1], sm.as[cur ^ 1], more ? kt + 1 : kt, false, w);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk + 1 < 4) {
        load_a_frag(fa[(kk + 1) & 1], sm.a[cur], kk + 1, wm, lane);
      } else {
        // vmcnt(12): the loads issued after A(kt+1) are B(kt+1) of slices 0-2, 4 each
        __builtin_amdgcn_s_waitcnt(0x0F7C);
        __syncthreads();
        if (more) load_a_frag(fa[0], sm.a[cur ^ 1], 0, wm, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[kk & 1][i], b[kk][j], acc[i][j],
                                                               0, 0, 0);
      // (in the last stage a harmless reload of the same slice, so every stage issues the same
      // loads and the wait count above holds)
      load_b_packed(b[kk], B, more ? kt + 1 : kt, kk, wn, lane);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // global load
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// ---- B operand in fragment order (MXFP8) ----------------------------------------------------
// E4M3 codes of a packed matrix with R rows and reduction length K (a multiple of 64): R/32 x
// K/64 fragments of 2 KB, fragment (n32, k64) at byte (n32 * K/64 + k64) * 2048, made of two
// 1 KB halves: half 0 holds in lane l's 16 bytes the codes 64 k64 + 16 (l / 32) .. +15 of row
// 32 n32 + l % 32, half 1 the codes 32 further -- together the lane's 32-byte operand of
// v_mfma_scale_f32_32x32x64_f8f6f4 (see load_frag). The UE8M0 scales follow the same blocks:
// 64 bytes per fragment, byte l the scale of that row's 32-code block 2 k64 + l / 32, which is
// the scale operand of lane l. The first r rows take the first r K code bytes and r K / 32 scale
// bytes, as in a row-major matrix.
struct PackedBMX {
  __amdgpu_buffer_rsrc_t r;   // codes, from the tile's first fragment
  __amdgpu_buffer_rsrc_t s;   // scales, from the tile's first fragment
  int k64s;                   // K / 64: fragments per 32-row block
};

__device__ __forceinline__ PackedBMX packed_b_mx(const uint8_t* codes, const uint8_t* scales,
                                                 int64_t row0, int nrows, int K) {
  PackedBMX p;
  p.r = make_rsrc(codes + row0 * K, int64_t(nrows) * K);
  p.s = make_rsrc(scales + row0 * (K / 32), int64_t(nrows) * (K / 32));
  p.k64s = K / 64;
  return p;
}

// Slice kk of stage kt (64 codes per row): the wave's 4 B fragments and their scale bytes.
__device__ __forceinline__ void load_b_packed_mx(i32x8 (&b)[4], int (&sb)[4], const PackedBMX& B,
                                                 int kt, int kk, int wn, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = (wn * 4 + j) * B.k64s + kt * 2 + kk;
    const u32x4 lo = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(B.r, f * 2048 + lane * 16, 0, 0));
    const u32x4 hi = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(B.r, f * 2048 + 1024 + lane * 16, 0, 0));
    b[j] = i32x8{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]),
                 int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
    sb[j] = int(__builtin_amdgcn_raw_buffer_load_b8(B.s, f * 64 + lane, 0, 0));
  }
}

// A fragments of E4M3 slice kk from the LDS stage (as load_frag) and their scale bytes.
__device__ __forceinline__ void load_a_frag_mx(i32x8 (&a)[4], int (&sa)[4], const uint8_t* A,
                                               const uint32_t* As, int kk, int wm, int lane) {
  const int h = lane >> 5;
  const int blk = kk * 2 + h;
  const int ch0 = kk * 4 + h, ch1 = kk * 4 + 2 + h;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ra = wm * 128 + i * 32 + (lane & 31);
    const u32x4 a0 = *reinterpret_cast<const u32x4*>(A + swz(ra, ch0));
    const u32x4 a1 = *reinterpret_cast<const u32x4*>(A + swz(ra, ch1));
    a[i] = i32x8{int(a0[0]), int(a0[1]), int(a0[2]), int(a0[3]),
                 int(a1[0]), int(a1[1]), int(a1[2]), int(a1[3])};
    sa[i] = int((As[ra] >> (8 * blk)) & 0xFFu);
  }
}

// The K loop of one MXFP8 output tile with a packed B operand: two E4M3 slices per stage. A
// codes and scales go through LDS by DMA (9 loads per wave per stage), issued into the
// double buffer as soon as the mid-stage barrier frees it, so each A stage has a full stage of
// matrix work to arrive; B codes and scale bytes go straight into registers, one stage ahead
// (12 loads per slice). The barrier leaves the 12 loads of B(kt+1) slice 0 in flight.
// Bit-identical to gemm_tile<true>.
__device__ __forceinline__ void gemm_tile_pb_mx(GemmLds& sm, const Operand& A, const PackedBMX& B,
                                                int ksteps, f32x16 (&acc)[4][4], int wm, int wn,
                                                int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if (ksteps <= 0) return;
  const int w = wave_id();
  const int last = ksteps - 1;
  i32x8 b[2][4];   // [slice][column block]
  int sb[2][4];
  i32x8 fa[2][4];
  int sa[2][4];
  issue_stage<kLoadAgent>(A, sm.a[0], sm.as[0], 0, true, w);
  issue_stage<kLoadAgent>(A, sm.a[1], sm.as[1], min(1, last), true, w);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) load_b_packed_mx(b[kk], sb[kk], B, 0, kk, wn, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  load_a_frag_mx(fa[0], sa[0], sm.a[0], sm.as[0], 0, wm, lane);
  for (int kt = 0; kt < ksteps; ++kt) {
    const int cur = kt & 1;
    const bool more = kt < last;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 0) {
        load_a_frag_mx(fa[1], sa[1], sm.a[cur], sm.as[cur], 1, wm, lane);
      } else {
        // vmcnt(12): everything but the 12 loads of B(kt+1) slice 0 has landed, A(kt+1) too
        __builtin_amdgcn_s_waitcnt(0x0F7C);
        __syncthreads();
        // Stage kt's fragments are all in registers now, so its buffer takes A(kt+2): a whole
        // stage of matrix work to cover the DMA, against one slice if it were issued at the
        // start of stage kt+1. Issued in every stage (near the end a harmless reload of the
        // last one) so that the compiler's waits for B count these 9 loads.
        issue_stage<kLoadAgent>(A, sm.a[cur], sm.as[cur], min(kt + 2, last), true, w);
        if (more) load_a_frag_mx(fa[0], sa[0], sm.a[cur ^ 1], sm.as[cur ^ 1], 0, wm, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[kk][i], b[kk][j], acc[i][j], 0, 0, 0, sa[kk][i], 0, sb[kk][j]);
      // (in the last stage a harmless reload of the same slice, so the wait count holds)
      load_b_packed_mx(b[kk], sb[kk], B, more ? kt + 1 : kt, kk, wn, lane);
#pragma unroll
      for (int q = 0; q < 12; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 3, 0);   // global loads
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// ---- tile scheduling ------------------------------------------------------------------------
// Logical workgroup id that gives the workgroups resident on one XCD (blockIdx % 8 on MI355X)
// consecutive ids, so consecutive tiles -- which share operands -- land in one L2.
__device__ __forceinline__ int xcd_logical_id() {
  const int G = gridDim.x, b = blockIdx.x;
  if (G % 8) return b;
  return (b % 8) * (G / 8) + b / 8;
}

// Grouped order: tile t -> (m-tile, n-tile), sweeping kGroupM m-tiles per group so that a
// run of consecutive tiles reuses kGroupM row panels and a few column panels.
constexpr int kGroupM = 4;
__device__ __forceinline__ void tile_coords(int t, int mtiles, int ntiles, int& mt, int& nt) {
  const int gsize = kGroupM * ntiles;
  const int g = t / gsize;
  const int first = g * kGroupM;
  const int gm = min(kGroupM, mtiles - first);
  const int local = t % gsize;
  mt = first + local % gm;
  nt = local / gm;
}

}  // namespace mok
