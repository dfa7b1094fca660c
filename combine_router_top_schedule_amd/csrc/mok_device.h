// Device helpers shared by the kernels: BF16 and E4M3 conversions, MX block scales, agent-scope
// atomics for cross-workgroup signalling.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mok {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> BF16 bits, round to nearest even (the conversion instruction of gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return uint32_t(f2bf(lo)) | (uint32_t(f2bf(hi)) << 16);
}

// ---- MXFP8 -------------------------------------------------------------------------------
// Shared exponent of a 32-element block: floor(log2(amax)) - 8, clamped to [-127, 127]; amax
// is finite and >= 0. Read straight from the fp32 exponent field (exact); subnormal amax is
// handled by normalising first.
__device__ __forceinline__ int mx_block_exp(float amax) {
  uint32_t b = __float_as_uint(amax);
  int ex = int((b >> 23) & 0xFF);
  // amax == 0 or fp32-subnormal amax: floor(log2) <= -127, so the exponent clamps to -127.
  if (ex == 0) return -127;
  int e = (ex - 127) - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 2^e as fp32 for e in [-149, 127], exact (subnormal below 2^-126).
__device__ __forceinline__ float exp2i(int e) {
  if (e >= -126) return __uint_as_float(uint32_t(e + 127) << 23);
  return __uint_as_float(1u << (e + 149));   // subnormal powers 2^-127 .. 2^-149
}

// Scale v (already divided by the block scale) to E4M3: clamp to +-448 so the conversion
// never produces NaN, then the hardware conversion rounds to nearest even. Two values per
// call, packed in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

// Quantise 32 values in registers to 32 E4M3 codes (8 dwords) and return the scale code.
__device__ __forceinline__ uint32_t mx_quant32(const float* v, uint32_t* out8) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = mx_block_exp(amax);
  // Dividing by the power of two 2^e is a multiplication by 2^-e (-e in [-127, 127], a
  // representable fp32); it is exact for every value that can round to a non-zero code.
  float inv = exp2i(-e);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out8[i] = e4m3x2(v[4 * i] * inv, v[4 * i + 1] * inv) |
              (e4m3x2(v[4 * i + 2] * inv, v[4 * i + 3] * inv) << 16);
  }
  return uint32_t(e + 127);
}

// Quantise 8 fp32 values held by each lane of an aligned group of 4 consecutive lanes, which
// together form one 32-element MX block: same rule as mx_quant32 (block amax over the 4 lanes
// by shuffles). Returns the 8 codes; *scode gets the block's scale code. Every lane of the wave
// must call it.
__device__ __forceinline__ uint2 mx_quant8_group4_f(const float (&f)[8], uint32_t* scode) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int e = mx_block_exp(amax);
  const float inv = exp2i(-e);
  *scode = uint32_t(e + 127);
  return uint2{e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16),
               e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16)};
}

// The same for 8 BF16 values packed in v.
__device__ __forceinline__ uint2 mx_quant8_group4(const u32x4& v, uint32_t* scode) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
  return mx_quant8_group4_f(f, scode);
}

// ---- agent-scope signalling ---------------------------------------------------------------
// On MI355X every XCD has its own L2. An agent-scope release would write back the whole local
// L2 and an acquire invalidate it, so none is used: words that carry their own payload (scan
// states, counters) are accessed with relaxed agent-scope atomics, which are coherent across
// XCDs without any cache maintenance, and bulk data handed from one workgroup to another stays
// inside one XCD (the producer's stores complete before it bumps a counter; the consumer reads
// with loads that miss in its CU's L1).
__device__ __forceinline__ uint32_t ld_relaxed_u(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed_u(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_relaxed(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_relaxed(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Record the first device-side failure in the workspace error word.
__device__ __forceinline__ void set_error(int* err, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace mok
