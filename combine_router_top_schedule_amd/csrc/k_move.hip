// Data-movement kernels: pull dispatch (gather into expert order, MXFP8 quantisation fused),
// the fixed-order weighted merge (combine), the MX weight quantiser and a fill kernel.
// All of them are HBM-bound: one wave per row, 16-byte accesses, coalesced along the row.
#include "mok_internal.h"
#include "mok_device.h"
#include "mok_rows.h"

namespace mok {
namespace {

__global__ void k_fill_u32(uint32_t* p, uint32_t v, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

struct FillRanges {
  FillRange r[kMaxFillRanges];
  int count;
};

__global__ void k_fill_ranges(FillRanges a) {
  for (int k = 0; k < a.count; ++k)
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < a.r[k].n;
         i += int64_t(gridDim.x) * blockDim.x)
      a.r[k].p[i] = a.r[k].v;
}

// Pull dispatch ("Mixture-of-Kittens (MoK)", section on pull dispatch; "把 MoE 通信延迟从 103μs
// 压到 18μs", section 03 part ①): the receiving side reads each routed row from its source
// segment and lays it out in expert order; MXFP8 rows are quantised along H on the way
// (section 03 part ③).
__global__ __launch_bounds__(256) void k_dispatch(const int32_t* hdr, const int32_t* perm,
                                                  const uint16_t* const* x_seg, uint8_t* xd,
                                                  int64_t rows_max, int H, int K, int S,
                                                  int T, int dtype) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int64_t rows = min(int64_t(hdr[kHdrRows]), rows_max);
  const int64_t NK = int64_t(S) * T * K;
  if (dtype != MOK_BF16 && H <= 8 * kRowBatchChunks) {
    // MXFP8: the wave's rows wave, wave + nwaves, ... quantised with the next row's loads (and
    // its source lookup) in flight.
    const int nrw = wave < rows ? int((rows - 1 - wave) / nwaves + 1) : 0;
    auto row_of = [&](int j) { return wave + int64_t(j) * nwaves; };
    quant_rows_mx_2(
        nrw, H, lane,
        [&](int j) -> const uint16_t* {
          const int32_t pair = perm[row_of(j)];
          if (pair < 0 || pair >= NK) return nullptr;
          const int64_t n = pair / K;
          return x_seg[n / T] + (n % T) * int64_t(H);
        },
        [&](int j) { return xd + row_of(j) * H; },
        [&](int j) { return xd + rows_max * H + row_of(j) * (H / 32); });
    return;
  }
  for (int64_t r = wave; r < rows; r += nwaves) {
    const int32_t pair = perm[r];
    const uint16_t* src = nullptr;
    if (pair >= 0 && pair < NK) {
      const int64_t n = pair / K;
      src = x_seg[n / T] + (n % T) * int64_t(H);
    }
    if (dtype == MOK_BF16) {
      copy_row_bf16(src, reinterpret_cast<uint16_t*>(xd) + r * H, H, lane);
    } else {
      quant_row_mx(src, xd + r * H, xd + rows_max * H + r * (H / 32), H, lane);
    }
  }
}

// Final weighted merge ("把 MoE 通信延迟从 103μs 压到 18μs", section 04): for every token of
// `list` (hdr[count_word] of them), out[n] = bf16( sum over k ascending, idx[n,k] local, of
// p[n,k] * y[n*K+k] ). The list is every touched token, or (in the fused paths, whose GEMM
// epilogues write the rows of tokens with a single local pair with the same arithmetic) only
// the tokens with several local pairs.
__global__ __launch_bounds__(256) void k_combine(const int32_t* hdr, int count_word,
                                                 const int32_t* list, const int32_t* idx,
                                                 const float* p, const uint16_t* slots,
                                                 uint16_t* const* out_seg, int H, int K, int S,
                                                 int T, int e0, int El) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int64_t N = int64_t(S) * T;
  const int64_t U = min(int64_t(hdr[count_word]), N);
  for (int64_t u = wave; u < U; u += nwaves) {
    const int64_t n = list[u];
    if (n < 0 || n >= N) continue;
    merge_row(n, idx, p, slots, out_seg[n / T] + (n % T) * int64_t(H), H, K, e0, El, lane);
  }
}

// Push record of every expert-ordered row (see PushRec); pad rows (code -1) get a raw record
// no tile uses.
__global__ __launch_bounds__(256) void k_push_rows(const int32_t* hdr, const int32_t* pcode,
                                                   uint16_t* slots, uint16_t* const* seg,
                                                   const float* p, PushRec* rec,
                                                   int64_t rows_max, int H, int K, int T) {
  const int64_t rows = min(int64_t(hdr[kHdrRows]), rows_max);
  for (int64_t r = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; r < rows;
       r += int64_t(gridDim.x) * blockDim.x) {
    const int32_t code = pcode[r];
    PushRec o{slots, -1.f, 0};
    if (code >= 0) {
      const int32_t pair = code & ~kSoleFlag;
      if (code & kSoleFlag) {
        const int n = pair / K;
        o.dst = seg[n / T] + int64_t(n % T) * H;
        o.w = p ? p[pair] : 1.f;
      } else {
        o.dst = slots + int64_t(pair) * H;
      }
    }
    rec[r] = o;
  }
}

// MX quantiser for weights: blocks of 32 along the last axis, or (transpose) of the
// transposed matrix along the input's rows.
__global__ __launch_bounds__(256) void k_quant_mx(const uint16_t* src, uint8_t* codes,
                                                  uint8_t* scales, int batch, int rows, int cols,
                                                  int transpose) {
  const int64_t nblk_per = transpose ? int64_t(cols) * (rows / 32) : int64_t(rows) * (cols / 32);
  const int64_t total = nblk_per * batch;
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < total;
       q += int64_t(gridDim.x) * blockDim.x) {
    const int64_t bt = q / nblk_per, w = q % nblk_per;
    const uint16_t* m = src + bt * int64_t(rows) * cols;
    float v[32];
    int64_t out_row, out_blk, out_w;
    if (!transpose) {
      const int64_t r = w / (cols / 32), c0 = (w % (cols / 32)) * 32;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = bf2f(m[r * cols + c0 + i]);
      out_row = r; out_blk = c0 / 32; out_w = cols;
    } else {
      // consecutive threads take consecutive columns: the strided reads coalesce per row
      const int64_t c = w % cols, r0 = (w / cols) * 32;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = bf2f(m[(r0 + i) * cols + c]);
      out_row = c; out_blk = r0 / 32; out_w = rows;
    }
    uint32_t c8[8];
    const uint32_t sc = mx_quant32(v, c8);
    uint8_t* cb = codes + bt * int64_t(rows) * cols + out_row * out_w + out_blk * 32;
    reinterpret_cast<u32x4*>(cb)[0] = u32x4{c8[0], c8[1], c8[2], c8[3]};
    reinterpret_cast<u32x4*>(cb)[1] = u32x4{c8[4], c8[5], c8[6], c8[7]};
    scales[bt * int64_t(rows) * cols / 32 + out_row * (out_w / 32) + out_blk] = uint8_t(sc);
  }
}

int grid_for(int64_t work_items, int per_block, int cap) {
  int64_t b = cdiv(work_items, per_block);
  if (b < 1) b = 1;
  return int(b > cap ? cap : b);
}

}  // namespace

// Compute units of the current device, cached per device id (0 if unknown).
int device_cus() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices && cus > 0) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(grid_for(n, 256, 2048)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}

hipError_t launch_fill_ranges(const FillRange* r, int count, hipStream_t s) {
  if (count > kMaxFillRanges) return hipErrorInvalidValue;
  FillRanges a{};
  int64_t nmax = 0;
  for (int k = 0; k < count; ++k) {
    if (r[k].n <= 0) continue;
    a.r[a.count++] = r[k];
    nmax = r[k].n > nmax ? r[k].n : nmax;
  }
  if (a.count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_ranges, dim3(grid_for(nmax, 256, 2048)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dispatch(const Layout& L, const uint8_t* saved, const void* const* x_seg,
                           uint8_t* xd, hipStream_t s) {
  const int cap = 8 * (device_cus() > 0 ? device_cus() : 256);
  trace_before(MOK_TRACE_DISPATCH, s);
  hipLaunchKernelGGL(k_dispatch, dim3(grid_for(L.rows_max, 4, cap)), dim3(256), 0, s,
                     reinterpret_cast<const int32_t*>(saved),
                     reinterpret_cast<const int32_t*>(saved + L.sv_perm),
                     reinterpret_cast<const uint16_t* const*>(x_seg), xd, L.rows_max, L.H, L.K,
                     L.S, L.T, L.dtype);
  trace_after(MOK_TRACE_DISPATCH, s);
  return hipGetLastError();
}

hipError_t launch_combine(const Layout& L, const uint8_t* saved, const int32_t* idx, const float* p,
                          const uint16_t* slots, void* const* out_seg, bool skip_sole,
                          hipStream_t s) {
  const int cap = 8 * (device_cus() > 0 ? device_cus() : 256);
  trace_before(MOK_TRACE_COMBINE, s);
  hipLaunchKernelGGL(k_combine, dim3(grid_for(L.N, 4, cap)), dim3(256), 0, s,
                     reinterpret_cast<const int32_t*>(saved), skip_sole ? kHdrUm : kHdrU,
                     reinterpret_cast<const int32_t*>(saved + (skip_sole ? L.sv_multi
                                                                         : L.sv_touched)),
                     idx, p, slots, reinterpret_cast<uint16_t* const*>(out_seg), L.H, L.K, L.S,
                     L.T, L.e0, L.El);
  trace_after(MOK_TRACE_COMBINE, s);
  return hipGetLastError();
}

hipError_t launch_push_rows(const Layout& L, const uint8_t* saved, uint16_t* slots,
                            void* const* seg, const float* p, PushRec* rec, hipStream_t s) {
  hipLaunchKernelGGL(k_push_rows, dim3(grid_for(L.rows_max, 256, 1024)), dim3(256), 0, s,
                     reinterpret_cast<const int32_t*>(saved),
                     reinterpret_cast<const int32_t*>(saved + L.sv_pcode), slots,
                     reinterpret_cast<uint16_t* const*>(seg), p, rec, L.rows_max, L.H, L.K, L.T);
  return hipGetLastError();
}

hipError_t launch_quantize_mx(int batch, int rows, int cols, const uint16_t* src, int transpose,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t blocks = int64_t(batch) * rows * (cols / 32);
  hipLaunchKernelGGL(k_quant_mx, dim3(grid_for(blocks, 256, 8192)), dim3(256), 0, s, src, codes,
                     scales, batch, rows, cols, transpose);
  return hipGetLastError();
}

}  // namespace mok
