// Router top-k, gating and the schedule table.
//
// The router picks K experts per token anew each step, so per-expert loads change every
// step; a schedule table then counts the tokens of every local expert, fixes each pair's row
// on the receiving side and keeps an expert's rows contiguous ("把 MoE 通信延迟从 103μs 压到
// 18μs", section 02). One table serves dispatch, combine and their backward mirrors
// ("Mixture-of-Kittens (MoK)", section on pull dispatch).
//
// Two kernels, no host synchronisation:
//  1. k_topk_scan: one thread per token computes top-k and the softmax gate; the block then
//     counts, per local expert, the pairs of its 256 tokens (ballot + popcount, an LDS
//     histogram per wave) and joins a single-pass decoupled look-back scan over blocks
//     (Merrill & Garland, 2016) that yields each pair's rank inside its expert, in ascending
//     token order. The last block writes counts, offsets, P and U.
//  2. k_place: turns ranks into rows (offset + rank) and fills perm (row -> pair) and tokpos
//     (pair -> row).
// A third single-workgroup kernel, k_tiles, cuts the expert-ordered rows into GEMM m-tiles
// for a given minibatch size.
#include "mok_internal.h"
#include "mok_device.h"

namespace mok {
namespace {

constexpr uint32_t kFlagAgg = 1u << 30;
constexpr uint32_t kFlagInc = 2u << 30;
constexpr uint32_t kValMask = (1u << 30) - 1;
constexpr int kSpinLimit = 1 << 22;

struct RouterArgs {
  const float* logits;
  int32_t* idx;
  float* p;
  int32_t* hdr;          // saved header
  int32_t* rank;         // tokpos, used here as the within-expert rank of each local pair
  int32_t* touched;
  int32_t* multi;        // touched tokens with more than one local pair, ascending
  uint32_t* state;       // [blocks][El + 2] look-back words
  int32_t* ticket;
  int32_t* err;
  int64_t N;
  int E, K, e0, El, row_align, nblocks;
};

// Ranking key of (logit x, expert e): the fp32 bits mapped to an order-preserving unsigned
// integer in the high word (negative values flipped entirely, non-negative ones with the sign
// bit set), and 0xFFFFFFFF - e in the low word. Larger key = larger logit, and on equal logits
// the lower expert id. -0.0 is mapped to +0.0 first so the two tie.
__device__ __forceinline__ uint64_t rank_key(float x, int e) {
  x = x == 0.f ? 0.f : x;
  const uint32_t u = __float_as_uint(x);
  const uint32_t m = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(m) << 32) | uint32_t(0xFFFFFFFFu - uint32_t(e));
}
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t m = uint32_t(k >> 32);
  return __uint_as_float((m & 0x80000000u) ? (m & 0x7FFFFFFFu) : ~m);
}
__device__ __forceinline__ int key_expert(uint64_t k) {
  return int(0xFFFFFFFFu - uint32_t(k));
}

// Insert a key into a descending top-KM list held in registers: one branch-free bubble pass
// that keeps the larger key at each position and carries the smaller one down.
template <int KM>
__device__ __forceinline__ void topk_insert(uint64_t (&key)[KM], uint64_t k) {
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const uint64_t kj = key[j];
    const bool c = k > kj;
    key[j] = c ? k : kj;
    k = c ? kj : k;
  }
}

// Sorts KM unique keys into descending order: odd-even transposition, KM rounds of
// compare-exchanges on neighbours (branch-free).
template <int KM>
__device__ __forceinline__ void sort_desc(uint64_t (&key)[KM]) {
#pragma unroll
  for (int r = 0; r < KM; ++r) {
#pragma unroll
    for (int j = r & 1; j + 1 < KM; j += 2) {
      const uint64_t x = key[j], y = key[j + 1];
      const bool c = y > x;
      key[j] = c ? y : x;
      key[j + 1] = c ? x : y;
    }
  }
}

// One thread per token: the block's 256 tokens stream their logits through LDS in chunks of
// 32 experts (coalesced 128-byte row pieces in, conflict-free column reads out), and each
// thread keeps its token's top-KM in registers. Two LDS chunk buffers: the loads of chunk
// c+1 are in flight while chunk c is ranked.
template <int KM>
__global__ __launch_bounds__(256) void k_topk_scan(RouterArgs a) {
  __shared__ int s_b;
  __shared__ float s_l[2][kTopkTokensPerBlock][33];
  __shared__ uint64_t s_mask[kTopkTokensPerBlock];
  __shared__ int s_wcnt[4][kMaxLocalExperts + 2];
  __shared__ int s_excl[kMaxLocalExperts + 2];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid == 0) s_b = atomicAdd(a.ticket, 1);   // dispatch-ordered block id for the look-back
  __syncthreads();
  const int b = s_b;
  const int64_t n_base = int64_t(b) * kTopkTokensPerBlock;
  const int64_t n_me = n_base + tid;

  uint64_t key[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) key[j] = 0;   // below every real key
  const bool vec4 = (a.E & 3) == 0;
  // Thread t covers rows t/8 + 32q, experts c0 + 4*(t%8) .. +3. Every load is issued
  // unconditionally from a clamped (in-bounds) address and masked when stored, so all eight
  // rows' loads are in flight together.
  float4 val[8];
  // (the branch on vec4 stays outside the row loop: inside it, the two paths were merged into
  // four 4-byte loads per row)
  auto load_chunk = [&](int c0) {
    const int col = c0 + 4 * (tid & 7);
    if (vec4) {
      const int cc = min(col, a.E - 4);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t n = min(n_base + (tid >> 3) + 32 * q, a.N - 1);
        val[q] = *reinterpret_cast<const float4*>(a.logits + n * a.E + cc);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t n = min(n_base + (tid >> 3) + 32 * q, a.N - 1);
        val[q].x = a.logits[n * a.E + min(col, a.E - 1)];
        val[q].y = a.logits[n * a.E + min(col + 1, a.E - 1)];
        val[q].z = a.logits[n * a.E + min(col + 2, a.E - 1)];
        val[q].w = a.logits[n * a.E + min(col + 3, a.E - 1)];
      }
    }
  };
  load_chunk(0);
  for (int c0 = 0, buf = 0; c0 < a.E; c0 += 32, buf ^= 1) {
    const int col = c0 + 4 * (tid & 7);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int r = (tid >> 3) + 32 * q;
      const bool rok = n_base + r < a.N;
      s_l[buf][r][4 * (tid & 7) + 0] = (rok && col + 0 < a.E) ? val[q].x : -INFINITY;
      s_l[buf][r][4 * (tid & 7) + 1] = (rok && col + 1 < a.E) ? val[q].y : -INFINITY;
      s_l[buf][r][4 * (tid & 7) + 2] = (rok && col + 2 < a.E) ? val[q].z : -INFINITY;
      s_l[buf][r][4 * (tid & 7) + 3] = (rok && col + 3 < a.E) ? val[q].w : -INFINITY;
    }
    // One barrier per chunk suffices with two buffers: a thread writing buffer `buf` again
    // (two chunks later) has passed the barrier after which every thread finished ranking it.
    __syncthreads();
    if (c0 + 32 < a.E) load_chunk(c0 + 32);
    const int ce = min(32, a.E - c0);
    // The token's 32 logits of the chunk, read together (one LDS round trip, not one per
    // candidate).
    float lv[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) lv[u] = s_l[buf][tid][u];
    // The first chunk starts the list as its first KM candidates, sorted by a compare-exchange
    // network instead of KM insertions.
    int u0 = 0;
    if (c0 == 0 && ce >= KM) {
#pragma unroll
      for (int j = 0; j < KM; ++j) key[j] = rank_key(lv[j], j);
      sort_desc<KM>(key);
      u0 = KM;
    }
    // Only a candidate above the list's smallest key can enter it: one 64-bit compare per
    // candidate builds the chunk's mask, and only those are inserted, in expert order (one the
    // list has outgrown meanwhile passes through unchanged). A wave iterates as often as its
    // busiest lane (a few times per chunk once the list has filled, against 32 insertions).
    // The keys are unique, so the list is the one inserting every candidate gives.
    const uint64_t kth = key[KM - 1];
    uint32_t m = 0;
#pragma unroll
    for (int u = 0; u < 32; ++u) m |= uint32_t(rank_key(lv[u], c0 + u) > kth) << u;
    m &= (ce >= 32 ? 0xFFFFFFFFu : (1u << ce) - 1u) & (0xFFFFFFFFu << u0);
    while (m) {
      const int u = __builtin_ctz(m);
      m &= m - 1;
      topk_insert<KM>(key, rank_key(s_l[buf][tid][u], c0 + u));
    }
  }
  float v[KM];
  int id[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    v[j] = key_value(key[j]);
    id[j] = key_expert(key[j]);
  }
  uint64_t mask = 0;
  if (n_me < a.N) {
    // p_k = exp(l_k - l_0) / sum_j exp(l_j - l_0), fp32, k ascending
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < KM; ++k)
      if (k < a.K) sum += expf(v[k] - v[0]);
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < a.K) {
        a.idx[n_me * a.K + k] = id[k];
        a.p[n_me * a.K + k] = expf(v[k] - v[0]) / sum;
        const int le = id[k] - a.e0;
        if (le >= 0 && le < a.El) mask |= 1ull << le;
      }
    }
  }
  s_mask[tid] = mask;
  __syncthreads();

  // ---- per-block counts per local expert (value El counts touched tokens, El + 1 those with
  // more than one local pair) ----
  const uint64_t mymask = s_mask[tid];
  const uint64_t lt = (1ull << lane) - 1;
  const int nc = a.El + 2;   // counted values
  auto counted = [&](int e) -> bool {
    return e < a.El ? ((mymask >> e) & 1) : e == a.El ? mymask != 0 : __popcll(mymask) > 1;
  };
  for (int e = 0; e < nc; ++e) {
    bool bit = counted(e);
    uint64_t bal = __ballot(bit);
    if (lane == 0) s_wcnt[wave][e] = __popcll(bal);
  }
  __syncthreads();

  // ---- single-pass decoupled look-back ----
  // Publish this block's aggregates, then each wave takes counted values e = wave, wave+4, ...
  // and inspects predecessors 64 at a time (lane i looks at block base - i): the nearest
  // inclusive prefix ends the walk; aggregates before it are summed; an unpublished
  // predecessor makes the wave re-read the window (bounded).
  if (tid < nc) {
    const uint32_t agg = uint32_t(s_wcnt[0][tid] + s_wcnt[1][tid] + s_wcnt[2][tid] + s_wcnt[3][tid]);
    st_relaxed_u(a.state + int64_t(b) * nc + tid, (b == 0 ? kFlagInc : kFlagAgg) | agg);
  }
  for (int e = wave; e < nc; e += 4) {
    const uint32_t agg = uint32_t(s_wcnt[0][e] + s_wcnt[1][e] + s_wcnt[2][e] + s_wcnt[3][e]);
    uint32_t excl = 0;
    int base = b - 1;
    int spins = 0;
    while (base >= 0) {
      const int j = base - lane;
      const uint32_t w = j >= 0 ? ld_relaxed_u(a.state + int64_t(j) * nc + e) : kFlagInc;
      const uint32_t flag = w & ~kValMask;
      const uint64_t inc = __ballot(flag == kFlagInc);
      const uint64_t inv = __ballot(flag == 0);
      const int first = inc ? __builtin_ctzll(inc) : 64;          // nearest inclusive prefix
      const uint64_t upto = first >= 63 ? ~0ull : ((2ull << first) - 1);   // lanes 0..first
      if (inv & upto & (first == 64 ? ~0ull : upto)) {            // a nearer block unpublished
        if (++spins > kSpinLimit) { set_error(a.err, MOK_ERR_DEVICE_TIMEOUT); break; }
        __builtin_amdgcn_s_sleep(1);
        continue;
      }
      uint32_t part = (uint64_t(1) << lane) & upto ? (w & kValMask) : 0u;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
      excl += part;
      if (first < 64) break;
      base -= 64;
    }
    if (lane == 0) {
      if (b > 0) st_relaxed_u(a.state + int64_t(b) * nc + e, kFlagInc | (excl + agg));
      s_excl[e] = int(excl);
      if (b == a.nblocks - 1) {
        // Last block: inclusive values are the totals.
        const int total = int(excl + agg);
        if (e < a.El) a.hdr[kHdrCounts + e] = total;
        else a.hdr[e == a.El ? kHdrU : kHdrUm] = total;
      }
    }
  }
  __syncthreads();

  // ---- ranks of this block's pairs, and the touched-token lists ----
  const int64_t n = n_base + tid;
  for (int e = 0; e < nc; ++e) {
    bool bit = counted(e);
    uint64_t bal = __ballot(bit);
    if (bit) {
      int r = s_excl[e] + __popcll(bal & lt);
      for (int w = 0; w < wave; ++w) r += s_wcnt[w][e];
      if (e < a.El) {
        int k = 0;
        for (int q = 0; q < a.K; ++q)
          if (a.idx[n * a.K + q] == a.e0 + e) k = q;
        a.rank[n * a.K + k] = r | (__popcll(mymask) == 1 ? kSoleFlag : 0);
      } else if (r < a.N) {
        (e == a.El ? a.touched : a.multi)[r] = int32_t(n);
      }
    }
  }
}

// Offsets need every count; the last block's counts are published before this kernel ends,
// so they are read in k_place (a later launch on the same stream).
struct PlaceArgs {
  const int32_t* idx;
  const int32_t* err;    // the router's error word (workspace)
  int32_t* hdr;
  int32_t* perm;
  int32_t* tokpos;
  int32_t* pcode;        // [rows_max]: perm | kSoleFlag when the pair is its token's only local
                         // pair
  int64_t NK, rows_max;
  int K, e0, El, row_align;
};

__global__ __launch_bounds__(256) void k_place(PlaceArgs a) {
  __shared__ int s_off[kMaxLocalExperts + 1];
  __shared__ int s_cnt[kMaxLocalExperts];
  if (threadIdx.x == 0) {
    int off = 0, P = 0;
    for (int e = 0; e < a.El; ++e) {
      int c = a.hdr[kHdrCounts + e];
      s_cnt[e] = c;
      s_off[e] = off;
      P += c;
      off += (c + a.row_align - 1) / a.row_align * a.row_align;
    }
    s_off[a.El] = off;
    if (blockIdx.x == 0) {
      for (int e = 0; e <= a.El; ++e) a.hdr[kHdrOffsets + e] = s_off[e];
      a.hdr[kHdrP] = P;
      a.hdr[kHdrRows] = off;
      a.hdr[kHdrStatus] = *a.err;
    }
  }
  __syncthreads();
  // Pad rows (MXFP8 alignment) carry pair -1.
  if (a.row_align > 1 && blockIdx.x == 0) {
    for (int q = threadIdx.x; q < a.El * a.row_align; q += blockDim.x) {
      int e = q / a.row_align, i = q % a.row_align;
      int r = s_off[e] + s_cnt[e] + i;
      if (r < s_off[e + 1]) {
        a.perm[r] = -1;
        a.pcode[r] = -1;
      }
    }
  }
  for (int64_t q = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q < a.NK;
       q += int64_t(gridDim.x) * blockDim.x) {
    int le = a.idx[q] - a.e0;
    if (le >= 0 && le < a.El) {
      // A rank outside the expert's range only follows a failed look-back (error word set);
      // never write outside the table.
      const int word = a.tokpos[q];
      const int rank = word & ~kSoleFlag;
      const int row = s_off[le] + rank;
      const bool ok = word >= 0 && rank < s_cnt[le] && row < a.rows_max;
      if (ok) {
        a.perm[row] = int32_t(q);
        a.pcode[row] = int32_t(q) | (word & kSoleFlag);
      }
      a.tokpos[q] = ok ? row : -1;
    } else {
      a.tokpos[q] = -1;
    }
  }
}

// Cut rows into m-tiles: for each minibatch j (rows [jM, (j+1)M)) and each local expert e,
// the intersection with e's real rows, in chunks of kTileM. Ordered by j, then e, then row. One
// wave: lane e owns expert e (El <= 64); per minibatch an exclusive scan over the lanes places
// each expert's tiles.
__global__ __launch_bounds__(64) void k_tiles(const int32_t* hdr, MTile* tiles, int32_t* ntiles,
                                              int El, int M, int64_t tiles_max) {
  const int lane = threadIdx.x;
  const int rows = hdr[kHdrRows];
  const int J = M > 0 ? (rows + M - 1) / M : 0;
  const int off = lane < El ? hdr[kHdrOffsets + lane] : 0;
  const int cnt = lane < El ? hdr[kHdrCounts + lane] : 0;
  int64_t base = 0;
  for (int j = 0; j < J; ++j) {
    const int lo = j * M, hi = min(rows, (j + 1) * M);
    const int r0 = max(lo, off), r1 = min(hi, off + cnt);
    const int n = (lane < El && r1 > r0) ? (r1 - r0 + kTileM - 1) / kTileM : 0;
    int incl = n;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int v = __shfl_up(incl, d, 64);
      if (lane >= d) incl += v;
    }
    const int64_t first = base + incl - n;
    for (int q = 0; q < n && first + q < tiles_max; ++q)
      tiles[first + q] = MTile{j, lane, r0 + q * kTileM, min(kTileM, r1 - r0 - q * kTileM)};
    base += __shfl(incl, 63, 64);
  }
  if (lane == 0) *ntiles = int32_t(min(base, tiles_max));
}

}  // namespace

hipError_t launch_router(const Layout& L, const float* logits, int32_t* idx, float* p,
                         uint8_t* saved, uint8_t* ws, hipStream_t s, bool clear_error) {
  int32_t* hdr = reinterpret_cast<int32_t*>(saved);
  int32_t* wsh = reinterpret_cast<int32_t*>(ws);
  uint32_t* state = reinterpret_cast<uint32_t*>(ws + L.ws_state);
  // One launch clears the workspace header (error word unless asked to keep it, scan ticket),
  // the ring record header (nothing resident until a fused forward writes it), the look-back
  // scan state and the schedule header.
  const int keep = clear_error ? 0 : 1;   // kWsError is word 0
  const FillRange fills[] = {
      {reinterpret_cast<uint32_t*>(wsh) + keep, kWsWords - keep, 0u},
      {reinterpret_cast<uint32_t*>(saved + L.sv_rhdr), kRhWords, 0u},
      {state, int64_t(L.topk_blocks) * (L.El + 2), 0u},
      {reinterpret_cast<uint32_t*>(hdr), kHdrWords, 0u},
  };
  hipError_t err = launch_fill_ranges(fills, 4, s);
  if (err != hipSuccess) return err;
  RouterArgs a{logits, idx, p, hdr,
               reinterpret_cast<int32_t*>(saved + L.sv_tokpos),
               reinterpret_cast<int32_t*>(saved + L.sv_touched),
               reinterpret_cast<int32_t*>(saved + L.sv_multi),
               state, wsh + kWsTicket, wsh + kWsError,
               L.N, L.E, L.K, L.e0, L.El, L.row_align, L.topk_blocks};
  // top-KM list with KM >= K; its first K entries are the top-K
  if (L.K <= 1) hipLaunchKernelGGL(k_topk_scan<1>, dim3(L.topk_blocks), dim3(256), 0, s, a);
  else if (L.K <= 2) hipLaunchKernelGGL(k_topk_scan<2>, dim3(L.topk_blocks), dim3(256), 0, s, a);
  else if (L.K <= 4) hipLaunchKernelGGL(k_topk_scan<4>, dim3(L.topk_blocks), dim3(256), 0, s, a);
  else if (L.K <= 8) hipLaunchKernelGGL(k_topk_scan<8>, dim3(L.topk_blocks), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(k_topk_scan<16>, dim3(L.topk_blocks), dim3(256), 0, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  PlaceArgs pa{idx, wsh + kWsError, hdr, reinterpret_cast<int32_t*>(saved + L.sv_perm),
               reinterpret_cast<int32_t*>(saved + L.sv_tokpos),
               reinterpret_cast<int32_t*>(saved + L.sv_pcode), L.NK,
               L.rows_max, L.K, L.e0, L.El, L.row_align};
  int pblocks = int(cdiv(L.NK, 256));
  if (pblocks > 4096) pblocks = 4096;
  hipLaunchKernelGGL(k_place, dim3(pblocks), dim3(256), 0, s, pa);
  return hipGetLastError();
}

// ---- the router without a caller workspace ---------------------------------------------------
// Its scratch (error word, scan ticket, look-back states) lives in this array, one copy per
// device, kept until the process ends. Host code never passes `scratch` itself to a kernel (on
// the host it names a stand-in, not device memory): it passes the address hipGetSymbolAddress
// returns for the current device, looked up once per device.
static __device__ __align__(256) uint8_t scratch[MOK_SCRATCH_BYTES];

mok_status launch_router_noalloc(const Layout& L, const float* logits, int32_t* idx, float* p,
                                 uint8_t* saved, hipStream_t s) {
  if (router_ws_bytes(L) > int64_t(MOK_SCRATCH_BYTES)) return MOK_ERR_SCRATCH;
  static std::atomic<uint8_t*> ptr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOK_ERR_HIP;
  uint8_t* base = ptr[dev].load(std::memory_order_acquire);
  if (!base) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return MOK_ERR_HIP;
    base = static_cast<uint8_t*>(q);
    ptr[dev].store(base, std::memory_order_release);
  }
  // launch_router clears the header, the scan ticket and the look-back states it uses.
  return launch_router(L, logits, idx, p, saved, base, s) == hipSuccess ? MOK_OK : MOK_ERR_HIP;
}

hipError_t launch_tiles_to(const Layout& L, int M, const uint8_t* saved, MTile* tiles,
                           int32_t* ntiles, hipStream_t s) {
  hipLaunchKernelGGL(k_tiles, dim3(1), dim3(64), 0, s, reinterpret_cast<const int32_t*>(saved),
                     tiles, ntiles, L.El, M, L.tiles_max);
  return hipGetLastError();
}

hipError_t launch_tiles(const Layout& L, int M, const uint8_t* saved, uint8_t* ws, hipStream_t s) {
  return launch_tiles_to(L, M, saved, reinterpret_cast<MTile*>(ws + L.ws_tiles),
                         reinterpret_cast<int32_t*>(ws) + kWsNumTiles, s);
}

}  // namespace mok
