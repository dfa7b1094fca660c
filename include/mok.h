/*
 * mok.h — C ABI of an MI355X (gfx950) implementation of one GPU's share of a deterministic
 * fused Mixture-of-Experts layer: router top-k, schedule table, pull dispatch into a ring
 * token buffer, grouped SwiGLU expert GEMM, push combine with a fixed-order weighted merge,
 * and the backward pass with the router-weight gradient fused into SwiGLU backward.
 *
 * The layer is the one described on the "Mixture-of-Kittens (MoK)" pages ("Mixture-of-Kittens
 * (MoK)"; "Cursor Open-Sources Mixture-of-Kittens (MoK): A Deterministic MoE Training
 * Megakernel for GB300 NVL72 Racks"; "把 MoE 通信延迟从 103μs 压到 18μs：Cursor 开源 GPU
 * 内核 MoK"). Each entry point below names the passage that defines its operation.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named *_dev, and every pointer inside mok_weights / mok_weight_grads, are device
 *   pointers (HBM). mok_desc, mok_weights, mok_weight_grads and mok_sizes are host structs.
 * - Ownership: the caller allocates and frees every buffer. The library never allocates
 *   device memory and keeps no mutable global state apart from the benchmark hook set by
 *   mok_trace_kernel; calls on different streams with different buffers are independent.
 * - Streams: every call is asynchronous and stream-ordered on `stream` (a hipStream_t passed
 *   as void*; NULL is the default stream). No call synchronises the host or copies device
 *   data to the host, except mok_device_status and the tuner mok_autotune.
 * - Errors: argument errors are detected on the host and returned before anything is
 *   launched. A failed launch returns MOK_ERR_HIP. A device-side failure (a bounded wait that
 *   ran out) is recorded in the workspace's error word and reported by mok_device_status.
 * - Determinism: identical inputs give bit-identical outputs on every call. No reduction uses
 *   floating-point atomics; every sum has a fixed order.
 * - Segments: x_seg, out_seg, dout_seg and dx_seg are DEVICE arrays of S device pointers,
 *   each to a BF16 [T][H] row-major block (token t of segment s is global token n = s*T + t).
 *   They stand in for the peer ranks an expert-parallel layer pulls from.
 * - Layouts: BF16 is stored as 16-bit patterns. Weights keep the reduction axis contiguous:
 *   wg, wu [E_loc][I][H]; wd [E_loc][H][I]. Logits are fp32 [N][E]; topk_idx int32 [N][K];
 *   topk_p fp32 [N][K]. A pair id is n*K + k.
 */
#ifndef MOK_H_
#define MOK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOK_ABI_VERSION 5

typedef enum {
  MOK_OK = 0,
  MOK_ERR_NULL = 1,            /* a required pointer is NULL                             */
  MOK_ERR_SHAPE = 2,           /* a size is out of range or inconsistent                 */
  MOK_ERR_DTYPE = 3,           /* unknown dtype, or a field the dtype needs is missing   */
  MOK_ERR_ALIGN = 4,           /* a device pointer is misaligned (16 bytes; packed: 256) */
  MOK_ERR_WORKSPACE = 5,       /* reserved                                               */
  MOK_ERR_RING = 6,            /* ring_bytes below mok_sizes.ring_min_bytes              */
  MOK_ERR_HIP = 7,             /* a HIP runtime call or kernel launch failed             */
  MOK_ERR_DEVICE_TIMEOUT = 8,  /* a device-side bounded wait ran out (see ws error word) */
  MOK_ERR_UNSUPPORTED = 9,     /* not supported on this device                           */
  MOK_ERR_SCRATCH = 10         /* the shape needs more than the static scratch of
                                  mok_schedule_noalloc (MOK_SCRATCH_BYTES)                 */
} mok_status;

typedef enum { MOK_BF16 = 0, MOK_MXFP8 = 1 } mok_dtype;

/* Debug flags (mok_desc.flags). None changes a result. */
#define MOK_FLAG_SKIP_ONE_SIGNAL 0x1u  /* test only: withhold one ring signal so the bounded
                                          wait must expire and report a device timeout     */
#define MOK_FLAG_TRACE 0x2u            /* the fused forward records one mok_trace_record per
                                          item (gathers, gate/up and down tiles) in the
                                          workspace: mok_sizes.trace_offset, up to
                                          trace_records of them (the count is int32 word 3 of
                                          ws; records past the capacity are dropped). The
                                          workspace grows by the trace region.               */
#define MOK_FLAG_POISON 0x4u           /* the fused forward fills a ring slot with NaN bytes
                                          (0xFF) when it is released, before the slot's next
                                          tile is gathered: any read of a released slot shows
                                          up as NaN in the outputs                           */

/* One phase-trace record (MOK_FLAG_TRACE). Times are s_memrealtime ticks (100 MHz). */
typedef struct {
  int32_t workgroup;
  int32_t info;        /* kind (1 prologue gather, 2 gather, 3 gate/up tile, 4 down tile) |
                          xcd << 8 | macrobatch << 16                                      */
  int32_t tile;        /* row tile within its macrobatch                                 */
  int32_t item;        /* the XCD's GEMM item number, or its row-tile index for gathers   */
  uint64_t t_wait;     /* started waiting for the item's inputs                          */
  uint64_t t_begin;    /* inputs there, work starts                                      */
  uint64_t t_end;      /* results stored and signalled                                    */
  uint64_t reserved;
} mok_trace_record;

/* Shapes and tunables of the layer, as the pages state it: hidden size, expert count, top-k,
 * expert intermediate size, BF16 or MXFP8 ("Mixture-of-Kittens (MoK)", benchmark section;
 * "把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ②). */
typedef struct {
  int32_t hidden;              /* H; multiple of 128                                      */
  int32_t num_experts;         /* E; 1..1024                                              */
  int32_t top_k;               /* K; 1..min(E, 16)                                        */
  int32_t intermediate;        /* I; multiple of 128                                      */
  int32_t num_segments;        /* S >= 1 (stand-ins for peer ranks)                       */
  int32_t tokens_per_segment;  /* T >= 1                                                  */
  int32_t expert_begin;        /* e0: first local expert                                  */
  int32_t num_local_experts;   /* E_loc: 1..64, e0 + E_loc <= E                           */
  int32_t minibatch_tokens;    /* M: ring minibatch rows (MXFP8: multiple of 32); 0 = default */
  int32_t comm_cus;            /* CUs given to dispatch/combine in the fused kernels;
                                  0 = library default (16 for BF16; 24 for MXFP8, whose
                                  dispatch also quantises every row)                       */
  int64_t ring_bytes;          /* size of the caller's ring token buffer                  */
  int32_t dtype;               /* mok_dtype                                               */
  uint32_t flags;              /* MOK_FLAG_*                                              */
} mok_desc;

/* Buffer sizes for a descriptor. Everything is sized from host-known bounds only
 * (rows_max = N * min(K, E_loc), plus row padding in MXFP8 mode), so no call needs to read a
 * device-side count back to the host. */
typedef struct {
  size_t saved_bytes;    /* schedule table; written by mok_schedule / mok_layer_fwd, read by
                            every later stage and by mok_layer_bwd                          */
  size_t ws_bytes;       /* scratch of one call (counters, error word, tile tables, ...,
                            and room to pack the weights when mok_weights.packed is NULL)   */
  size_t bwd_ws_bytes;   /* scratch of mok_layer_bwd (>= ws_bytes): replayed activations,
                            gathered dOut, dg|du, transposed weight-gradient operands        */
  size_t slots_bytes;    /* push/receive buffer Z: N*K rows of H BF16, indexed by pair id   */
  size_t xd_bytes;       /* staged path: dispatched rows in expert order                    */
  size_t act_bytes;      /* staged path: g|u and h per dispatched row                       */
  size_t wq_bytes;       /* MXFP8: one quantised weight tensor (codes + scales)             */
  int64_t rows_max;      /* bound on expert-order rows                                       */
  int32_t ring_slots;    /* R: activation slots of the fused-path ring, i.e. row tiles whose
                            g|u the backward finds resident (8 XCD shares, each 3 gather
                            slots, 3 h slots, then R/8 activation slots)                     */
  int32_t minibatch;     /* M actually used (after the default is applied)                  */
  int64_t slot_bytes;    /* bytes of one activation slot (g|u of 256 rows)                  */
  /* Layout of the schedule table inside `saved` (byte offsets). Words 0..191 are a header:
   * [0] P (local pairs), [1] rows (P plus MXFP8 padding), [2] U (touched tokens),
   * [3] touched tokens with several local pairs, [4] the router's device-side status,
   * [16 + e] count of local expert e, [96 + e] first row of expert e (e = 0..E_loc). */
  int64_t perm_offset;    /* int32 [rows_max]: expert-order row -> pair id (-1: pad row)     */
  int64_t tokpos_offset;  /* int32 [N*K]: pair id -> row (-1: not local)                     */
  int64_t touched_offset; /* int32 [N]: tokens with a local pair, ascending (first U valid)  */
  int64_t x_slot_bytes;   /* bytes of one gather slot of the ring (X rows of 256 tokens)      */
  int64_t ring_min_bytes; /* smallest ring_bytes the fused path accepts (two activation slots
                             per XCD share after its gather and h slots)                    */
  /* The grouped-GEMM tile table inside `ws`, written by mok_expert_ffn and mok_layer_fwd:
   * int32 quads {minibatch j, local expert, first expert-order row, rows}, ordered by j, then
   * expert, then row; tiles never straddle an expert or a minibatch. Its length is int32 word
   * 2 of ws. */
  int64_t tiles_offset;
  int64_t tiles_max;
  int64_t trace_offset;   /* MOK_FLAG_TRACE: byte offset of the records inside ws (else 0)  */
  int64_t trace_records;  /* capacity in records (0 without MOK_FLAG_TRACE)                 */
  int64_t h_slot_bytes;   /* bytes of one h slot of the ring (h of 256 rows: BF16, or MXFP8
                             codes and scales along I)                                      */
  int64_t packed_bytes;   /* size of the packed weights mok_pack_weights writes (BF16: 12 E_loc
                             H I bytes; MXFP8: 6 E_loc H I code bytes, then 6 E_loc H I / 32
                             scale bytes)                                                   */
} mok_sizes;

/* Expert weights (device pointers). BF16 mode uses wg/wu/wd; MXFP8 mode uses E4M3 codes
 * with UE8M0 scales per 32 elements along each GEMM's reduction axis, produced by
 * mok_quantize_mx:
 *   forward : wg_q/wg_s, wu_q/wu_s = Wg, Wu [E_loc][I][H] blocked along H;
 *             wd_q/wd_s = Wd [E_loc][H][I] blocked along I;
 *   backward: wgt_q/wgt_s, wut_q/wut_s = Wg^T, Wu^T [E_loc][H][I] blocked along I;
 *             wdt_q/wdt_s = Wd^T [E_loc][I][H] blocked along H.
 * Codes have the shape of the matrix, scales the shape with the last axis divided by 32. */
typedef struct {
  const void* wg;
  const void* wu;
  const void* wd;
  const uint8_t *wg_q, *wg_s, *wu_q, *wu_s, *wd_q, *wd_s;
  const uint8_t *wgt_q, *wgt_s, *wut_q, *wut_s, *wdt_q, *wdt_s;
  /* Optional: the weights packed by mok_pack_weights (packed_bytes, 256-byte aligned), made
   * once per weight update. Every expert GEMM reads its weight operand from these planes; when
   * NULL, each call first packs the planes it needs from the fields above into its own
   * workspace (one launch per plane). */
  const void* packed;
} mok_weights;

/* Weight gradients, fp32, same layouts as the BF16 weights. Fully overwritten. */
typedef struct {
  float* dwg;
  float* dwu;
  float* dwd;
} mok_weight_grads;

int mok_abi_version(void);
const char* mok_status_str(mok_status s);

/* Validate `desc` and report every buffer size. Host only; launches nothing. */
mok_status mok_query_sizes(const mok_desc* desc, mok_sizes* sizes);

/* The three sizes a caller of the fused entry points needs, in the form the layer's scope
 * states them: *ws_bytes = workspace of mok_layer_fwd and mok_layer_bwd (the backward's, which
 * is the larger), *saved_bytes = the schedule table and ring record, *slot_bytes = the
 * push/receive buffer (N*K rows of H BF16). Host only; same validation as mok_query_sizes. */
mok_status mok_workspace_size(const mok_desc* desc, size_t* ws_bytes, size_t* saved_bytes,
                              size_t* slot_bytes);

/* Two-wave minibatch floor: the smallest minibatch for which the gate/up grouped GEMM
 * (N = 2*I columns) gives every one of `cus` compute units at least two tiles of
 * tile_m x tile_n. The pages size minibatches this way ("Mixture-of-Kittens (MoK)", section
 * on overlap granularity; "把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ②). Host only. */
int64_t mok_two_wave_floor(int32_t cus, int32_t tile_m, int32_t tile_n, int32_t intermediate);

/* Router top-k + gating + schedule table ("把 MoE 通信延迟从 103μs 压到 18μs", section 02:
 * the router decides each token's experts, then the table counts tokens per expert, fixes
 * their rows on the receiving side and keeps each expert's rows contiguous; "Mixture-of-Kittens
 * (MoK)", section on pull dispatch: one table serves all four transfer operations).
 *   logits_dev   fp32 [N][E]
 *   topk_idx_dev int32 [N][K] out: experts by descending logit, ties to the lower id
 *   topk_p_dev   fp32 [N][K] out: softmax over the K selected logits
 *   saved_dev    out: counts, offsets, row -> pair map (perm), pair -> row map (tokpos),
 *                touched-token list; P, U and J stay on the device
 *   ws_dev       scratch (ws_bytes) */
mok_status mok_schedule(const mok_desc* desc, const float* logits_dev, int32_t* topk_idx_dev,
                        float* topk_p_dev, void* saved_dev, void* ws_dev, void* stream);

/* mok_schedule for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same outputs, bit for bit, with
 * the router's scratch (its error word and the look-back scan state, 4 * ceil(N/256) *
 * (E_loc + 2) bytes plus 256) taken from a static array of MOK_SCRATCH_BYTES that the library
 * holds on each device it runs on until the process ends, instead of a caller's workspace.
 *   - No allocation or free happens in the call. The first call on a device looks the array up
 *     (hipGetSymbolAddress) with that device current.
 *   - Returns MOK_ERR_SCRATCH, before launching anything, when N and E_loc need more scratch.
 *   - Every call on one device shares that device's array: calls that overlap in time on one
 *     device (other streams, other host threads) race and give undefined results; calls ordered
 *     on one stream are fine. The call clears what it needs before use.
 *   - A device-side failure (the scan's bounded wait) is recorded in int32 word 4 of saved_dev's
 *     header (mok_device_status, which reads a workspace, does not see it). */
#define MOK_SCRATCH_BYTES (1u << 20)
mok_status mok_schedule_noalloc(const mok_desc* desc, const float* logits_dev,
                                int32_t* topk_idx_dev, float* topk_p_dev, void* saved_dev,
                                void* stream);

/* The router's gate projection, the step before top-k: logits[n][e] = sum_h X[n][h] W_r[e][h]
 * for every token n of the segments (fp32 [N][E], BF16 operands, fp32 accumulation in a fixed
 * order). The result feeds mok_schedule / mok_layer_fwd. The router-weight gradient is part of
 * the layer ("Mixture-of-Kittens (MoK)", benchmark section; "Cursor Open-Sources
 * Mixture-of-Kittens (MoK)", Technical Details).
 *   wr_dev  BF16 [E][H] (the reduction axis contiguous); E must be a multiple of 4. */
mok_status mok_router_fwd(const mok_desc* desc, const void* const* x_seg_dev, const void* wr_dev,
                          float* logits_dev, void* stream);

/* Backward of the gate projection, given dlogits (from mok_layer_bwd when every expert is
 * local, or completed at the source in expert parallelism):
 *   dwr_dev  fp32 [E][H], overwritten: dW_r = dlogits^T X;
 *   dx_seg   BF16 token rows, updated in place: dX[n] = bf16(float(dX[n]) + dlogits[n] W_r)
 *            for every token n (write or zero dX first);
 *   ws_dev   mok_router_ws_size bytes (X^T, dlogits^T, W_r^T, zero-padded).
 * dlogits enter the contraction rounded to BF16. */
mok_status mok_router_ws_size(const mok_desc* desc, size_t* ws_bytes);
mok_status mok_router_bwd(const mok_desc* desc, const void* const* x_seg_dev, const void* wr_dev,
                          const float* dlogits_dev, float* dwr_dev, void* const* dx_seg_dev,
                          void* ws_dev, void* stream);

/* Pull dispatch, staged form: the receiving side reads every routed token row from its
 * source segment and writes it in expert order ("Mixture-of-Kittens (MoK)", section on pull
 * dispatch; "把 MoE 通信延迟从 103μs 压到 18μs", section 03 part ①). In MXFP8 mode each row is
 * quantised along H on the way (same page, section 03 part ③).
 *   x_seg_dev  device array of S pointers to BF16 [T][H]
 *   xd_dev     out, xd_bytes: BF16 [rows_max][H], or (MXFP8) codes [rows_max][H] followed by
 *              scales [rows_max][H/32]; only rows < rows(P) are written */
mok_status mok_dispatch(const mok_desc* desc, const void* saved_dev,
                        const void* const* x_seg_dev, void* xd_dev, void* ws_dev, void* stream);

/* Grouped SwiGLU expert FFN, staged form, with the push-combine epilogue: for each local
 * expert over its rows, g = x Wg^T, u = x Wu^T, h = silu(g) u, y = h Wd^T; y is written in
 * BF16 to slots[pair id] (the token's receive slot) ("把 MoE 通信延迟从 103μs 压到 18μs",
 * section 03 parts ① and ②).
 *   xd_dev     from mok_dispatch
 *   act_dev    out, act_bytes: g|u BF16 [rows_max][2I] then h ([rows_max][I] BF16, or MXFP8
 *              codes [rows_max][I] + scales [rows_max][I/32])
 *   slots_dev  out: BF16 [N*K][H]; only local pairs' rows are written */
mok_status mok_expert_ffn(const mok_desc* desc, const void* saved_dev, const void* xd_dev,
                          const mok_weights* w, void* act_dev, void* slots_dev, void* ws_dev,
                          void* stream);

/* Final weighted merge ("把 MoE 通信延迟从 103μs 压到 18μs", section 04: the benchmarked layer
 * ends with it): out[n] = bf16( sum over k ascending with idx[n,k] local of
 * p[n,k] * float(slots[n*K+k]) ) for every token with at least one local pair. With
 * topk_p_dev == NULL the sum is unweighted (the input-gradient merge of backward).
 * Rows of tokens with no local pair are not written. */
mok_status mok_combine(const mok_desc* desc, const void* saved_dev, const int32_t* topk_idx_dev,
                       const float* topk_p_dev, const void* slots_dev, void* const* out_seg_dev,
                       void* ws_dev, void* stream);

/* Fused forward: schedule, then one persistent kernel whose compute units are split between
 * dispatch/combine workers and GEMM workers, coordinated through counters in HBM with no
 * host synchronisation; tokens flow through the fixed-size ring in minibatches of M rows
 * ("把 MoE 通信延迟从 103μs 压到 18μs", section 03 parts ② and ③; "Mixture-of-Kittens (MoK)",
 * section on the ring token buffer). Outputs as mok_schedule + mok_combine, except that
 * slots_dev is scratch here: the down GEMM writes the output row of a token with a single
 * local pair itself (bf16(p * bf16(y)), the merge over one term), and only pairs of tokens
 * with several local pairs pass through the slots. ring_bytes must
 * be at least mok_sizes.ring_min_bytes (else MOK_ERR_RING); the ring keeps g|u of the last
 * R = mok_sizes.ring_slots row tiles (256 expert-ordered rows each) for mok_layer_bwd.
 * SwiGLU: h = silu(g) u is formed from the BF16-rounded g and u that the ring keeps, so the
 * backward recomputes exactly the h the down GEMM used. */
mok_status mok_layer_fwd(const mok_desc* desc, const void* const* x_seg_dev,
                         const float* logits_dev, const mok_weights* w,
                         void* const* out_seg_dev, int32_t* topk_idx_dev, float* topk_p_dev,
                         void* saved_dev, void* ring_dev, void* slots_dev, void* ws_dev,
                         void* stream);

/* Macrobatch interleave: `num_macro` consecutive layer calls (1..8 macrobatches, each with its
 * own tokens, logits, outputs, schedule table and slots, the same weights) in one persistent
 * launch. The pages' ring buffer interleaves dispatch and combine at macrobatch boundaries: the
 * previous macrobatch's combine and the next one's dispatch run at the same time
 * ("Mixture-of-Kittens (MoK)", ring token buffer section; "Cursor Open-Sources
 * Mixture-of-Kittens (MoK)", Technical Details; "把 MoE 通信延迟从 103μs 压到 18μs", section 03
 * part ③). Here the row tiles of all macrobatches form one list taken in macrobatch order, so
 * macrobatch b+1 is pulled and computed while macrobatch b's last tiles finish and push their
 * results; then each macrobatch's merge of tokens with several local pairs runs.
 *   x_seg_dev, logits_dev, out_seg_dev, topk_idx_dev, topk_p_dev, saved_dev, slots_dev: HOST
 *     arrays of num_macro entries, each what mok_layer_fwd takes for that call (distinct
 *     outputs per macrobatch);
 *   ring_dev: one ring, as for mok_layer_fwd; ws_dev: mok_macro_ws_size(desc, num_macro) bytes.
 * Every output equals, bit for bit, that of num_macro separate mok_layer_fwd calls. Each saved
 * table records the ring slots its own tiles still hold at the end, so mok_layer_bwd of any
 * macrobatch (in any order, ring untouched in between) reuses them. */
mok_status mok_macro_ws_size(const mok_desc* desc, int32_t num_macro, size_t* ws_bytes);
mok_status mok_layer_fwd_macro(const mok_desc* desc, int32_t num_macro,
                               const void* const* const* x_seg_dev, const float* const* logits_dev,
                               const mok_weights* w, void* const* const* out_seg_dev,
                               int32_t* const* topk_idx_dev, float* const* topk_p_dev,
                               void* const* saved_dev, void* ring_dev, void* const* slots_dev,
                               void* ws_dev, void* stream);

/* Fused backward of L = sum_n <dOut[n], out[n]>, walking the ring in reverse so the
 * minibatches still resident after the forward are not replayed ("Mixture-of-Kittens (MoK)",
 * section on the ring token buffer; "Cursor Open-Sources Mixture-of-Kittens (MoK)",
 * Technical Details). Per minibatch: pull dOut rows (reverse combine), a = dOut Wd_e with
 * dp = <a, h>, dh = p a and SwiGLU backward fused in the epilogue (the router-weight
 * gradient inside SwiGLU backward, "Mixture-of-Kittens (MoK)", benchmark section),
 * dx = dg Wg_e + du Wu_e pushed to slots[pair id] (a token with a single local pair gets its
 * dX row written directly), and the weight gradients. Then the dX merge over k ascending of the
 * tokens with several local pairs and, when E_loc == E, dlogits.
 *   dp_dev       fp32 [N][K], written at local pairs only
 *   dlogits_dev  fp32 [N][E] or NULL; must be NULL unless E_loc == E
 *   g            weight gradients, fully overwritten
 *   ring_dev     the ring the matching mok_layer_fwd used, untouched since (or NULL). Row tiles
 *                whose ring slot still holds them give back their g|u and h; all other rows
 *                are replayed (X gathered again, gate/up recomputed). After the staged path
 *                (mok_schedule ...) or with NULL every row is replayed. The results are the
 *                same bit for bit either way.
 * saved_dev must hold the state the matching forward left (schedule table and ring record). */
mok_status mok_layer_bwd(const mok_desc* desc, const void* const* dout_seg_dev,
                         const void* const* x_seg_dev, const mok_weights* w,
                         const int32_t* topk_idx_dev, const float* topk_p_dev,
                         const void* saved_dev, void* ring_dev, void* slots_dev,
                         void* const* dx_seg_dev, float* dp_dev, float* dlogits_dev,
                         const mok_weight_grads* g, void* ws_dev, void* stream);
/* (mok_layer_bwd: ws_dev must hold bwd_ws_bytes; the call clears its error word first.) */

/* MXFP8 quantiser (OCP MX v1.0: E4M3 codes, one UE8M0 scale per 32 elements; shared scale
 * 2^(floor(log2 amax) - 8), round to nearest even, saturate to +-448, amax 0 -> scale 0).
 * Quantises `batch` BF16 matrices [rows][cols]. transpose == 0: blocks run along cols, codes
 * [batch][rows][cols], scales [batch][rows][cols/32]. transpose == 1: the output is the
 * transposed matrix blocked along the input's rows: codes [batch][cols][rows], scales
 * [batch][cols][rows/32]. The blocked axis must be a multiple of 32. */
mok_status mok_quantize_mx(int32_t batch, int32_t rows, int32_t cols, const void* src_dev,
                           int32_t transpose, uint8_t* codes_dev, uint8_t* scales_dev,
                           void* stream);

/* Weight packing, once per weight update: writes the weight operands of the four expert GEMMs
 * into `packed_dev` (mok_sizes.packed_bytes, 256-byte aligned) in the order the MFMA matrix
 * cores read them, so that each GEMM loads its weight fragments with whole 1 KB reads straight
 * into registers instead of staging them through LDS. Four planes per set of local experts: Wg
 * and Wu interleaved for the gate/up GEMM, Wd for the down GEMM, Wd^T for the a GEMM and
 * [Wg^T | Wu^T] for the dx GEMM. BF16 (from wg, wu, wd): in a plane of R rows and reduction
 * length K, 1 KB block (n32, k16) at offset (n32 K/16 + k16) KB holds in its 16-byte lane l the
 * elements 16 k16 + 8 (l/32) .. +7 of row 32 n32 + l%32. MXFP8 (from the codes and scales of
 * both blockings): 2 KB block (n32, k64) holds in lane l of its first 1 KB the codes 64 k64 +
 * 16 (l/32) .. +15 of row 32 n32 + l%32 and in its second 1 KB the 16 codes 32 further; the
 * scale planes follow the code planes with 64 bytes per block, byte l the scale of that row's
 * code block 2 k64 + l/32. The layout is the library's own; callers only pass the buffer back
 * in mok_weights.packed. Stream-ordered, no host sync. */
mok_status mok_pack_weights(const mok_desc* desc, const mok_weights* w, void* packed_dev,
                            void* stream);

/* One measured configuration of mok_autotune. */
typedef struct {
  int32_t minibatch_tokens;   /* M tried                                                      */
  int32_t comm_cus;           /* dispatch CUs tried                                           */
  float ms;                   /* median time of mok_layer_fwd over the repetitions            */
} mok_tune_result;

/* Per-shape tuner of the fused forward's minibatch size and compute-unit split: the pages note
 * that a different hidden size, top-k or expert count needs a different minibatch and a
 * different number of communication SMs ("把 MoE 通信延迟从 103μs 压到 18μs", section 05;
 * section 03 part ② on the minibatch trade-off). Runs mok_layer_fwd, on the caller's inputs and
 * buffers (sized for `desc`), for every candidate pair
 *   comm_cus in {8, 16, 24, 32, 48} (clipped to the device), and
 *   minibatch_tokens in {M, 2M, 4M, all rows} (M = desc's minibatch after its default; larger
 *   minibatches never need larger buffers),
 * `reps` times each (after one warm-up call), and writes the fastest into *tuned (a copy of desc
 * with those two fields set) and its median time into *best_ms. If `results` is not NULL, up to
 * `max_results` measured candidates are written there and their count to *n_results.
 * Outputs of the layer do not depend on the choice (the same bit-identical results for every
 * candidate). Unlike every other call this one SYNCHRONISES the host with `stream` (it
 * measures): call it once per shape, outside timed regions and graph capture. It allocates no
 * device memory (HIP events only). A device-side failure aborts with its status. */
mok_status mok_autotune(const mok_desc* desc, const void* const* x_seg_dev,
                        const float* logits_dev, const mok_weights* w, void* const* out_seg_dev,
                        int32_t* topk_idx_dev, float* topk_p_dev, void* saved_dev, void* ring_dev,
                        void* slots_dev, void* ws_dev, void* stream, int32_t reps,
                        mok_desc* tuned, float* best_ms, mok_tune_result* results,
                        int32_t max_results, int32_t* n_results);

/* Waits for `stream`, then reads the workspace error word. The only synchronising call apart
 * from mok_autotune. */
mok_status mok_device_status(const void* ws_dev, void* stream, mok_status* out);

/* Number of compute units of the current device (0 if unknown). */
int32_t mok_device_cus(void);

/* Measurement hook (benchmarks only): from the next call on, the library records `before`
 * (a hipEvent_t) on the call's stream right before it launches the kernel `kernel` and `after`
 * right after it; MOK_TRACE_NONE (or NULL events) switches it off. Kernels:
 * MOK_TRACE_FUSED_FWD   the persistent forward kernel of mok_layer_fwd;
 * MOK_TRACE_BWD_GEMM1   mok_layer_bwd's first GEMM launch: a = dOut Wd (with dp and SwiGLU
 *                       backward) and dW_down;
 * MOK_TRACE_BWD_GEMM2   its second: dx (pushed to the slots), dW_gate and dW_up;
 * MOK_TRACE_DISPATCH    the pull-dispatch gather kernel of mok_dispatch;
 * MOK_TRACE_COMBINE     the merge kernel (mok_combine, and the merges of tokens with several
 *                       local pairs after the fused forward and in the backward).
 * Process-wide setting, not thread-safe; it changes no result. */
#define MOK_TRACE_NONE 0
#define MOK_TRACE_FUSED_FWD 1
#define MOK_TRACE_BWD_GEMM1 2
#define MOK_TRACE_BWD_GEMM2 3
#define MOK_TRACE_DISPATCH 4
#define MOK_TRACE_COMBINE 5
mok_status mok_trace_kernel(int32_t kernel, void* before, void* after);

#ifdef __cplusplus
}
#endif

#endif /* MOK_H_ */
