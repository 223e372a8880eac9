/*
 * wfattn.h -- C ABI of libwfattn.so: block-causal mixed-noise chunk attention on MI355X (gfx950).
 *
 * What is computed.  One call is one DiT layer's attention for every head over a query set of
 * one or more latent chunks.  Queries attend fully to the tokens of their own chunk and to every
 * token of every earlier, cleaner chunk, and never to a later, noisier one:
 *   - Wave Forcing project page, "01 - The design gap", column "C - Directed live frontier":
 *     full attention inside a chunk, block-causal across chunks;
 *   - same page, "Key observation": only the reverse noisy -> clean edge is removed;
 *   - KipQuest paper page, "The deep dive": the context of a chunk is the anchor, the clean
 *     history, the live store and the earlier chunks in flight.
 * The K/V of every chunk sit in a read-only pool of fixed-size pages that producers filled in
 * place; attention reads its prefix where it lies, with no assembly (project page, "03 -
 * End-to-end KV transport", "Layout" panel; KipQuest page, "The deep dive", on the paged
 * variant).  For query row i of chunk a and head h:
 *   o[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k_j[h,:]>) * v_j[h,:]
 * over the keys j of every chunk b with chunk_order[b] <= chunk_order[a];
 *   lse[h,i] = log sum_j exp(scale * <q, k_j>)   (natural log).
 *
 * Conventions used by every entry point.
 *   - Device pointers are plain pointers returned by hipMalloc (or torch); the library never
 *     allocates, frees or retains device memory, and never writes q, the pools or the scales.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Device work is
 *     enqueued asynchronously and nothing synchronizes; device faults surface at the caller's
 *     next synchronization.
 *   - Every entry point returns a status; out-parameters are written only on WFATTN_OK.  Every
 *     check except WFATTN_ERR_DEVICE runs before the first HIP call, so nothing is enqueued when
 *     a check fails.  Nothing prints or aborts.
 *   - Layouts (row-major, innermost last):
 *       q, out           [Lq, H, d]            Lq = tokens of the query chunks, concatenated
 *       k_pool, v_pool   [num_pages, page_size, H, d]
 *       lse              [H, Lq] fp32
 *       q_scale          [nqb, H] fp32, nqb = sum over query chunks of ceil(tokens/64); the 64-row
 *                        blocks restart at the first row of each query chunk
 *       k_scale          [num_pages * page_size / 64, H] fp32 (blocks align to pages)
 */
#ifndef WFATTN_H
#define WFATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum wfattn_status {
  WFATTN_OK = 0,
  WFATTN_ERR_NULL = 1,        /* a required pointer is NULL                                    */
  WFATTN_ERR_INVALID = 2,     /* malformed table: token count < 1, order not a permutation    */
                              /* (with ties allowed: an order outside [0, num_chunks)),       */
                              /* page count != ceil(tokens/page_size), duplicate or unknown   */
                              /* query chunk, heads < 1, bad plan handle                      */
  WFATTN_ERR_RANGE = 3,       /* page id out of range or used twice; a size overflows int32   */
  WFATTN_ERR_UNSUPPORTED = 4, /* head_dim not 64/128, page_size not a multiple of 64, device  */
                              /* pointer not 16-byte aligned, dtype or option not supported   */
  WFATTN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than wfattn_workspace_bytes()      */
  WFATTN_ERR_DEVICE = 6,      /* a HIP call or kernel launch failed                           */
  WFATTN_ERR_NOMEM = 7        /* host memory for the plan could not be allocated              */
} wfattn_status;

typedef enum wfattn_dtype {
  WFATTN_BF16 = 0, /* q, pools and out in bf16                                                 */
  WFATTN_FP32 = 1  /* q, pools and out in fp32; converted to bf16 in the workspace, computed   */
                   /* in bf16 like WFATTN_BF16, output written in fp32                         */
} wfattn_dtype;

/* Workspace modes for wfattn_workspace_bytes. */
#define WFATTN_WS_BF16 0
#define WFATTN_WS_FP32 1
#define WFATTN_WS_FP8 2

/* One round's chunk table.  All arrays are host memory; wfattn_plan copies what it needs. */
typedef struct wfattn_chunk_table {
  int32_t num_chunks;           /* chunks whose K/V are in the pool, query chunks included      */
  const int32_t* chunk_tokens;  /* [num_chunks], each >= 1                                      */
  const int32_t* chunk_order;   /* [num_chunks], a permutation of 0..num_chunks-1; 0 = cleanest */
                                /* (oldest).  Key chunk b is visible to query chunk a iff       */
                                /* chunk_order[b] <= chunk_order[a].  A strict order by default: */
                                /* a tie would be a two-way edge, which the method removes.     */
                                /* With wfattn_opts.order_ties = 1, values in [0, num_chunks)   */
                                /* may repeat and chunks of equal order see each other.         */
  const int32_t* page_offsets;  /* [num_chunks+1], CSR into page_ids; chunk c owns exactly      */
                                /* ceil(chunk_tokens[c]/page_size) pages, token u of chunk c is */
                                /* in page page_ids[page_offsets[c] + u/page_size], slot        */
                                /* u % page_size                                                */
  const int32_t* page_ids;      /* [page_offsets[num_chunks]], physical page ids, each in       */
                                /* [0, num_pages) and used at most once                         */
  int32_t num_pages;            /* pool capacity in pages                                       */
  int32_t page_size;            /* tokens per page, a positive multiple of 64                   */
  int32_t num_query_chunks;     /* >= 1                                                         */
  const int32_t* query_chunks;  /* [num_query_chunks], distinct chunk ids; Q/out rows are their */
                                /* tokens concatenated in this order                            */
  int32_t num_heads;            /* H, the same for Q and K/V                                    */
  int32_t head_dim;             /* d: 64 or 128                                                 */
  float softmax_scale;          /* <= 0 means 1/sqrt(head_dim)                                  */
} wfattn_chunk_table;

/* Planner options; zero-initialise for defaults. */
typedef struct wfattn_opts {
  int32_t split_k;   /* 0: the planner decides (whole items, or equal-cost ranges per workgroup */
                     /* cut across items when that balances better); 1: never cut an item's key */
                     /* range; n > 1: cut every item's key range into up to n parts; parts are  */
                     /* merged through their LSEs                                                */
  int32_t xcd_remap; /* 0: default (on); 1: on; -1: off.  Groups one head's work on one XCD     */
  int32_t order_ties; /* 0: chunk_order must be a permutation (the directed frontier: a later,  */
                      /* noisier chunk is never visible).  1: equal orders allowed; chunks of  */
                      /* one order form a window that attends to itself both ways (the live    */
                      /* bidirectional window of Rolling Forcing, Wave Forcing project page,   */
                      /* "01 - The design gap", column "A - Live frontier"), while every       */
                      /* cleaner order stays one-way.  Other values: UNSUPPORTED.              */
  int32_t num_cus;   /* compute units the persistent schedule spreads over: 0 = 256 (a whole      */
                     /* MI355X); else 1..4096, e.g. hipDeviceProp_t.multiProcessorCount of a     */
                     /* partitioned device (wfattn_device_geometry reads both counts)            */
  int32_t num_xcds;  /* L2 domains (XCDs) those CUs are dealt to round-robin by workgroup index:  */
                     /* 0 = 8 when num_cus is 0, else 1; must divide the CU count                 */
  int32_t block_m;   /* query rows per work item: 0 or 256 (the kernels' query tile; fixed)       */
  int32_t block_n;   /* keys per tile: 0 or 64 (the kernels' key tile; fixed).  Other values of  */
                     /* either: UNSUPPORTED                                                      */
} wfattn_opts;

typedef struct wfattn_plan_s wfattn_plan_t; /* opaque, host memory only, immutable once built   */

/* Validate `table` and build the work list: for each query chunk its visible key prefix in
 * clean -> noisy order, query tiles that never cross a chunk, key tiles that never cross a page,
 * and a schedule over the CUs.  The visible set of query chunk a is every chunk b with
 * chunk_order[b] <= chunk_order[a] (Wave Forcing project page, "01 - The design gap", column "C -
 * Directed live frontier" and "Key observation"), and it is read where the producers put it
 * (same page, "03 - End-to-end KV transport", "Layout" panel), so the plan only lists page rows.
 * Host only, no HIP call.  The plan owns copies of everything it needs; free it with
 * wfattn_plan_free.  Errors: NULL, INVALID, RANGE, UNSUPPORTED (an option out of range), NOMEM. */
wfattn_status wfattn_plan(const wfattn_chunk_table* table, const wfattn_opts* opts /* NULL ok */,
                          wfattn_plan_t** plan_out);
void wfattn_plan_free(wfattn_plan_t* plan); /* NULL ok */

/* Lq of the plan (rows of q/out), or -1 for a NULL plan. */
int64_t wfattn_query_rows(const wfattn_plan_t* plan);

/* Bytes of device workspace wfattn_fwd (mode WFATTN_WS_BF16 / _FP32) or wfattn_fwd_fp8
 * (WFATTN_WS_FP8) needs with this plan; 0 for a NULL plan or unknown mode.  The workspace holds
 * the uploaded work list and page table, split-K partials and (fp32 mode) bf16 staging. */
size_t wfattn_workspace_bytes(const wfattn_plan_t* plan, int32_t mode);

/* Copy the plan's work list and page table into `ws` on `stream` (asynchronous; the plan must
 * stay alive until the copy has run).  Do it once per round; every wfattn_fwd / wfattn_fwd_fp8
 * with this plan then reuses the workspace.  Errors: NULL, INVALID, WORKSPACE, UNSUPPORTED
 * (ws not 256-byte aligned), DEVICE. */
wfattn_status wfattn_plan_upload(const wfattn_plan_t* plan, void* ws, size_t ws_bytes,
                                 void* stream);

/* Introspection for host tests.  The schedule is a list of items -- (head, query tile of up to
 * 256 rows of one query chunk) with that chunk's whole visible key-tile prefix -- cut into
 * segments (a key-tile range of one item), which the persistent workgroups run in order; items
 * cut into several segments are merged through their LSEs afterwards.
 * what = 0: summary, 10 int32 (items, key tiles, merge groups, partial slots, block_m, block_n,
 *           most segments of one item, query chunks, segments, workgroups);
 * what = 1: items, 8 int32 each (head, first Q row, rows, first Q-scale block, query chunk
 *           index, visible key tiles, last visible chunk rank, 0);
 * what = 2: key tiles in clean -> noisy order, 2 int32 each (first pool row, valid keys);
 * what = 3: merge groups, 4 int32 each (item, first partial slot, parts, 0);
 * what = 4: segments in workgroup order, 4 int32 each (item, first key tile, end key tile,
 *           partial slot or -1);
 * what = 5: workgroups, 2 int32 each (first segment, end segment);
 * what = 6: chunks by chunk id, 4 int32 each (first key tile, tokens, rank in clean -> noisy
 *           order, last rank visible to it).
 * Copies min(cap, total) int32 into buf (buf may be NULL when cap == 0) and stores the total
 * count of int32 in *n.  Errors: NULL, INVALID (bad plan or unknown `what`). */
wfattn_status wfattn_plan_describe(const wfattn_plan_t* plan, int32_t what, int32_t* buf,
                                   size_t cap, size_t* n);

/* bf16 (or fp32 I/O) forward: out = softmax(scale q k^T) v over each query row's visible keys
 * (the block-causal chunk mask of the project page, "01 - The design gap", column C: full inside a
 * chunk, every earlier and cleaner chunk, never a later and noisier one), with the pages read in
 * place ("03 - End-to-end KV transport", "Layout" panel).
 * q, k_pool, v_pool, out in `dtype`; lse NULL or [H, Lq] fp32.  fp32 I/O converts Q and only
 * the pool rows some query can see to bf16 in the workspace.
 * ws must hold wfattn_workspace_bytes(plan, dtype == WFATTN_FP32 ? WFATTN_WS_FP32 :
 * WFATTN_WS_BF16) bytes and have been filled by wfattn_plan_upload from this plan.  Device
 * pointers must be 16-byte aligned (ws 256-byte).  Padding slots of the pools are never read.
 * Concurrent calls on different streams need different workspaces.  The call only enqueues
 * kernels (no allocation, copy, fill or synchronisation), so it may be captured in a HIP graph
 * once the workspace has been uploaded.
 * Errors: NULL, INVALID, UNSUPPORTED, WORKSPACE, DEVICE. */
wfattn_status wfattn_fwd(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q,
                         const void* k_pool, const void* v_pool, void* out, float* lse, void* ws,
                         size_t ws_bytes, void* stream);

/* The forward of wfattn_fwd (same mask, same pages) with the scores from FP8 operands (the
 * reduced-precision K/V of the project page's "03 - End-to-end KV transport", "Precision" panel):
 * e4m3 (OCP E4M3FN) Q.K^T: q8 [Lq,H,d] and k8_pool [num_pages,page_size,H,d] are
 * e4m3 codes with one fp32 scale per (64-row block, head) (value = decode(code) * scale, the
 * layout of q_scale / k_scale is given at the top of this file); v_pool and out are bf16.
 * Scores are accumulated in fp32 and scaled once per block pair; P.V runs in bf16.
 * ws: wfattn_workspace_bytes(plan, WFATTN_WS_FP8).  Errors as wfattn_fwd. */
wfattn_status wfattn_fwd_fp8(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                             const uint8_t* k8_pool, const float* k_scale, const void* v_pool,
                             void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/* wfattn_fwd_fp8 with the gate of wfattn_fwd_gated: the same flags, need, spin_limit and
 * gate_status, with the same meaning and the same guarantees (k8_pool and v_pool 256-byte
 * aligned).  The key scales are read with the same device-coherent loads as the flags, so a
 * producer may write them while the call runs.
 * Errors: as wfattn_fwd_fp8, plus NULL (flags, need, gate_status), RANGE (spin_limit < 0 or
 * above WFATTN_GATE_SPIN_MAX), UNSUPPORTED (pools not 256-byte aligned). */
wfattn_status wfattn_fwd_fp8_gated(const wfattn_plan_t* plan, const uint8_t* q8,
                                   const float* q_scale, const uint8_t* k8_pool,
                                   const float* k_scale, const void* v_pool, void* out, float* lse,
                                   void* ws, size_t ws_bytes, const uint32_t* flags,
                                   const uint32_t* need, int32_t spin_limit, uint32_t* gate_status,
                                   void* stream);

/* Measurement aid: wfattn_fwd and wfattn_fwd_fp8 with one more argument, a hipEvent_t (passed
 * as void*, created by the caller) that is recorded on `stream` between the attention launch and
 * the launch of the merge of split key ranges, so that the two can be timed apart with events.
 * Otherwise identical.  Errors: as wfattn_fwd / wfattn_fwd_fp8, plus NULL (no event). */
wfattn_status wfattn_fwd_marked(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q,
                                const void* k_pool, const void* v_pool, void* out, float* lse,
                                void* ws, size_t ws_bytes, void* attn_done_event, void* stream);
wfattn_status wfattn_fwd_fp8_marked(const wfattn_plan_t* plan, const uint8_t* q8,
                                    const float* q_scale, const uint8_t* k8_pool,
                                    const float* k_scale, const void* v_pool, void* out, float* lse,
                                    void* ws, size_t ws_bytes, void* attn_done_event, void* stream);

/* Block quantizer: x_bf16 [rows, heads, head_dim] -> x8 (e4m3 codes, same shape) and
 * scales [ceil(rows/64), heads].  For each block of 64 consecutive rows (the last may be short)
 * and head: amax = max |x| over the block (NaN ignored), scale = amax/448, code = round-to-
 * nearest-even e4m3 of x * (448/amax) clamped to [-448, 448]; amax == 0 gives scale 1.  All in
 * fp32.  The K pool is quantized as rows = num_pages*page_size; Q once per query chunk (pass the
 * chunk's first row and its first scale block).  The reduced-precision K/V transport is the
 * project page's "03 - End-to-end KV transport", "Precision" panel.
 * Errors: NULL, UNSUPPORTED (head_dim not 64/128, pointers not 16-byte aligned), RANGE
 * (rows < 0 or heads < 1), DEVICE. */
wfattn_status wfattn_quantize_fp8(const void* x_bf16, int64_t rows, int32_t heads,
                                  int32_t head_dim, uint8_t* x8, float* scales, void* stream);

/* ---- e4m3 K/V storage ---------------------------------------------------------------------
 * K and V both stored as e4m3 (the project page's "03 - End-to-end KV transport", "Precision"
 * panel: FP8 K/V halves the bytes moved; here it halves the K/V bytes the attention gathers).
 * The e4m3 V pool has its own layout, [num_pages * page_size / 64, H, d, 64]: per (64-key block,
 * head) the block's d x 64 codes stored channel by channel, and inside each 32-key half of a
 * channel the 8-key groups in the order 0, 2, 1, 3; codes of slots past a chunk's last token are
 * 0.  One fp32 scale per (64-key block, head), layout as k_scale.  v_pool value of key u of a block
 * = decode(code) * scale. */

/* e4m3 V pool from a bf16 pool: v_bf16 [rows, heads, head_dim] (rows = num_pages * page_size, a
 * multiple of 64) -> v8 (the layout above) and scales [rows/64, heads].  Per (64-row block, head)
 * exactly the rule of wfattn_quantize_fp8 (amax over the finite values, scale = amax/448, RNE
 * codes), except that a NaN value -- a padding slot -- gets code 0.
 * Errors: NULL, UNSUPPORTED (head_dim not 64/128, alignment), RANGE (rows < 0 or not a multiple
 * of 64, heads < 1), DEVICE. */
wfattn_status wfattn_quantize_v_fp8(const void* v_bf16, int64_t rows, int32_t heads,
                                    int32_t head_dim, uint8_t* v8, float* scales, void* stream);

/* Forward with e4m3 Q.K^T (as wfattn_fwd_fp8) and e4m3 V (v8_pool, v_scale: the layout above).
 * Each V code converts exactly to bf16 and P.V runs as a bf16 MFMA with fp32 accumulation; the V
 * block scale is folded into the softmax weights (s_v * P), and the normaliser sums the weights
 * that multiply V.  ws: wfattn_workspace_bytes(plan, WFATTN_WS_FP8).  Errors as wfattn_fwd_fp8. */
wfattn_status wfattn_fwd_fp8kv(const wfattn_plan_t* plan, const uint8_t* q8, const float* q_scale,
                               const uint8_t* k8_pool, const float* k_scale, const uint8_t* v8_pool,
                               const float* v_scale, void* out, float* lse, void* ws,
                               size_t ws_bytes, void* stream);
/* Measurement aid: wfattn_fwd_fp8kv with the event of wfattn_fwd_marked. */
wfattn_status wfattn_fwd_fp8kv_marked(const wfattn_plan_t* plan, const uint8_t* q8,
                                      const float* q_scale, const uint8_t* k8_pool,
                                      const float* k_scale, const uint8_t* v8_pool,
                                      const float* v_scale, void* out, float* lse, void* ws,
                                      size_t ws_bytes, void* attn_done_event, void* stream);

/* ---- producer side: publish a chunk's K/V, and a forward gated on it ------------------------
 * The producers write each chunk's keys and values straight into the slots the consumer reads
 * (project page, "03 - End-to-end KV transport", panel "03 - Layout"), and a consumer uses a
 * chunk's states only once they are complete (KipQuest page, "The deep dive").  Ordering between
 * a producer stream and the consumer's stream is the caller's (an event); the flags let the
 * forward check, chunk by chunk, that what it is about to read is the generation it expects. */

/* Write chunk `chunk`'s K and V, each bf16 [chunk_tokens[chunk], H, d] in projection layout
 * (token-major, 16-byte aligned), into that chunk's pages of k_pool / v_pool (bf16
 * [num_pages, page_size, H, d]): token u goes to page page_ids[page_offsets[chunk] + u/page_size],
 * slot u % page_size.  Slots past the chunk's last token are not written.  If flags is not NULL
 * (uint32 [num_chunks], device), flags[chunk] = generation is stored afterwards, on the same
 * stream, with release ordering.  ws: a workspace filled by wfattn_plan_upload from this plan
 * (it holds the page layout).  The chunk's pages may not be read by other work until this has run.
 * Errors: NULL, INVALID (bad plan, chunk out of range), UNSUPPORTED (alignment), WORKSPACE,
 * DEVICE. */
wfattn_status wfattn_publish_kv(const wfattn_plan_t* plan, int32_t chunk, const void* k_src,
                                const void* v_src, void* k_pool, void* v_pool, uint32_t* flags,
                                uint32_t generation, const void* ws, size_t ws_bytes, void* stream);

/* Publish for the e4m3 path: like wfattn_publish_kv, but K goes into k8_pool (e4m3 codes,
 * [num_pages, page_size, H, d]) with its scales in k_scale ([num_pages * page_size / 64, H]),
 * quantized exactly as wfattn_quantize_fp8 does, one block per 64 tokens of the chunk and head
 * (each block is one page-aligned 64-row block of the pool).  Only the chunk's tokens enter a
 * block's amax; pool slots past the chunk's end are not written.  V is copied as bf16.
 * Errors as wfattn_publish_kv. */
wfattn_status wfattn_publish_kv_fp8(const wfattn_plan_t* plan, int32_t chunk, const void* k_src,
                                    const void* v_src, uint8_t* k8_pool, float* k_scale,
                                    void* v_pool, uint32_t* flags, uint32_t generation,
                                    const void* ws, size_t ws_bytes, void* stream);

/* Fused pre-attention epilogue of one chunk (the producer's step right after its QKV projection:
 * project page, "03 - End-to-end KV transport", on publishing K/V as soon as they are projected,
 * and "Precision", on requantization cost).  qkv: bf16 [chunk_tokens, 3, H, d], the projection
 * output with q, k and v of a token side by side.  cos_t, sin_t: fp32 [chunk_tokens, d/2], the
 * caller's rotary angles per token and channel pair (any positional scheme, e.g. one over frames,
 * height and width).  Q and K are rotated pair by pair:
 *   (x[2i], x[2i+1]) -> (x[2i] c - x[2i+1] s, x[2i] s + x[2i+1] c),
 * every product and sum rounded to fp32 on its own (no fused multiply-add), then the result
 * rounded to bf16 (RNE).  Outputs:
 *   q_out   bf16 [chunk_tokens, H, d] (NULL: not written);
 *   q8, q_scale  e4m3 codes of the rotated bf16 Q with one scale per (64-row block of the
 *           chunk, head), as wfattn_quantize_fp8 (NULL: not written); pass the chunk's place in
 *           the call's q8 / q_scale arrays;
 *   K       rotated, into the chunk's pages: k_pool (bf16) or k8_pool + k_scale (e4m3 as
 *           wfattn_publish_kv_fp8) -- exactly one of k_pool and k8_pool;
 *   V       unchanged, into the chunk's pages of v_pool;
 *   flags   as wfattn_publish_kv.
 * Errors: NULL, INVALID (bad plan, chunk out of range, both or neither of k_pool and k8_pool),
 * UNSUPPORTED (alignment: 16 bytes, scales 4), WORKSPACE, DEVICE. */
wfattn_status wfattn_rope_publish(const wfattn_plan_t* plan, int32_t chunk, const void* qkv,
                                  const float* cos_t, const float* sin_t, void* q_out, uint8_t* q8,
                                  float* q_scale, void* k_pool, uint8_t* k8_pool, float* k_scale,
                                  void* v_pool, uint32_t* flags, uint32_t generation,
                                  const void* ws, size_t ws_bytes, void* stream);

/* The producer's QKV projection with the epilogue of wfattn_rope_publish fused into it: publish
 * K/V right after projecting them, at every layer (KipQuest paper page, "The deep dive"), without
 * the [chunk_tokens, 3, H, d] projection output going through memory.  x: bf16 [chunk_tokens,
 * hidden] (the chunk's hidden states, hidden a multiple of 64); w: bf16 [hidden, 3*H*d], columns
 * ordered (q|k|v, head, channel), so qkv = x . w is the qkv input of wfattn_rope_publish.  The
 * product is accumulated in fp32 on the matrix cores; every other step, output and argument is
 * that of wfattn_rope_publish (rotation of q and k on the fp32 products, bf16 rounding, e4m3 of
 * the bf16 values, page placement, flag).
 * Errors: as wfattn_rope_publish, plus UNSUPPORTED (hidden not a positive multiple of 64), RANGE
 * (x larger than 2 GiB). */
wfattn_status wfattn_qkv_rope_publish(const wfattn_plan_t* plan, int32_t chunk, const void* x,
                                      const void* w, int32_t hidden, const float* cos_t,
                                      const float* sin_t, void* q_out, uint8_t* q8, float* q_scale,
                                      void* k_pool, uint8_t* k8_pool, float* k_scale, void* v_pool,
                                      uint32_t* flags, uint32_t generation, const void* ws,
                                      size_t ws_bytes, void* stream);

/* Upper bound of spin_limit in wfattn_fwd_gated: one poll is followed by a sleep of about 4000
 * clocks, so a gate gives up after about 2 s at most. */
#define WFATTN_GATE_SPIN_MAX (1 << 20)

/* wfattn_fwd (bf16 I/O) with a gate: before a work item reads any key, every chunk b it sees must
 * have flags[b] >= need[b] (uint32 device arrays [num_chunks]).  The item's first wave polls the
 * flags with device-coherent relaxed loads at most spin_limit + 1 times (0: check once, never
 * wait), sleeping between polls; if a poll had to wait, an acquire fence at device scope follows
 * the successful one.  If the flags are still short, the item is skipped and bit 0 of
 * *gate_status (device, set with an atomic OR, never cleared by the library) is set.  Rows of
 * skipped items, and of items merged with them, are then unspecified; every other row is exact.
 * No page of a chunk is read before its flag has been seen, so k_pool and v_pool must be 256-byte
 * aligned (then no cache line holds bytes of two pages).  A wait never deadlocks: it ends after
 * spin_limit polls even if no producer ever runs.
 * Errors: as wfattn_fwd, plus NULL (flags, need, gate_status), RANGE (spin_limit < 0 or above
 * WFATTN_GATE_SPIN_MAX), UNSUPPORTED (pools not 256-byte aligned). */
wfattn_status wfattn_fwd_gated(const wfattn_plan_t* plan, const void* q, const void* k_pool,
                               const void* v_pool, void* out, float* lse, void* ws, size_t ws_bytes,
                               const uint32_t* flags, const uint32_t* need, int32_t spin_limit,
                               uint32_t* gate_status, void* stream);

/* ---- forward without allocation --------------------------------------------------------------
 * For callers that cannot allocate device memory or own a workspace: serving loops and harnesses
 * that forbid hipMalloc, and code that must not allocate while it records work.  wfattn_fwd with
 * the workspace taken from a device array inside the library (WFATTN_NOALLOC_MAX_BYTES = 64 MiB
 * per GPU, held until the process ends).  Each call copies the plan's work list and page table
 * into that array on `stream` (hipMemcpyAsync from the plan's host memory: the plan must stay
 * alive until the copy has run) and then runs the same kernels as wfattn_fwd, so the results are
 * those of wfattn_fwd, bit for bit.  It calls no hipMalloc, hipFree or other allocating routine.
 * All calls on one GPU share its array, which keeps the last call's contents: calls that overlap
 * on one GPU (two streams, two threads) race and give undefined results; calls ordered on one
 * stream are safe.  q, k_pool, v_pool, out, lse as wfattn_fwd.
 * Errors: NULL, INVALID, UNSUPPORTED (dtype, alignment), WORKSPACE (the plan needs more than
 * WFATTN_NOALLOC_MAX_BYTES: wfattn_workspace_bytes(plan, mode) tells), DEVICE.  Every check but
 * DEVICE runs before the first HIP call. */
#define WFATTN_NOALLOC_MAX_BYTES (64u << 20)
wfattn_status wfattn_fwd_noalloc(const wfattn_plan_t* plan, wfattn_dtype dtype, const void* q,
                                 const void* k_pool, const void* v_pool, void* out, float* lse,
                                 void* stream);

/* Static string naming a status. */
const char* wfattn_status_str(wfattn_status status);

/* The compute units and XCDs of HIP device `device`, for wfattn_opts.num_cus / num_xcds
 * (hipDeviceProp_t.multiProcessorCount and the device's XCC count).  Errors: NULL, DEVICE. */
wfattn_status wfattn_device_geometry(int32_t device, int32_t* num_cus, int32_t* num_xcds);

/* ABI version of this header: 3 (2 gave wfattn_opts.order_ties its meaning; 3 replaced the
 * reserved word of wfattn_opts with num_cus and added num_xcds, block_m and block_n). */
int32_t wfattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WFATTN_H */
