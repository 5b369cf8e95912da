/*
 * mkv.h -- C ABI of the mixed FP8 / TQ3 paged decode-attention library for
 * AMD MI355X (gfx950).
 *
 * The method (Minima-KV, arXiv 2608.23834, page 1, Abstract): a paged KV
 * cache keeps Recent and protected Anchor pages in FP8 and moves older
 * non-anchor pages to packed 3-bit TQ3; every live page stays addressable;
 * format-specific kernels compute partial attention states that a globally
 * normalised online-softmax (log-sum-exp) merge combines, with no
 * cache-sized dense dequantised shadow.  Pages of both formats live in one
 * PagedAttention block structure (page 2, "Technical Deep Dive", fourth
 * bullet).  The pages specify no API, bit layout or numerics beyond that;
 * the readings taken are stated at each declaration.
 *
 * General contract for every entry point:
 *  - All pointers named "device" are device pointers owned by the caller.
 *    The library never allocates or frees device memory, never keeps a
 *    pointer after returning, and never synchronises the stream (except the
 *    explicitly synchronous mkv_workspace_status).
 *  - All work is enqueued asynchronously on `stream` (a hipStream_t, passed as
 *    void*; NULL = the legacy default stream) in call order.
 *  - The return value is MKV_OK (0) or a negative MKV_ERR_* code; on error
 *    nothing was enqueued and mkv_last_error() (thread-local) describes the
 *    failed check.  No C++ exception crosses this boundary.
 *  - Host-checkable errors (null pointers, unsupported shapes, misalignment,
 *    counts out of range, a workspace that is too small) are returned as
 *    codes.  Errors found in device data (a page id outside the pool, a tier
 *    byte that contradicts the slab an id points into, a seq_len longer than
 *    the request's block table) are recorded in the workspace status word
 *    (read it with mkv_workspace_status) and the affected requests' outputs
 *    are set to NaN.  NaN or Inf inputs are outside the contract.
 *  - The library keeps no device state of its own that calls share (except
 *    the array of mkv_decode_attn_noalloc): calls whose workspaces and outputs
 *    are disjoint may run concurrently on different streams.
 */
#ifndef MKV_H
#define MKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  MKV_OK = 0,
  MKV_ERR_NULL = -1,      /* a required pointer is NULL                          */
  MKV_ERR_SHAPE = -2,     /* unsupported head_dim / page_size / GQA group         */
  MKV_ERR_ALIGN = -3,     /* slabs and float tensors must be 16-byte aligned     */
  MKV_ERR_WORKSPACE = -4, /* ws_bytes smaller than mkv_decode_workspace_bytes()  */
  MKV_ERR_RANGE = -5,     /* a count or index is out of its valid range          */
  MKV_ERR_HIP = -6        /* a HIP launch failed; message carries the HIP error  */
};

/* Device status bits (mkv_workspace_status). */
enum {
  MKV_DEV_BAD_PAGE_ID = 1,   /* block-table entry outside [0, n_fp8 + n_tq3)        */
  MKV_DEV_BAD_TIER = 2,      /* tier byte contradicts the slab the id points into   */
  MKV_DEV_BAD_SEQ_LEN = 4,   /* seq_len < 0 or longer than the request's block table */
  MKV_DEV_NO_FREE_PAGE = 8,  /* lifecycle: too few free ids, or a stack top outside its array */
  MKV_DEV_NO_PLAN = 16       /* attend / merge on a workspace that holds no plan for this batch */
};

/* Tier map values: one byte per physical page id.  Recent and Anchor pages
 * are FP8, Stale pages are TQ3 (arXiv 2608.23834, page 1, Abstract; the
 * R/A/S names follow page 2, "Enhanced Key Takeaways", first bullet). */
enum { MKV_TIER_RECENT = 0, MKV_TIER_ANCHOR = 1, MKV_TIER_STALE = 2, MKV_TIER_FREE = 0xFF };

/* Head geometry.  Supported: head_dim in {128, 256}, page_size == 16,
 * num_q_heads % num_kv_heads == 0 and G = num_q_heads / num_kv_heads <= 16.
 * Query head i reads KV head i / G (grouped-query attention).  Each KV page
 * is read once per KV head for all G query heads (up to 8 query rows in one
 * matrix-core tile with their fp16 remainders, 9..16 rows in a 16-row tile). */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t page_size;
} mkv_layout;

/* Page formats (frozen: the demote kernel writes them, the decode,
 * materialise and gather kernels read them, and the golden rows in
 * tests/golden/ pin them; any change is a new format).  The pages name the
 * formats but fix none of these details (arXiv 2608.23834, page 1,
 * Abstract: FP8 Recent / Anchor pages, packed TQ3 stale pages); this is the
 * reading this library implements.
 *
 * FP8 page: [kv head][K = 0, V = 1][16 tokens][head_dim] OCP E4M3FN bytes
 *   (round to nearest even, saturating to +-448); value = decode(byte) * the
 *   pool's k_scale or v_scale.
 *
 * TQ3 page: one block of 14 * head_dim bytes per KV head, head h at
 *   h * 14 * head_dim.  Per token, K or V and group of 32 channels: an fp16
 *   scale s = fp16_RNE(fl32(absmax / 3)) (saturating to 65504) of the group's
 *   fp32 values x, and per channel a 3-bit code u = q + 4, q in [-3, 3] the
 *   integer nearest x / s with ties to even (exact fp32 thresholds 0.5 s,
 *   1.5 s, 2.5 s; s = 0 gives q = 0); the value is (u - 4) * s.  Codes go 8
 *   to 3 bytes: a "triple" is a little-endian 24-bit word, slot k at bits
 *   [3k, 3k + 3).  With d = head_dim and G = d / 32 groups, a block is:
 *   [0, 6d)    K codes.  Token t's row starts at byte 3 d t / 8; in it,
 *              quarter j in [0, 4) (channels 8 j .. 8 j + 7 of every group)
 *              starts at byte 3 j G and is G / 4 blocks of 4 triples.
 *              Channel c = 32 g + 8 j + e (e in [0, 8)), with gg = g mod 4,
 *              is in triple 4 floor(g / 4) + 2 (gg mod 2) + floor(e / 4) of
 *              its quarter, at slot 2 (e mod 4) + floor(gg / 2).
 *   [6d, 12d)  V codes.  The triple at byte 6 d + 3 ((16 j + n) G + p), for
 *              j in [0, 4), n in [0, 16), p in [0, G), holds tokens
 *              4 j .. 4 j + 3 of channels a = n d / 16 + 2 p and a + 1:
 *              slot 2 r is (a, token 4 j + r), slot 2 r + 1 is (a + 1,
 *              token 4 j + r).
 *   [12d, 13d) K scales, [13d, 14d) V scales: fp16, the scale of token
 *              t = 4 j + r and group g at element (j G + g) * 4 + r.
 *   Read as 6-bit fields, a block of 4 K triples holds in field f the codes
 *   of channel 8 j + (f mod 8) of groups 4 b + floor(f / 8) (low 3 bits) and
 *   4 b + 2 + floor(f / 8) (high 3 bits); each GPU lane's codes of one token
 *   quarter, or of 4 tokens of 2 V channels, are contiguous. */

/* One layer's page pool.
 *  fp8_slab: device, n_fp8 FP8 pages of mkv_fp8_page_bytes() bytes each
 *            (the FP8 page format above).
 *  tq3_slab: device, n_tq3 TQ3 pages of mkv_tq3_page_bytes() bytes each
 *            (the TQ3 page format above).
 *  tier:     device, n_fp8 + n_tq3 bytes, shared by all layers.
 *  Physical ids [0, n_fp8) are FP8 slots, [n_fp8, n_fp8 + n_tq3) TQ3 slots;
 *  a page with tier R or A must have an FP8 id, tier S a TQ3 id.
 *  k_scale / v_scale: per-layer fp32 FP8 scales (value = decode(byte) * scale),
 *           any finite value > 0.  TQ3 pages demoted from this pool carry
 *           the scale in their fp16 group scales; decode keeps every TQ3 V
 *           product exact and finite for any v_scale, provided the TQ3 pages
 *           were demoted with the same v_scale (their scales are then at most
 *           fp16(448 * v_scale / 3)).  FP8 K scores are (q . code) * k_scale
 *           in fp32.
 *  tq3_signs: NULL, or device int8[head_dim] of +1 / -1 (16-byte aligned): the layer's TQ3
 *            pages are "rotated TQ3".  The pages cite TurboQuant, which
 *            rotates before scalar quantisation (page 1, Abstract and its
 *            references); the rotated variant reads TQ3 that way.  Each
 *            (token, KV head, K or V) row x of head_dim values is stored as the
 *            TQ3 codes of y = c H (signs . x), H the Sylvester-Hadamard matrix
 *            applied by the fast transform in fp32, stage s pairing channels i
 *            and i + 2^s as (a + b, a - b) for s = 0, 1, ..., and c = 1/16 at
 *            head_dim 256, 1/8 at 128.  Demotion rotates; decode with the
 *            matrix-core kernels (single- and multi-query, any G) rotates the
 *            queries of TQ3 pages and rotates their partial states back;
 *            materialisation takes TQ3 values back through the same fast
 *            transform in fp32.  The VALU baseline kernels return
 *            MKV_ERR_RANGE for such a pool.  FP8 pages are never rotated. */
typedef struct {
  uint8_t* fp8_slab;
  uint8_t* tq3_slab;
  const uint8_t* tier;
  int32_t n_fp8;
  int32_t n_tq3;
  float k_scale;
  float v_scale;
  const int8_t* tq3_signs;
} mkv_pool;

/* A decode batch: ragged CSR block tables shared by all layers.
 *  bt_offsets: device int32[batch + 1], request b owns bt_pages[bt_offsets[b] ..
 *              bt_offsets[b+1]); logical page j of request b is entry
 *              bt_offsets[b] + j and holds tokens [16 j, 16 j + 16).
 *  bt_pages:   device int32[bt_capacity], physical page ids.
 *  seq_lens:   device int32[batch], tokens attended per request (after this
 *              step's append: the new token is attended).
 *  bt_capacity: host-known number of entries in bt_pages (>= bt_offsets[batch]). */
typedef struct {
  const int32_t* bt_offsets;
  const int32_t* bt_pages;
  const int32_t* seq_lens;
  int32_t batch;
  int32_t bt_capacity;
} mkv_batch;

/* Bytes of one FP8 page (2 * 16 * num_kv_heads * head_dim) and of one TQ3
 * page (num_kv_heads * 14 * head_dim); 0 for an unsupported layout. */
size_t mkv_fp8_page_bytes(const mkv_layout* layout);
size_t mkv_tq3_page_bytes(const mkv_layout* layout);

/* Append: quantise new tokens to FP8 on Recent pages (arXiv 2608.23834,
 * page 1, Abstract: Recent pages are FP8).
 *  k, v:   device fp32 [batch][n_new][num_kv_heads][head_dim].
 *  pos:    device int32[batch]; token i of request b is written at position
 *          pos[b] + i, i.e. logical page (pos[b]+i)/16, slot (pos[b]+i)%16.
 *  counts: device int32[batch] or NULL; if given only the first counts[b]
 *          (<= n_new) tokens of request b are written.
 * Each byte is e4m3fn_RNE_saturating(fl32(x / scale)) with the pool's k_scale
 * or v_scale.  Target pages must be FP8 ids; a token whose logical page lies
 * outside the request's block table or maps to a non-FP8 id is skipped on
 * device (the caller owns the page table).  n_new in [0, 65535]. */
int mkv_append(const mkv_layout* layout, const mkv_pool* pool,
               const float* k, const float* v, int32_t n_new,
               const int32_t* bt_offsets, const int32_t* bt_pages,
               const int32_t* pos, const int32_t* counts, int32_t batch,
               void* stream);

/* Demote: FP8 page src_fp8[i] -> TQ3 page dst_tq3[i] ("older non-anchor pages
 * move to packed TQ3", arXiv 2608.23834, page 1, Abstract).
 *  src_fp8, dst_tq3: device int32[n]; src in [0, n_fp8), dst in
 *  [n_fp8, n_fp8 + n_tq3) (ids outside are skipped on device).
 * For every head, K and V, token and 32-channel group: x = fl32(decode(e) *
 * scale); a = max|x|; s = fp16_RNE(fl32(a / 3)) (saturating); q = nearest
 * integer to x / s with ties to even, clamped to [-3, 3] (0 when s == 0);
 * code u = q + 4 packed 8 per 3 bytes.  Bit-exact with the oracle.  The
 * caller then rewrites block-table entries and tier bytes (stream-ordered)
 * and may reuse the FP8 slots.  Demoting a page that a concurrent decode on
 * another stream reads is a race the caller must avoid. */
int mkv_demote_pages(const mkv_layout* layout, const mkv_pool* pool,
                     const int32_t* src_fp8, const int32_t* dst_tq3, int32_t n,
                     void* stream);

/* Demote the same pages in n_layers layers with one launch.  The tier map is
 * shared by all layers, so a page that ages leaves FP8 in every layer at once.
 * pools: host array of n_layers descriptors with equal n_fp8 and n_tq3. */
int mkv_demote_pages_layers(const mkv_layout* layout, const mkv_pool* pools,
                            int32_t n_layers, const int32_t* src_fp8,
                            const int32_t* dst_tq3, int32_t n, void* stream);

/* Workspace size for mkv_decode_attn / mkv_decode_attn_layers with at most
 * `batch` requests, `bt_capacity` block-table entries and `n_layers` layers.
 * It holds the plan (compacted per-format page lists, split-K chunk tables)
 * and the partial states; it is bounded by a constant number of split-K
 * chunks, not by context length, so it is never a cache-sized shadow. */
size_t mkv_decode_workspace_bytes(const mkv_layout* layout, int32_t batch,
                                  int32_t bt_capacity, int32_t n_layers);

/* Decode attention for one layer: q fp32 [batch][num_q_heads][head_dim]
 * (device) -> out fp32 [batch][num_q_heads][head_dim] (device) and, if lse is
 * not NULL, lse fp32 [batch][num_q_heads] (natural log of the softmax
 * denominator including its max).  Scores are (q . k) * sm_scale.  The
 * matrix-core kernels carry q * sm_scale * log2(e) as an fp16 pair (about 22
 * significant bits, absolute resolution 2^-25), so |q * sm_scale| must stay
 * below 40000.
 * The FP8 pages of each request are attended by the FP8 partial kernel, the
 * TQ3 pages by the TQ3 partial kernel (split-K over pages, each KV page read
 * once per GQA group), and a log-sum-exp merge combines the partial states
 * (arXiv 2608.23834, page 1, Abstract).  seq_len == 0 gives out = 0 and
 * lse = -inf.  ws: device, 256-byte aligned, ws_bytes >=
 * mkv_decode_workspace_bytes(layout, batch->batch, batch->bt_capacity, 1). */
int mkv_decode_attn(const mkv_layout* layout, const mkv_pool* pool,
                    const mkv_batch* batch, const float* q, float sm_scale,
                    float* out, float* lse, void* ws, size_t ws_bytes,
                    void* stream);

/* mkv_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same decode, the same kernels and bit-identical results, with the
 * workspace in a static device array of the library (32 MiB on each GPU the
 * library runs on, held until the process ends) instead of a caller buffer.
 * The call allocates nothing.  The array belongs to the current device
 * (hipGetDevice); `stream` must be a stream of that device.  Every call on a
 * GPU shares that GPU's array, so calls that overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 * Returns MKV_ERR_WORKSPACE when the batch needs more workspace than the
 * array holds (mkv_decode_workspace_bytes(layout, batch->batch,
 * batch->bt_capacity, 1) > 32 MiB).  Device-data errors give NaN outputs as
 * in mkv_decode_attn; their status word sits in the array and is not
 * exported. */
int mkv_decode_attn_noalloc(const mkv_layout* layout, const mkv_pool* pool,
                            const mkv_batch* batch, const float* q, float sm_scale,
                            float* out, float* lse, void* stream);

/* Decode attention for n_layers (1..64) layers that share one tier map and one set
 * of block tables (the pages' canary decodes 16 full-attention layers per
 * step).  pools: host array of n_layers descriptors with equal n_fp8, n_tq3
 * and tier.  q, out: [n_layers][batch][num_q_heads][head_dim]; lse (nullable)
 * [n_layers][batch][num_q_heads].  The plan is computed once and every
 * kernel launch covers all layers.  ws_bytes >= mkv_decode_workspace_bytes(
 * layout, batch->batch, batch->bt_capacity, n_layers). */
int mkv_decode_attn_layers(const mkv_layout* layout, const mkv_pool* pools,
                           int32_t n_layers, const mkv_batch* batch,
                           const float* q, float sm_scale, float* out,
                           float* lse, void* ws, size_t ws_bytes, void* stream);

/* The decode path in its separate steps, for callers that run layers one at
 * a time (a model's layers are sequential) and reuse one plan per step:
 *
 * mkv_decode_plan: from the tier map (pool->tier, n_fp8, n_tq3) and the block
 *   tables, compact each request's pages into an FP8 list and a TQ3 list and
 *   cut them into split-K chunks sized for n_layers layers per launch.  Writes
 *   the plan into ws (ws_bytes >= mkv_decode_workspace_bytes(layout,
 *   batch->batch, batch->bt_capacity, n_layers)).
 * mkv_attend_fp8 / mkv_attend_tq3: the format-specific partial-attention
 *   kernels over the FP8 (resp. TQ3) chunks of the plan in ws, for n_layers
 *   (<= the plan's) layers; they leave partial states (m, l, acc) in ws.
 * mkv_merge: the log-sum-exp merge of those partial states into out / lse.
 * q, out, lse and pools as in mkv_decode_attn_layers.  The plan must come from
 * mkv_decode_plan with the same layout, batch descriptor and tier state;
 * between mkv_attend_* and mkv_merge the workspace must not be reused.  The
 * plan stamps the workspace with a word derived from the batch, the
 * block-table capacity and the query tokens; a partial-attention or merge call
 * that finds no matching stamp (no plan was made in this workspace, or one for
 * another batch) reads no plan data: it sets MKV_DEV_NO_PLAN in the status and
 * the merge writes NaN outputs.  A stale plan for the same batch shape is not
 * detected. */
int mkv_decode_plan(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch,
                    int32_t n_layers, void* ws, size_t ws_bytes, void* stream);
int mkv_attend_fp8(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                   size_t ws_bytes, void* stream);
int mkv_attend_tq3(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                   size_t ws_bytes, void* stream);
int mkv_merge(const mkv_layout* layout, int32_t n_layers, const mkv_batch* batch, float* out,
              float* lse, void* ws, size_t ws_bytes, void* stream);
/* mkv_attend_partials: mkv_attend_fp8 and mkv_attend_tq3 in one launch (the
 * FP8 and TQ3 work items of the plan side by side in one grid, each running
 * its own format's code); the partial states it leaves in ws are bit-identical
 * to those of the two separate calls. */
int mkv_attend_partials(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                        const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                        size_t ws_bytes, void* stream);

/* mkv_attend: mkv_attend_fp8 + mkv_attend_tq3 + mkv_merge with the two
 * partial kernels in one launch: the FP8 and TQ3 work items of the plan in ws
 * run side by side in one grid (each item runs its own format's kernel code),
 * then the merge.  Same arguments and plan requirements as the separate calls;
 * results are identical to them bit for bit. */
int mkv_attend(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
               const mkv_batch* batch, const float* q, float sm_scale, float* out, float* lse,
               void* ws, size_t ws_bytes, void* stream);

/* mkv_append_attend: mkv_append of each request's newest token followed by
 * mkv_attend, with the append done inside the partial-attention launch (a
 * decode step appends, then attends over tokens [0, seq_len): arXiv
 * 2608.23834, page 1, Abstract, Recent pages in FP8).
 *  k_new, v_new: device fp32 [n_layers][batch][Hkv][head_dim], 16-byte
 *    aligned: K and V of the token at position seq_lens[b] - 1 of request b.
 *    That token's logical page (the request's last) must be an FP8 page of
 *    the pool (tier Recent); it is written exactly as mkv_append writes it.
 *    A request whose last logical page is TQ3 gets NaN outputs and the
 *    status bit MKV_DEV_BAD_TIER (the token is not written).
 *  The other arguments and the plan requirements are those of mkv_attend
 *  (the plan counts the new token: seq_lens include it).  Results, and the
 *  cache bytes written, are identical to mkv_append + mkv_attend.  Needs the
 *  matrix-core kernels (returns MKV_ERR_RANGE otherwise). */
int mkv_append_attend(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                      const mkv_batch* batch, const float* k_new, const float* v_new,
                      const float* q, float sm_scale, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream);

/* Multi-query decode: each request's last n_query tokens (positions
 * seq_len - n_query .. seq_len - 1, already appended) are queries, and query
 * token t attends causally to the tokens at positions [0, seq_len - n_query +
 * t] (none if that range is empty: out = 0, lse = -inf), over the same mixed
 * pages and with the same format-specific partial kernels and log-sum-exp
 * merge as mkv_decode_attn (arXiv 2608.23834, page 1, Abstract: direct
 * heterogeneous decode).  n_query in [1, 16].  pools, n_layers and batch as
 * in mkv_decode_attn_layers (the plan is made by this call).
 *  q, out: device fp32 [n_layers][batch][n_query][num_q_heads][head_dim];
 *  lse (nullable): [n_layers][batch][n_query][num_q_heads].
 *  ws_bytes >= mkv_decode_workspace_bytes_multi(layout, batch->batch,
 *  batch->bt_capacity, n_layers, n_query).  The query rows of a KV head
 *  (n_query * G) are taken 8 at a time when there are at most 8 of them,
 *  else 16 at a time: one split-K work item per chunk, KV head and row
 *  block, so a page is read ceil(n_query * G / 16) times (once for up to 8
 *  rows), not n_query times.  n_query == 1 is mkv_decode_attn_layers.  Needs the
 *  matrix-core kernels for n_query > 1 (MKV_ERR_RANGE otherwise). */
size_t mkv_decode_workspace_bytes_multi(const mkv_layout* layout, int32_t batch,
                                        int32_t bt_capacity, int32_t n_layers, int32_t n_query);
int mkv_decode_attn_multi(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                          const mkv_batch* batch, int32_t n_query, const float* q,
                          float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                          void* stream);

/* Page-table gather (test support): copy the raw bytes of logical pages
 * [0, n_pages) of request b into out (device, n_pages records of
 * mkv_fp8_page_bytes() bytes; a TQ3 page fills the first mkv_tq3_page_bytes()
 * bytes of its record and the rest is zeroed).  Ids outside the pool give a
 * record of 0xFF bytes. */
int mkv_debug_gather(const mkv_layout* layout, const mkv_pool* pool,
                     const int32_t* bt_offsets, const int32_t* bt_pages,
                     int32_t b, int32_t n_pages, uint8_t* out, void* stream);

/* Streaming-read probe (measurement support): read the first
 * floor(bytes / 3584) * 3584 bytes at src (device, 16-byte aligned) once, in
 * units of 3584 bytes (one TQ3 page-head at head_dim 256) with the loads the
 * decode kernels stage pages with (HBM -> LDS, 16 bytes per lane,
 * non-temporal, three units in flight per wave, one 12-wave workgroup per CU),
 * computing nothing; its rate is the streaming ceiling of those loads.  Wave
 * w of the launch XORs the first 32-bit word of each unit it reads into
 * sink[w] (device, sink_words >= 12 words; the launch uses
 * 12 * min(CUs, sink_words / 12) of them), so the XOR of those words is the
 * XOR of every unit's first word. */
int mkv_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);

/* Item trace (measurement support): in a library built with
 * -DMKV_ITEM_TRACE=1 (`python -m mixed_format_paged_amd.build --item-trace`,
 * libmkv_trace.so), the attention kernels record for each workgroup w
 * (w < 4096) 32 words from word 32 w: the 100 MHz constant clock at entry
 * (word 0), once the query fragments of its item are built (1), once the
 * item's partial state is stored (2); the item as pages | tq3 << 32 |
 * KV head << 40 | request << 48 (3); for wave v < 12, the clock when its first
 * page has landed (4 + v) and when it leaves its page loop (16 + v).  A
 * workgroup that runs several items keeps its last one.  Copies the first
 * min(words, 4096 * 32) words to host memory `host` (synchronous, after the
 * device's pending work).  MKV_ERR_RANGE from a library built without the
 * trace (the product build records nothing). */
int mkv_debug_item_trace(uint64_t* host, size_t words);

/* Materialise: dequantise logical pages [page_lo, page_lo + n_pages) of
 * request b to dense bfloat16 K and V.  The pages' quality profile runs on
 * materialised pages while their decode path reads the mixed pages in place
 * without a dense dequantised buffer (arXiv 2608.23834, page 1, Abstract;
 * page 2, "Technical Deep Dive"): this call builds that buffer, for
 * consumers that need dense values and as the measured comparison.
 *  k_out, v_out: device uint16 (bf16 bits) [n_pages * 16][num_kv_heads]
 *    [head_dim], 16-byte aligned; token 16 i + t of the output is slot t of
 *    logical page page_lo + i.
 * Element values: an FP8 page gives bf16_RNE(fl32(decode(e) * scale)) with the
 * pool's k_scale / v_scale; a TQ3 page gives bf16_RNE((u - 4) * s) (exact in
 * fp32 before the rounding); a rotated TQ3 page (tq3_signs) gives
 * bf16_RNE(signs . (H y) / 16) per token row, y = (u - 4) * s and H applied by
 * the format's fast transform in fp32 (stage s pairs channels i and i + 2^s),
 * the butterflies being the only rounding before the bf16 one.  A page's format follows its id (< n_fp8: FP8);
 * the tier map is not read.  A logical page outside the request's block
 * table, or an id outside the pool, gives bf16 NaN (0x7FC0) for all its
 * elements.  Tokens past the request's seq_len are converted like the
 * others.  0 <= b < batch->batch; page_lo, n_pages >= 0 (n_pages == 0: no-op). */
int mkv_materialize(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch,
                    int32_t b, int32_t page_lo, int32_t n_pages, uint16_t* k_out,
                    uint16_t* v_out, void* stream);

/* ---- page lifecycle ------------------------------------------------------
 * Recent and protected Anchor pages stay FP8, older non-anchor pages move to
 * packed TQ3, and every live-request page stays addressable (arXiv
 * 2608.23834, page 1, Abstract).  The pages describe no allocator; these
 * calls implement one on the device, with these readings:
 *  - Free ids are two stacks: fp8_free[0 .. free_tops[0]) holds free FP8 ids,
 *    tq3_free[0 .. free_tops[1]) free TQ3 ids (physical ids n_fp8 ...); a pop
 *    takes the entry just below the top.  A free id has tier MKV_TIER_FREE.
 *  - Which pages are Anchors is the caller's policy: it writes tier A.
 *
 * mkv_lifecycle_step: one decode step adds one token to every request.  A
 *   request whose seq_len is a multiple of 16 starts logical page seq_len/16:
 *   it pops an FP8 id, written into its block-table row, tier Recent.  Its
 *   page count is then n + 1 and, with a Recent window of recent_pages pages,
 *   logical page n - recent_pages leaves the window: if its tier is Recent it
 *   pops a TQ3 id and is demoted (mkv_demote_pages' rule) in every layer, its
 *   block-table entry is switched to the TQ3 id (tier Stale) and its FP8 id
 *   (tier free) is pushed back; Anchor pages stay FP8 and other tiers are
 *   left alone.  seq_lens[b] += 1.  Requests pop in request order and the
 *   freed FP8 ids are pushed in the same order after the pops, so the result
 *   is deterministic.  Run it before the step's append (mkv_append or
 *   mkv_append_attend at position seq_lens[b] - 1) and decode plan.
 *   All or nothing: a full block-table row (bt_offsets[b+1] - bt_offsets[b]
 *   entries), an id outside the pool, a tier that contradicts an id, too few
 *   free ids or a stack top outside its array change nothing and set
 *   MKV_DEV_* bits in the workspace status (mkv_workspace_status).
 *   pools: host array of n_layers descriptors sharing n_fp8, n_tq3 and the
 *   tier map `tier` (device, written).  bt_offsets: device int32[batch + 1];
 *   bt_pages (int32[bt_capacity]), seq_lens (int32[batch]), fp8_free
 *   (int32[n_fp8]), tq3_free (int32[n_tq3]) and free_tops (int32[2]) are
 *   device arrays, read and written.  ws: device, 256-byte aligned, ws_bytes
 *   >= mkv_lifecycle_workspace_bytes(batch).
 * mkv_lifecycle_release: every live page (the first ceil(seq_len / 16)
 *   entries of the row) of the listed requests goes back to its stack, in
 *   list order then logical order; its tier becomes free and the request's
 *   seq_len 0.  requests: device int32[n_req], each listed at most once.
 *   All or nothing as above; ws_bytes >= mkv_lifecycle_workspace_bytes(0). */
size_t mkv_lifecycle_workspace_bytes(int32_t batch);
int mkv_lifecycle_step(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                       const int32_t* bt_offsets, int32_t* bt_pages, int32_t* seq_lens,
                       int32_t batch, int32_t bt_capacity, uint8_t* tier, int32_t* fp8_free,
                       int32_t* tq3_free, int32_t* free_tops, int32_t recent_pages, void* ws,
                       size_t ws_bytes, void* stream);
int mkv_lifecycle_release(const mkv_layout* layout, const mkv_pool* pool,
                          const int32_t* bt_offsets, const int32_t* bt_pages, int32_t* seq_lens,
                          int32_t batch, int32_t bt_capacity, uint8_t* tier, int32_t* fp8_free,
                          int32_t* tq3_free, int32_t* free_tops, const int32_t* requests,
                          int32_t n_req, void* ws, size_t ws_bytes, void* stream);

/* Partial-kernel family of the decode calls (measurement support): 1 (the
 * default) selects the matrix-core kernels, 0 the plain VALU kernels kept as
 * the measured baseline.  Process-wide; a call reads the setting once, when
 * it starts, so calls running on other threads are not affected mid-way.
 * Under 0, mkv_append_attend, multi-query decode and rotated TQ3 pools
 * return MKV_ERR_RANGE (the baseline covers plain single-query decode).  Returns MKV_OK, or MKV_ERR_RANGE for another kind. */
int mkv_set_partial_kind(int32_t kind);

/* Synchronise `stream` and return the device status bits (MKV_DEV_*) left in
 * the workspace by the last decode or lifecycle call on it (0 = no device-data error);
 * negative MKV_ERR_* on failure. */
int mkv_workspace_status(const void* ws, void* stream);

/* Static description of a status code. */
const char* mkv_status_string(int status);

/* Thread-local description of the last failed call on this thread. */
const char* mkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MKV_H */
