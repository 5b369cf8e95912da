// mkv_internal.h -- plan / workspace structures shared by the host API and
// the kernels of the mixed FP8 / TQ3 decode path.
//
// Split-K over pages: each request's pages are split by format (FP8 pages
// read by the FP8 partial kernel, TQ3 pages by the TQ3 partial kernel, as the
// format-specific kernels of arXiv 2608.23834, page 1, Abstract), each
// format's list is cut into chunks of Pp pages, and every (layer, chunk, KV
// head) work item produces one partial state (m, l, acc) for the G query
// heads of its group.  A log-sum-exp merge combines all partials of a
// request, one or two levels deep.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mkv {

constexpr int kMaxLayers = 64;        // layers covered by one launch
// Waves (of 64 lanes) that share one split-K work item: the partial-attention
// workgroup is 12 waves, three per SIMD, one workgroup per CU (the kernel's
// register budget is 512 / kAttendWavesPerSimd VGPRs per lane).
constexpr int kAttendWavesPerSimd = 3;
constexpr int kItemWaves = 4 * kAttendWavesPerSimd;
// split-K work items aimed for per launch: one per CU of the 256
constexpr int kTargetItems = 256;
constexpr int kMinChunkPages = 4;     // smallest chunk
constexpr int kMaxChunkPages = 512;   // largest chunk: longer contexts get more chunks than the target
// Chunks are cut by cost: in the partial-attention kernel an FP8 page-head
// takes about 4/3 the time of a TQ3 page-head (2.3 times the bytes, a third of
// the arithmetic), so an FP8 segment of nf pages at chunk size P (in TQ3 pages)
// takes ceil(4 nf / (3 P)) chunks, never fewer than kMinChunkPages pages each.
constexpr int kFp8WeightNum = 4, kFp8WeightDen = 3;
__host__ __device__ inline int fp8_chunk_count(int nf, int P) {
  if (nf <= 0) return 0;
  const long long den = (long long)kFp8WeightDen * P;
  const int by_weight = (int)(((long long)nf * kFp8WeightNum + den - 1) / den);
  const int by_min = (nf + kMinChunkPages - 1) / kMinChunkPages;
  return by_weight < by_min ? by_weight : by_min;
}
// Upper bound of the chunks of any plan for bt_capacity pages at chunk size
// kMaxChunkPages, in weighted pages (the FP8 weight applied to every page).
__host__ __device__ inline int max_size_chunks(int bt_capacity) {
  const long long den = (long long)kFp8WeightDen * kMaxChunkPages;
  return (int)(((long long)bt_capacity * kFp8WeightNum + den - 1) / den);
}
constexpr int kMaxG = 8;              // query rows of an 8-row block (attend wave states, merge row groups)
constexpr int kMaxGroup = 16;         // query heads per KV head supported (more than 8: 16-row blocks)
constexpr int kDevBadPageId = 1, kDevBadTier = 2, kDevBadSeqLen = 4, kDevNoFreePage = 8, kDevNoPlan = 16;

// Per-request plan fields, each an int32[batch + 1] row of req[].
enum ReqField {
  R_NF = 0,      // FP8 pages of the request
  R_NT,          // TQ3 pages
  R_TAIL,        // tokens on the last logical page (1..16), 0 for an empty request
  R_LASTFMT,     // format of the last logical page: 0 FP8, 1 TQ3, -1 none
  R_INVALID,     // MKV_DEV_* bits of the request; nonzero: outputs are NaN
  R_CF_OFF,      // first FP8 chunk of the request (exclusive prefix; [batch] = total)
  R_CT_OFF,      // first TQ3 chunk of the request
  R_POFF,        // first partial index of the request (per layer)
  R_PREVFMT,     // format of logical page n - 2: 0 FP8, 1 TQ3, -1 none
  R_PREVIDX,     // its absolute index in that format's page list (-1: none)
  R_FIELDS
};

enum TotalField {
  T_NCF = 0,     // FP8 chunks in total
  T_NCT,         // TQ3 chunks in total
  T_NP,          // partials per layer
  T_PPF,         // FP8 chunk size in TQ3 pages (each FP8 page weighs 4/3)
  T_PPT,         // pages per TQ3 chunk
  T_STAMP,       // plan_stamp of the plan (written last by the planning kernel)
  T_FIELDS = 16
};

// Chunk descriptor: x = request, y = first index into the format's page list
// (absolute, in the request's CSR range), z = pages | (tokens on its last
// page << 16) | (kChunkHoldsTail if its last page is the request's last
// logical page), w = partial index within the layer.  Each chunk-table entry
// is four int4: the descriptor, then the first page of each of the
// kItemWaves waves that share a work item (chunk_order(k) for k = 0..11,
// clamped to the chunk's last page), so a workgroup can start staging after
// one load.
constexpr int kChunkHoldsTail = 1 << 30;
constexpr int kChunkInts = 16;        // ints per chunk-table entry
static_assert(kChunkInts == 4 + kItemWaves, "a chunk-table entry holds the first page of every wave");
// Order in which a work item takes its chunk's pages: k-th page taken = page
// (k + count - 1) % count of the chunk when the chunk holds the request's last
// logical page (so that page, the one the in-launch append writes, is the
// first page of wave 0), else page k.  Wave w takes the pages k = w, w + 12, ...
__host__ __device__ inline int chunk_order(int k, int count, bool holds_tail) {
  return holds_tail ? (k == 0 ? count - 1 : k - 1) : k;
}
__host__ __device__ inline int chunk_pages(int z) { return z & 0xffff; }
__host__ __device__ inline int chunk_last_tok(int z) { return (z >> 16) & 0x1f; }
struct Plan {
  int32_t* status;      // [1] MKV_DEV_* bits
  int32_t* totals;      // [T_FIELDS]
  int32_t* req;         // [R_FIELDS][batch + 1]
  int32_t* list_f;      // [bt_capacity] FP8 page ids, request-CSR order
  int32_t* list_t;      // [bt_capacity] TQ3 slot ids (id - n_fp8)
  int4* chunks_f;       // [chunk_cap][2]: descriptor, first page ids
  int4* chunks_t;       // [chunk_cap][2]
  float* q_rot;         // [L][batch][Hq][d]: queries of rotated TQ3 pages (rotated pools only)
  float* part_ml;       // [L][Hkv][np_cap][R][2]  (m in log2 units, l); part_ml_index
  float* part_acc;      // [L][Hkv][d / 32][np_cap][R][32]; part_acc_index
  int batch;
  int bt_capacity;
  int table_cap;        // chunk-table entries per format (independent of the layer count)
  int np_cap;           // partial states per layer in this call's workspace view
  int chunks_target;    // chunks aimed for per format (set by the planning call)
  // Query rows: n_query tokens per request (the request's last n_query
  // positions, causal) times G heads per KV head, R = n_query * G rows, taken
  // in blocks of up to kRowBlock rows; one work item per (chunk, KV head,
  // block).  Partial states hold R rows per KV head.
  int n_query;
  int nblk;
  int rowblk;           // rows per block: 8, or 16 for multi-query with more than 8 rows
};
// The word a plan leaves in totals[T_STAMP], from the fields its consumers
// must share with it (batch, block-table capacity, table capacity, query
// tokens).  The kernels that read a plan check it first: a workspace that
// holds no plan for this batch is refused (kDevNoPlan, NaN outputs), not read.
__host__ __device__ inline int32_t plan_stamp(const Plan& p) {
  uint32_t h = 0x6d6b7650u;
  h = (h ^ (uint32_t)p.batch) * 0x9E3779B1u;
  h = (h ^ (uint32_t)p.bt_capacity) * 0x85EBCA77u;
  h = (h ^ (uint32_t)p.table_cap) * 0xC2B2AE3Du;
  h = (h ^ (uint32_t)p.n_query) * 0x27D4EB2Fu;
  return (int32_t)(h ^ (h >> 15));
}
// Partial-state layout: the states one merge workgroup reads (one layer, KV
// head and 32-channel slice; a request's consecutive partials; all R rows)
// form one contiguous run, R * 32 floats per partial.
constexpr int kStateSlice = 32;
__host__ __device__ inline size_t part_acc_index(int np_cap, int hkv, int d, int R, int layer, int h, int pidx,
                                                 int row, int c) {
  return ((((size_t)layer * hkv + h) * (d / kStateSlice) + c / kStateSlice) * np_cap + pidx) * (size_t)R * kStateSlice +
         (size_t)row * kStateSlice + c % kStateSlice;
}
__host__ __device__ inline size_t part_ml_index(int np_cap, int hkv, int R, int layer, int h, int pidx, int row) {
  return ((((size_t)layer * hkv + h) * np_cap + pidx) * (size_t)R + row) * 2;
}
constexpr int kRowBlock = 8;          // query rows of one work item (MFMA rows 0..7, their remainders 8..15)
constexpr int kMaxQuery = 16;         // query tokens per request

// Workspace layout.  The plan part (status .. chunk tables) has offsets that do
// not depend on the layer count, so a plan made for L layers can be consumed
// by calls for <= L layers; the state part scales with the layer count.
struct WsSizes {
  size_t off_status, off_totals, off_req, off_list_f, off_list_t, off_chunks_f, off_chunks_t;
  size_t off_q_rot, off_part_ml, off_part_acc, total;
  int table_cap, np_cap, chunks_target;
  int n_query, nblk, rowblk;
};

WsSizes workspace_sizes(int hq, int hkv, int d, int batch, int bt_capacity, int n_layers, int n_query = 1);
Plan plan_from_ws(void* ws, const WsSizes& s, int batch, int bt_capacity);

// Per-launch layer table (passed by value as a kernel argument).
struct LayerTable {
  uint8_t* fp8[kMaxLayers];
  uint8_t* tq3[kMaxLayers];
  float k_scale[kMaxLayers];
  float v_scale[kMaxLayers];
  // TQ3 V values u s, with u <= 7, reach 7 * 149.375 v_scale, past the fp16
  // range once v_scale > 62.7.  The P V products then take s 2^-E, exact
  // (see tq3_v_exponent), and the partial state is scaled back by
  // tq3_v_up = 2^E in fp32.
  float tq3_v_up[kMaxLayers];
  const int8_t* signs[kMaxLayers];    // rotated TQ3 pages (NULL: plain TQ3)
  int any_signs;                      // some layer of the table is rotated
};

// Smallest E >= 0 with 7 s 2^-E <= 65504 for every TQ3 V scale s a layer
// with this v_scale can hold (s <= fp16(fl32(448 v_scale) / 3), saturated at
// 65504), so the products u s 2^-E of P V stay finite in fp16; E <= 3.  The
// shift is exact: E > 0 only when v_scale > 62.6, and then every nonzero s is
// at least fp16(2^-9 v_scale / 3) > 0.04, so s 2^-E stays a normal fp16.
inline int tq3_v_exponent(float v_scale) {
  double smax = 448.0 * (double)v_scale / 3.0 * (1.0 + 1.0 / 1024.0);
  if (smax > 65504.0) smax = 65504.0;
  int e = 0;
  while (7.0 * smax > 65504.0 * (double)(1 << e)) ++e;
  return e;
}

struct Geometry {
  int hq, hkv, d, G;
  int n_fp8, n_tq3;
  int partial_kind;     // the call's partial-kernel family (1 matrix cores, 0 VALU), read once per call
};

// ---- launchers (each returns hipGetLastError() of its launch) --------------
hipError_t launch_append(const Geometry& g, uint8_t* fp8_slab, float k_scale, float v_scale,
                         const float* k, const float* v, int n_new, const int32_t* bt_offsets,
                         const int32_t* bt_pages, const int32_t* pos, const int32_t* counts,
                         int batch, hipStream_t stream);
hipError_t launch_demote(const Geometry& g, const LayerTable& lt, int n_layers,
                         const int32_t* src, const int32_t* dst, int n, hipStream_t stream);
// Block-table, tier and free-stack updates done by the demote kernel for the
// page lifecycle (bt_pages == NULL: none).
struct TableUpdate {
  int32_t* bt_pages;
  uint8_t* tier;
  int32_t* fp8_free;
  const int32_t* entry;       // [n] block-table entry of each demoted page
  const int32_t* push_base;   // device: free-stack slot of the first freed FP8 id
};
// Demote src[i] -> dst[i] for i < *n_dev (n_dev == NULL: i < n); n bounds the grid.
hipError_t launch_demote_listed(const Geometry& g, const LayerTable& lt, int n_layers, const int32_t* src,
                                const int32_t* dst, int n, const int32_t* n_dev, const TableUpdate* upd,
                                hipStream_t stream);
hipError_t launch_lifecycle_step(const Geometry& g, const LayerTable& lt, int n_layers, const int32_t* bt_offsets,
                                 int32_t* bt_pages, int32_t* seq_lens, int batch, int bt_capacity, uint8_t* tier,
                                 int32_t* fp8_free, int32_t* tq3_free, int32_t* tops, int recent, int32_t* ws,
                                 hipStream_t stream);
hipError_t launch_lifecycle_release(const Geometry& g, const int32_t* bt_offsets, const int32_t* bt_pages,
                                    int32_t* seq_lens, int batch, int bt_capacity, uint8_t* tier, int32_t* fp8_free,
                                    int32_t* tq3_free, int32_t* tops, const int32_t* requests, int n_req, int32_t* ws,
                                    hipStream_t stream);
hipError_t launch_gather(const Geometry& g, const uint8_t* fp8_slab, const uint8_t* tq3_slab,
                         const int32_t* bt_offsets, const int32_t* bt_pages, int b, int n_pages,
                         uint8_t* out, hipStream_t stream);
hipError_t launch_materialize(const Geometry& g, const uint8_t* fp8_slab, const uint8_t* tq3_slab,
                              float k_scale, float v_scale, const int32_t* bt_offsets,
                              const int32_t* bt_pages, int bt_capacity, int b, int page_lo,
                              int n_pages, uint16_t* k_out, uint16_t* v_out, const int8_t* signs,
                              hipStream_t stream);
// Item trace of the attention kernels (built with MKV_ITEM_TRACE=1 only):
// kTraceBlocks workgroups x kTraceSlots 64-bit words.  read_item_trace copies
// up to `words` of them to host memory: 0 on success, -1 when the library is
// not a trace build, -2 when the copy fails.
constexpr int kTraceBlocks = 4096, kTraceSlots = 32;
int read_item_trace(uint64_t* host, size_t words);

hipError_t launch_plan(const Geometry& g, const uint8_t* tier, const int32_t* bt_offsets,
                       const int32_t* bt_pages, const int32_t* seq_lens, const Plan& plan,
                       hipStream_t stream);
// Partial kernels: `tq3` selects the format.  q is [layers][batch][hq][d];
// qscale = sm_scale * log2(e) (scores are kept in log2 units).
hipError_t launch_partial_valu(bool tq3, const Geometry& g, const LayerTable& lt, int n_layers,
                               const float* q, size_t q_layer_stride, float qscale,
                               const Plan& plan, hipStream_t stream);
// Matrix-core partial kernels: which = 0 FP8 items, 1 TQ3 items, 2 both
// formats' items in one launch.
// New-token rows appended by the partial-attention launch itself (k == NULL:
// none): k, v fp32 [n_layers][batch][Hkv][d], row stride `ls` floats per layer.
struct AppendIn {
  const float* k;
  const float* v;
  size_t ls;
};

hipError_t launch_partial_mfma(int which, const Geometry& g, const LayerTable& lt, int n_layers,
                               const float* q, size_t q_layer_stride, float qscale,
                               const Plan& plan, const AppendIn& ap, hipStream_t stream);
// Streaming-read probe (mkv_stream_read): sink_words >= kItemWaves.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t stream);
size_t stream_read_unit();
// appended: the partials come from a launch with the in-launch append
// (requests whose last logical page is TQ3 then get NaN outputs).
hipError_t launch_merge(const Geometry& g, int n_layers, const Plan& plan, float* out,
                        float* lse, size_t out_layer_stride, size_t lse_layer_stride,
                        hipStream_t stream, bool appended = false);

}  // namespace mkv
