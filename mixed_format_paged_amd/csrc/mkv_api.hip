// mkv_api.hip -- the C ABI (include/mkv.h): argument validation, workspace
// layout and kernel launches for mixed FP8 / TQ3 paged decode attention.
//
// Decode step (arXiv 2608.23834, page 1, Abstract: format-specific kernels
// produce partial attention states, a globally normalised online-softmax
// merge combines them, no dense shadow):
//   plan (once per call, shared by every layer) -> FP8 partial kernel ->
//   TQ3 partial kernel -> merge, all enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <mutex>

#include "mkv.h"
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

// Which partial-kernel family decode calls use: 1 = matrix cores, 0 = the
// plain VALU kernels (kept as the measured baseline).  Set by
// mkv_set_partial_kind from any thread; each call reads it once, when it
// starts (Geometry::partial_kind), and uses that value throughout.
static std::atomic<int> g_partial_kind{1};

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_layout(const mkv_layout* L, Geometry* g) {
  if (!L) return fail(MKV_ERR_NULL, "layout is NULL");
  if (L->page_size != kPage) return fail(MKV_ERR_SHAPE, "page_size %d unsupported (must be 16)", L->page_size);
  if (L->head_dim != 128 && L->head_dim != 256)
    return fail(MKV_ERR_SHAPE, "head_dim %d unsupported (128 or 256)", L->head_dim);
  if (L->num_kv_heads <= 0 || L->num_q_heads <= 0 || L->num_q_heads % L->num_kv_heads)
    return fail(MKV_ERR_SHAPE, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                L->num_q_heads, L->num_kv_heads);
  const int G = L->num_q_heads / L->num_kv_heads;
  if (G > kMaxGroup) return fail(MKV_ERR_SHAPE, "GQA group %d > %d unsupported", G, kMaxGroup);
  g->hq = L->num_q_heads;
  g->hkv = L->num_kv_heads;
  g->d = L->head_dim;
  g->G = G;
  return MKV_OK;
}

int check_pool(const mkv_pool* p, Geometry* g, bool need_fp8, bool need_tq3, bool need_tier) {
  if (!p) return fail(MKV_ERR_NULL, "pool is NULL");
  if (p->n_fp8 < 0 || p->n_tq3 < 0) return fail(MKV_ERR_RANGE, "negative pool size");
  if ((int64_t)p->n_fp8 + p->n_tq3 > 0x7fffffff) return fail(MKV_ERR_RANGE, "pool too large");
  if (need_fp8 && !p->fp8_slab && p->n_fp8 > 0) return fail(MKV_ERR_NULL, "fp8_slab is NULL");
  if (need_tq3 && !p->tq3_slab && p->n_tq3 > 0) return fail(MKV_ERR_NULL, "tq3_slab is NULL");
  if (need_tier && !p->tier) return fail(MKV_ERR_NULL, "tier is NULL");
  if (!aligned16(p->fp8_slab) || !aligned16(p->tq3_slab)) return fail(MKV_ERR_ALIGN, "slabs must be 16-byte aligned");
  if (!aligned16(p->tq3_signs)) return fail(MKV_ERR_ALIGN, "tq3_signs must be 16-byte aligned");
  if (!(p->k_scale > 0.0f) || !(p->v_scale > 0.0f) || std::isinf(p->k_scale) || std::isinf(p->v_scale))
    return fail(MKV_ERR_RANGE, "k_scale and v_scale must be finite and > 0");
  g->n_fp8 = p->n_fp8;
  g->n_tq3 = p->n_tq3;
  return MKV_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// MKV_DEBUG_SYNC=1 in the environment (read at every call): after a call
// has enqueued its work, synchronise the stream and check it, so a failing
// launch is reported by the call that made it (MKV_ERR_HIP) rather than by a
// later one; device-data status bits left in the call's workspace are
// printed to stderr (the call still returns MKV_OK for them, as without the
// flag: they are read with mkv_workspace_status).
bool debug_sync() {
  const char* v = std::getenv("MKV_DEBUG_SYNC");
  return v && v[0] == '1' && v[1] == '\0';
}

int debug_finish(int rc, void* stream, const void* ws, const char* what) {
  if (rc != MKV_OK || !debug_sync()) return rc;
  hipError_t e = hipStreamSynchronize(as_stream(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  if (ws) {
    int32_t status = 0;
    e = hipMemcpy(&status, ws, sizeof status, hipMemcpyDeviceToHost);   // status is the first field
    if (e != hipSuccess) return hip_fail(e, what);
    if (status) std::fprintf(stderr, "[mkv] %s: device status bits 0x%x\n", what, (unsigned)status);
  }
  return MKV_OK;
}

void set_layer(LayerTable* lt, int l, const mkv_pool& p) {
  lt->fp8[l] = p.fp8_slab;
  lt->tq3[l] = p.tq3_slab;
  lt->k_scale[l] = p.k_scale;
  lt->v_scale[l] = p.v_scale;
  lt->tq3_v_up[l] = (float)(1 << tq3_v_exponent(p.v_scale));
  lt->signs[l] = p.tq3_signs;
  lt->any_signs |= p.tq3_signs != nullptr;
}

}  // namespace

WsSizes workspace_sizes(int hq, int hkv, int d, int batch, int bt_capacity, int n_layers, int n_query) {
  WsSizes s{};
  const int G = hq / hkv;
  const int R = n_query * G;                         // query rows per KV head
  const int rowblk = R > kRowBlock ? 2 * kRowBlock : kRowBlock;   // 16-row blocks past 8 rows
  const int nblk = (R + rowblk - 1) / rowblk;
  const int Le = n_layers < kMaxLayers ? n_layers : kMaxLayers;
  const int per = Le * hkv * nblk;
  s.n_query = n_query;
  s.nblk = nblk;
  s.rowblk = rowblk;
  s.chunks_target = (kTargetItems + per - 1) / per;
  if (s.chunks_target < 1) s.chunks_target = 1;
  // chunks per format <= min(pages / kMinChunkPages, max(target, weighted
  // pages / kMaxChunkPages)) + batch (an FP8 page weighs 4/3 TQ3 pages)
  const int by_pages = (bt_capacity + kMinChunkPages - 1) / kMinChunkPages;
  const int by_max = max_size_chunks(bt_capacity);
  auto chunk_bound = [&](int target) {
    const int t = target > by_max ? target : by_max;
    return (t < by_pages ? t : by_pages) + batch;
  };
  // chunk tables: sized for the largest chunk count any layer count can plan
  s.table_cap = chunk_bound((kTargetItems + hkv - 1) / hkv);
  // partial states per layer of a plan made for this layer count.  The planner
  // takes pp >= weighted pages / max(1, target - 2 batch) per chunk (or pp =
  // kMaxChunkPages) and each request adds at most one part-filled chunk per
  // format, so NP < max(target, weighted pages / kMaxChunkPages) + 2 batch; and
  // never more than one chunk per kMinChunkPages pages plus one per request
  // and format.
  const int t = s.chunks_target > by_max ? s.chunks_target : by_max;
  s.np_cap = t + 2 * batch < 2 * (by_pages + batch) ? t + 2 * batch : 2 * (by_pages + batch);
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align_up(o + bytes, 256); return at; };
  s.off_status = take(sizeof(int32_t));
  s.off_totals = take(sizeof(int32_t) * T_FIELDS);
  s.off_req = take(sizeof(int32_t) * R_FIELDS * (size_t)(batch + 1));
  s.off_list_f = take(sizeof(int32_t) * (size_t)bt_capacity);
  s.off_list_t = take(sizeof(int32_t) * (size_t)bt_capacity);
  s.off_chunks_f = take(sizeof(int32_t) * kChunkInts * (size_t)s.table_cap);
  s.off_chunks_t = take(sizeof(int32_t) * kChunkInts * (size_t)s.table_cap);
  const size_t states = (size_t)Le * s.np_cap * hkv * R;
  s.off_q_rot = take(sizeof(float) * (size_t)Le * batch * n_query * hq * d);
  s.off_part_ml = take(sizeof(float) * 2 * states);
  s.off_part_acc = take(sizeof(float) * d * states);
  s.total = o;
  return s;
}

Plan plan_from_ws(void* ws, const WsSizes& s, int batch, int bt_capacity) {
  char* base = static_cast<char*>(ws);
  Plan p{};
  p.status = reinterpret_cast<int32_t*>(base + s.off_status);
  p.totals = reinterpret_cast<int32_t*>(base + s.off_totals);
  p.req = reinterpret_cast<int32_t*>(base + s.off_req);
  p.list_f = reinterpret_cast<int32_t*>(base + s.off_list_f);
  p.list_t = reinterpret_cast<int32_t*>(base + s.off_list_t);
  p.chunks_f = reinterpret_cast<int4*>(base + s.off_chunks_f);
  p.chunks_t = reinterpret_cast<int4*>(base + s.off_chunks_t);
  p.q_rot = reinterpret_cast<float*>(base + s.off_q_rot);
  p.part_ml = reinterpret_cast<float*>(base + s.off_part_ml);
  p.part_acc = reinterpret_cast<float*>(base + s.off_part_acc);
  p.batch = batch;
  p.bt_capacity = bt_capacity;
  p.table_cap = s.table_cap;
  p.np_cap = s.np_cap;
  p.chunks_target = s.chunks_target;
  p.n_query = s.n_query;
  p.nblk = s.nblk;
  p.rowblk = s.rowblk;
  return p;
}

}  // namespace mkv

using namespace mkv;

extern "C" {

size_t mkv_fp8_page_bytes(const mkv_layout* layout) {
  Geometry g{};
  if (check_layout(layout, &g) != MKV_OK) return 0;
  return (size_t)fp8_page_bytes(g.hkv, g.d);
}

size_t mkv_tq3_page_bytes(const mkv_layout* layout) {
  Geometry g{};
  if (check_layout(layout, &g) != MKV_OK) return 0;
  return (size_t)tq3_page_bytes(g.hkv, g.d);
}

static int mkv_append_impl(const mkv_layout* layout, const mkv_pool* pool, const float* k, const float* v,
               int32_t n_new, const int32_t* bt_offsets, const int32_t* bt_pages,
               const int32_t* pos, const int32_t* counts, int32_t batch, void* stream) {
  Geometry g{};
  int rc = check_layout(layout, &g);
  if (rc) return rc;
  if ((rc = check_pool(pool, &g, true, false, false))) return rc;
  if (batch < 0 || n_new < 0 || n_new > 65535) return fail(MKV_ERR_RANGE, "batch %d / n_new %d out of range", batch, n_new);
  if ((int64_t)batch * n_new > 0x7fffffff) return fail(MKV_ERR_RANGE, "batch * n_new too large");
  if (batch == 0 || n_new == 0) return MKV_OK;
  if (!k || !v || !bt_offsets || !bt_pages || !pos) return fail(MKV_ERR_NULL, "k, v, bt_offsets, bt_pages and pos are required");
  if (!aligned16(k) || !aligned16(v)) return fail(MKV_ERR_ALIGN, "k and v must be 16-byte aligned");
  hipError_t e = launch_append(g, pool->fp8_slab, pool->k_scale, pool->v_scale, k, v, n_new,
                               bt_offsets, bt_pages, pos, counts, batch, as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "append launch");
}

static int mkv_demote_pages_layers_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                            const int32_t* src_fp8, const int32_t* dst_tq3, int32_t n, void* stream) {
  Geometry g{};
  int rc = check_layout(layout, &g);
  if (rc) return rc;
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(MKV_ERR_RANGE, "n_layers %d not in [1, %d]", n_layers, kMaxLayers);
  LayerTable lt{};
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = check_pool(&pools[l], &g, true, true, false))) return rc;
    if (pools[l].n_fp8 != pools[0].n_fp8 || pools[l].n_tq3 != pools[0].n_tq3)
      return fail(MKV_ERR_RANGE, "layer %d: pools must share n_fp8 and n_tq3", l);
    set_layer(&lt, l, pools[l]);
  }
  if (n < 0) return fail(MKV_ERR_RANGE, "n = %d", n);
  if ((int64_t)n * g.hkv * n_layers > 0x7fffffff) return fail(MKV_ERR_RANGE, "n too large");
  if (n == 0) return MKV_OK;
  if (!src_fp8 || !dst_tq3) return fail(MKV_ERR_NULL, "src_fp8 and dst_tq3 are required");
  hipError_t e = launch_demote(g, lt, n_layers, src_fp8, dst_tq3, n, as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "demote launch");
}

int mkv_demote_pages(const mkv_layout* layout, const mkv_pool* pool, const int32_t* src_fp8,
                     const int32_t* dst_tq3, int32_t n, void* stream) {
  return mkv_demote_pages_layers(layout, pool, 1, src_fp8, dst_tq3, n, stream);
}

size_t mkv_decode_workspace_bytes(const mkv_layout* layout, int32_t batch, int32_t bt_capacity,
                                  int32_t n_layers) {
  Geometry g{};
  if (check_layout(layout, &g) != MKV_OK || batch < 0 || bt_capacity < 0 || n_layers < 1) return 0;
  return workspace_sizes(g.hq, g.hkv, g.d, batch, bt_capacity, n_layers).total;
}

namespace {

// Validation shared by every decode entry point.  `pools` may be NULL for
// mkv_merge (which reads only the workspace).
int prepare_decode(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, void* ws, size_t ws_bytes, Geometry* g, Plan* plan,
                   LayerTable* lt, int n_query = 1) {
  int rc = check_layout(layout, g);
  if (rc) return rc;
  g->partial_kind = g_partial_kind.load(std::memory_order_relaxed);
  if (!batch) return fail(MKV_ERR_NULL, "batch is NULL");
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(MKV_ERR_RANGE, "n_layers %d not in [1, %d]", n_layers, kMaxLayers);
  if (pools) {
    for (int l = 0; l < n_layers; ++l) {
      if ((rc = check_pool(&pools[l], g, true, true, true))) return rc;
      if (pools[l].n_fp8 != pools[0].n_fp8 || pools[l].n_tq3 != pools[0].n_tq3 || pools[l].tier != pools[0].tier)
        return fail(MKV_ERR_RANGE, "layer %d: pools must share n_fp8, n_tq3 and the tier map", l);
      if (pools[l].tq3_signs && !g->partial_kind)
        return fail(MKV_ERR_RANGE, "layer %d: rotated TQ3 pages need the matrix-core kernels", l);
      if (lt) set_layer(lt, l, pools[l]);
    }
  }
  const int B = batch->batch;
  if (B < 0 || batch->bt_capacity < 0) return fail(MKV_ERR_RANGE, "batch %d / bt_capacity %d", B, batch->bt_capacity);
  if (B > 0 && (!batch->bt_offsets || !batch->seq_lens || (!batch->bt_pages && batch->bt_capacity > 0)))
    return fail(MKV_ERR_NULL, "bt_offsets, bt_pages and seq_lens are required");
  if (B > 0 && !ws) return fail(MKV_ERR_NULL, "ws is required");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MKV_ERR_ALIGN, "ws must be 256-byte aligned");
  const WsSizes s = workspace_sizes(g->hq, g->hkv, g->d, B, batch->bt_capacity, n_layers, n_query);
  if (B > 0 && ws_bytes < s.total) return fail(MKV_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, s.total);
  *plan = plan_from_ws(ws, s, B, batch->bt_capacity);
  return MKV_OK;
}

int check_qo(const float* q, const float* out, const float* lse, float sm_scale, bool need_q, bool need_out) {
  if (need_q) {
    if (!(sm_scale > 0.0f) || std::isinf(sm_scale)) return fail(MKV_ERR_RANGE, "sm_scale must be finite and > 0");
    if (!q) return fail(MKV_ERR_NULL, "q is required");
    if (!aligned16(q)) return fail(MKV_ERR_ALIGN, "q must be 16-byte aligned");
  }
  if (need_out) {
    if (!out) return fail(MKV_ERR_NULL, "out is required");
    if (!aligned16(out) || (lse && !aligned16(lse))) return fail(MKV_ERR_ALIGN, "out and lse must be 16-byte aligned");
  }
  return MKV_OK;
}

// which: 0 FP8 items, 1 TQ3 items, 2 both (one launch for the matrix-core
// kernels, two for the VALU baseline).
int run_attend(int which, const Geometry& g, const LayerTable& lt, int n_layers, const Plan& plan,
               const float* q, float sm_scale, int batch, hipStream_t st) {
  const float qscale = sm_scale * 1.4426950408889634f;   // scores in log2 units
  const size_t q_ls = (size_t)batch * g.hq * g.d;
  hipError_t e;
  if (g.partial_kind) {
    e = launch_partial_mfma(which, g, lt, n_layers, q, q_ls, qscale, plan, AppendIn{nullptr, nullptr, 0}, st);
  } else {
    e = hipSuccess;
    if (which != 1) e = launch_partial_valu(false, g, lt, n_layers, q, q_ls, qscale, plan, st);
    if (e == hipSuccess && which != 0) e = launch_partial_valu(true, g, lt, n_layers, q, q_ls, qscale, plan, st);
  }
  return e == hipSuccess ? MKV_OK : hip_fail(e, "partial-attention launch");
}

int run_merge(const Geometry& g, int n_layers, const Plan& plan, float* out, float* lse, int batch,
              hipStream_t st, bool appended = false) {
  hipError_t e = launch_merge(g, n_layers, plan, out, lse, (size_t)batch * g.hq * g.d,
                              (size_t)batch * g.hq, st, appended);
  return e == hipSuccess ? MKV_OK : hip_fail(e, "merge launch");
}

}  // namespace

static int mkv_decode_plan_impl(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch,
                    int32_t n_layers, void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  int rc = prepare_decode(layout, pool, 1, batch, ws, ws_bytes, &g, &plan, nullptr);
  if (rc) return rc;
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(MKV_ERR_RANGE, "n_layers %d not in [1, %d]", n_layers, kMaxLayers);
  // size the plan (chunks per format) for n_layers layers per launch
  const WsSizes s = workspace_sizes(g.hq, g.hkv, g.d, batch->batch, batch->bt_capacity, n_layers);
  if (batch->batch > 0 && ws_bytes < s.total) return fail(MKV_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, s.total);
  if (batch->batch == 0) return MKV_OK;
  plan = plan_from_ws(ws, s, batch->batch, batch->bt_capacity);
  hipError_t e = launch_plan(g, pool->tier, batch->bt_offsets, batch->bt_pages, batch->seq_lens, plan, as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "plan launch");
}

static int attend_entry(int which, const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                        const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                        size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  LayerTable lt{};
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  int rc = prepare_decode(layout, pools, n_layers, batch, ws, ws_bytes, &g, &plan, &lt);
  if (rc) return rc;
  if ((rc = check_qo(q, nullptr, nullptr, sm_scale, true, false))) return rc;
  if (batch->batch == 0) return MKV_OK;
  return run_attend(which, g, lt, n_layers, plan, q, sm_scale, batch->batch, as_stream(stream));
}

static int mkv_attend_fp8_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                   size_t ws_bytes, void* stream) {
  return attend_entry(0, layout, pools, n_layers, batch, q, sm_scale, ws, ws_bytes, stream);
}

static int mkv_attend_tq3_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                   size_t ws_bytes, void* stream) {
  return attend_entry(1, layout, pools, n_layers, batch, q, sm_scale, ws, ws_bytes, stream);
}

static int mkv_attend_partials_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                        const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                        size_t ws_bytes, void* stream) {
  return attend_entry(2, layout, pools, n_layers, batch, q, sm_scale, ws, ws_bytes, stream);
}

static int mkv_merge_impl(const mkv_layout* layout, int32_t n_layers, const mkv_batch* batch, float* out,
              float* lse, void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  int rc = prepare_decode(layout, nullptr, n_layers, batch, ws, ws_bytes, &g, &plan, nullptr);
  if (rc) return rc;
  if ((rc = check_qo(nullptr, out, lse, 1.0f, false, true))) return rc;
  if (batch->batch == 0) return MKV_OK;
  return run_merge(g, n_layers, plan, out, lse, batch->batch, as_stream(stream));
}

namespace {

int run_fused(const Geometry& g, const LayerTable& lt, int n_layers, const Plan& plan, const float* q,
              float sm_scale, float* out, float* lse, int B, hipStream_t st) {
  const int rc = run_attend(2, g, lt, n_layers, plan, q, sm_scale, B, st);
  return rc ? rc : run_merge(g, n_layers, plan, out, lse, B, st);
}

}  // namespace

static int mkv_attend_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
               const mkv_batch* batch, const float* q, float sm_scale, float* out, float* lse,
               void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  LayerTable lt{};
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  int rc = prepare_decode(layout, pools, n_layers, batch, ws, ws_bytes, &g, &plan, &lt);
  if (rc) return rc;
  if ((rc = check_qo(q, out, lse, sm_scale, true, true))) return rc;
  if (batch->batch == 0) return MKV_OK;
  return run_fused(g, lt, n_layers, plan, q, sm_scale, out, lse, batch->batch, as_stream(stream));
}

static int mkv_append_attend_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                      const mkv_batch* batch, const float* k_new, const float* v_new,
                      const float* q, float sm_scale, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  LayerTable lt{};
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  int rc = prepare_decode(layout, pools, n_layers, batch, ws, ws_bytes, &g, &plan, &lt);
  if (rc) return rc;
  if ((rc = check_qo(q, out, lse, sm_scale, true, true))) return rc;
  if (!k_new || !v_new) return fail(MKV_ERR_NULL, "k_new and v_new are required");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(MKV_ERR_ALIGN, "k_new and v_new must be 16-byte aligned");
  if (!g.partial_kind) return fail(MKV_ERR_RANGE, "mkv_append_attend needs the matrix-core partial kernels");
  if (batch->batch == 0) return MKV_OK;
  const int B = batch->batch;
  hipStream_t st = as_stream(stream);
  const float qscale = sm_scale * 1.4426950408889634f;   // scores in log2 units
  const size_t q_ls = (size_t)B * g.hq * g.d;
  const AppendIn ap{k_new, v_new, (size_t)B * g.hkv * g.d};
  hipError_t e = launch_partial_mfma(2, g, lt, n_layers, q, q_ls, qscale, plan, ap, st);
  if (e != hipSuccess) return hip_fail(e, "partial-attention launch");
  return run_merge(g, n_layers, plan, out, lse, B, st, true);
}

static int mkv_decode_attn_layers_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                           const mkv_batch* batch, const float* q, float sm_scale, float* out,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  LayerTable lt{};
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  int rc = prepare_decode(layout, pools, n_layers, batch, ws, ws_bytes, &g, &plan, &lt);
  if (rc) return rc;
  if ((rc = check_qo(q, out, lse, sm_scale, true, true))) return rc;
  const int B = batch->batch;
  if (B == 0) return MKV_OK;
  hipStream_t st = as_stream(stream);
  hipError_t e = launch_plan(g, pools[0].tier, batch->bt_offsets, batch->bt_pages, batch->seq_lens, plan, st);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  return run_fused(g, lt, n_layers, plan, q, sm_scale, out, lse, B, st);
}

size_t mkv_decode_workspace_bytes_multi(const mkv_layout* layout, int32_t batch, int32_t bt_capacity,
                                        int32_t n_layers, int32_t n_query) {
  Geometry g{};
  if (check_layout(layout, &g) != MKV_OK || batch < 0 || bt_capacity < 0 || n_layers < 1 || n_query < 1 ||
      n_query > kMaxQuery)
    return 0;
  return workspace_sizes(g.hq, g.hkv, g.d, batch, bt_capacity, n_layers, n_query).total;
}

static int mkv_decode_attn_multi_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                          const mkv_batch* batch, int32_t n_query, const float* q, float sm_scale,
                          float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  Plan plan{};
  LayerTable lt{};
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  if (n_query < 1 || n_query > kMaxQuery) return fail(MKV_ERR_RANGE, "n_query %d not in [1, %d]", n_query, kMaxQuery);
  int rc = prepare_decode(layout, pools, n_layers, batch, ws, ws_bytes, &g, &plan, &lt, n_query);
  if (rc) return rc;
  if ((rc = check_qo(q, out, lse, sm_scale, true, true))) return rc;
  if (n_query > 1 && !g.partial_kind) return fail(MKV_ERR_RANGE, "multi-query decode needs the matrix-core kernels");
  const int B = batch->batch;
  if (B == 0) return MKV_OK;
  hipStream_t st = as_stream(stream);
  hipError_t e = launch_plan(g, pools[0].tier, batch->bt_offsets, batch->bt_pages, batch->seq_lens, plan, st);
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  if (n_query == 1) return run_fused(g, lt, n_layers, plan, q, sm_scale, out, lse, B, st);
  const float qscale = sm_scale * 1.4426950408889634f;   // scores in log2 units
  const size_t rows = (size_t)B * n_query * g.hq;
  e = launch_partial_mfma(2, g, lt, n_layers, q, rows * g.d, qscale, plan, AppendIn{nullptr, nullptr, 0}, st);
  if (e != hipSuccess) return hip_fail(e, "partial-attention launch");
  e = launch_merge(g, n_layers, plan, out, lse, rows * g.d, rows, st);
  return e == hipSuccess ? MKV_OK : hip_fail(e, "merge launch");
}

int mkv_decode_attn(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch,
                    const float* q, float sm_scale, float* out, float* lse, void* ws,
                    size_t ws_bytes, void* stream) {
  return mkv_decode_attn_layers(layout, pool, 1, batch, q, sm_scale, out, lse, ws, ws_bytes, stream);
}

}  // extern "C"

// ---- decode for callers that cannot allocate -----------------------------
// mkv_decode_attn_noalloc runs mkv_decode_attn with its workspace in `scratch`,
// a file-scope device array: each GPU the library runs on holds one copy of
// kNoAllocScratchBytes for the life of the process.  In host code `scratch`
// names a host-side stand-in, not the device copy, so its device address is
// looked up once per device (hipGetSymbolAddress, with that device current)
// and only that address is ever handed to kernels.
namespace mkv {
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];        // device address of `scratch`, per device

int scratch_on_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MKV_ERR_RANGE, "device %d outside [0, %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MKV_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MKV_OK;
}
}  // namespace
}  // namespace mkv

extern "C" {

int mkv_decode_attn_noalloc(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch,
                            const float* q, float sm_scale, float* out, float* lse, void* stream) {
  Geometry g{};
  int rc = check_layout(layout, &g);
  if (rc) return rc;
  if (!batch) return fail(MKV_ERR_NULL, "batch is NULL");
  if (batch->batch < 0 || batch->bt_capacity < 0)
    return fail(MKV_ERR_RANGE, "batch %d / bt_capacity %d", batch->batch, batch->bt_capacity);
  const size_t need = workspace_sizes(g.hq, g.hkv, g.d, batch->batch, batch->bt_capacity, 1).total;
  if (need > kNoAllocScratchBytes)
    return fail(MKV_ERR_WORKSPACE, "this batch needs %zu bytes of workspace, more than the %zu-byte static scratch of "
                "mkv_decode_attn_noalloc (use mkv_decode_attn with a caller workspace)", need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_on_current_device(&ws))) return rc;
  return mkv_decode_attn(layout, pool, batch, q, sm_scale, out, lse, ws, kNoAllocScratchBytes, stream);
}

static int mkv_debug_gather_impl(const mkv_layout* layout, const mkv_pool* pool, const int32_t* bt_offsets,
                     const int32_t* bt_pages, int32_t b, int32_t n_pages, uint8_t* out, void* stream) {
  Geometry g{};
  int rc = check_layout(layout, &g);
  if (rc) return rc;
  if ((rc = check_pool(pool, &g, true, true, false))) return rc;
  if (b < 0 || n_pages < 0) return fail(MKV_ERR_RANGE, "b %d / n_pages %d", b, n_pages);
  if (n_pages == 0) return MKV_OK;
  if (!bt_offsets || !bt_pages || !out) return fail(MKV_ERR_NULL, "bt_offsets, bt_pages and out are required");
  if (!aligned16(out)) return fail(MKV_ERR_ALIGN, "out must be 16-byte aligned");
  hipError_t e = launch_gather(g, pool->fp8_slab, pool->tq3_slab, bt_offsets, bt_pages, b, n_pages,
                               out, as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "gather launch");
}

static int mkv_stream_read_impl(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  if (!src || !sink) return fail(MKV_ERR_NULL, "src and sink are required");
  if (!aligned16(src)) return fail(MKV_ERR_ALIGN, "src must be 16-byte aligned");
  if (sink_words < (size_t)kItemWaves) return fail(MKV_ERR_RANGE, "sink_words %zu < %d", sink_words, kItemWaves);
  if (bytes / stream_read_unit() > 0x7fffffffu) return fail(MKV_ERR_RANGE, "bytes too large");
  hipError_t e = launch_stream_read(src, bytes, sink, sink_words, as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "stream-read launch");
}

static int mkv_debug_item_trace_impl(uint64_t* host, size_t words) {
  if (!host) return fail(MKV_ERR_NULL, "host is required");
  const int rc = read_item_trace(host, words);
  if (rc == -1) return fail(MKV_ERR_RANGE, "this library is not an item-trace build (MKV_ITEM_TRACE=1)");
  if (rc != 0) return fail(MKV_ERR_HIP, "item-trace copy failed");
  return MKV_OK;
}

static int mkv_materialize_impl(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch, int32_t b,
                    int32_t page_lo, int32_t n_pages, uint16_t* k_out, uint16_t* v_out, void* stream) {
  Geometry g{};
  int rc = check_layout(layout, &g);
  if (rc) return rc;
  if ((rc = check_pool(pool, &g, true, true, false))) return rc;
  if (!batch) return fail(MKV_ERR_NULL, "batch is NULL");
  if (b < 0 || b >= batch->batch || page_lo < 0 || n_pages < 0)
    return fail(MKV_ERR_RANGE, "b %d (batch %d) / page_lo %d / n_pages %d", b, batch->batch, page_lo, n_pages);
  if ((int64_t)page_lo + n_pages > 0x7fffffff / kPage) return fail(MKV_ERR_RANGE, "page range too large");
  if (n_pages == 0) return MKV_OK;
  if (!batch->bt_offsets || !batch->bt_pages || !k_out || !v_out)
    return fail(MKV_ERR_NULL, "bt_offsets, bt_pages, k_out and v_out are required");
  if (!aligned16(k_out) || !aligned16(v_out)) return fail(MKV_ERR_ALIGN, "k_out and v_out must be 16-byte aligned");
  hipError_t e = launch_materialize(g, pool->fp8_slab, pool->tq3_slab, pool->k_scale, pool->v_scale,
                                    batch->bt_offsets, batch->bt_pages, batch->bt_capacity, b, page_lo,
                                    n_pages, k_out, v_out, pool->tq3_signs, as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "materialize launch");
}

size_t mkv_lifecycle_workspace_bytes(int32_t batch) {
  if (batch < 0) return 0;
  return align_up(sizeof(int32_t) * (4 + 3 * (size_t)batch), 256);
}

namespace {

// Checks shared by the lifecycle calls: layout, pools (equal sizes, the tier
// map given), the batch tables and the free stacks.
int check_lifecycle(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers, const int32_t* bt_offsets,
                    const void* bt_pages, int32_t* seq_lens, int32_t batch, int32_t bt_capacity, uint8_t* tier,
                    int32_t* fp8_free, int32_t* tq3_free, int32_t* free_tops, void* ws, size_t ws_bytes,
                    size_t ws_need, Geometry* g, LayerTable* lt) {
  int rc = check_layout(layout, g);
  if (rc) return rc;
  if (!pools) return fail(MKV_ERR_NULL, "pools is NULL");
  if (n_layers < 1 || n_layers > kMaxLayers) return fail(MKV_ERR_RANGE, "n_layers %d not in [1, %d]", n_layers, kMaxLayers);
  for (int l = 0; l < n_layers; ++l) {
    if ((rc = check_pool(&pools[l], g, true, true, true))) return rc;
    if (pools[l].n_fp8 != pools[0].n_fp8 || pools[l].n_tq3 != pools[0].n_tq3 || pools[l].tier != tier)
      return fail(MKV_ERR_RANGE, "layer %d: pools must share n_fp8, n_tq3 and the tier map passed in", l);
    if (lt) set_layer(lt, l, pools[l]);
  }
  if (batch < 0 || bt_capacity < 0) return fail(MKV_ERR_RANGE, "batch %d / bt_capacity %d", batch, bt_capacity);
  if (batch == 0) return MKV_OK;                      // no request: nothing to do
  if (!bt_offsets || !bt_pages || !seq_lens || !tier || !fp8_free || !tq3_free || !free_tops || !ws)
    return fail(MKV_ERR_NULL, "tables, tier map, free stacks, free_tops and ws are required");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MKV_ERR_ALIGN, "ws must be 256-byte aligned");
  if (ws_bytes < ws_need) return fail(MKV_ERR_WORKSPACE, "workspace %zu bytes < %zu required", ws_bytes, ws_need);
  return MKV_OK;
}

}  // namespace

static int mkv_lifecycle_step_impl(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                       const int32_t* bt_offsets, int32_t* bt_pages, int32_t* seq_lens, int32_t batch,
                       int32_t bt_capacity, uint8_t* tier, int32_t* fp8_free, int32_t* tq3_free,
                       int32_t* free_tops, int32_t recent_pages, void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  LayerTable lt{};
  int rc = check_lifecycle(layout, pools, n_layers, bt_offsets, bt_pages, seq_lens, batch, bt_capacity, tier,
                           fp8_free, tq3_free, free_tops, ws, ws_bytes, mkv_lifecycle_workspace_bytes(batch), &g, &lt);
  if (rc || batch == 0) return rc;
  if (recent_pages < 1) return fail(MKV_ERR_RANGE, "recent_pages %d must be >= 1", recent_pages);
  if ((int64_t)n_layers * batch * g.hkv > 0x7fffffff) return fail(MKV_ERR_RANGE, "batch too large");
  hipError_t e = launch_lifecycle_step(g, lt, n_layers, bt_offsets, bt_pages, seq_lens, batch, bt_capacity, tier,
                                       fp8_free, tq3_free, free_tops, recent_pages, static_cast<int32_t*>(ws),
                                       as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "lifecycle launch");
}

static int mkv_lifecycle_release_impl(const mkv_layout* layout, const mkv_pool* pool, const int32_t* bt_offsets,
                          const int32_t* bt_pages, int32_t* seq_lens, int32_t batch, int32_t bt_capacity,
                          uint8_t* tier, int32_t* fp8_free, int32_t* tq3_free, int32_t* free_tops,
                          const int32_t* requests, int32_t n_req, void* ws, size_t ws_bytes, void* stream) {
  Geometry g{};
  int rc = check_lifecycle(layout, pool, 1, bt_offsets, bt_pages, seq_lens, batch, bt_capacity, tier, fp8_free,
                           tq3_free, free_tops, ws, ws_bytes, mkv_lifecycle_workspace_bytes(0), &g, nullptr);
  if (rc || batch == 0) return rc;
  if (n_req < 0) return fail(MKV_ERR_RANGE, "n_req %d", n_req);
  if (n_req > 0 && !requests) return fail(MKV_ERR_NULL, "requests is required");
  hipError_t e = launch_lifecycle_release(g, bt_offsets, bt_pages, seq_lens, batch, bt_capacity, tier, fp8_free,
                                          tq3_free, free_tops, requests, n_req, static_cast<int32_t*>(ws),
                                          as_stream(stream));
  return e == hipSuccess ? MKV_OK : hip_fail(e, "lifecycle release launch");
}

int mkv_workspace_status(const void* ws, void* stream) {
  if (!ws) return fail(MKV_ERR_NULL, "ws is NULL");
  hipError_t e = hipStreamSynchronize(as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "stream synchronize");
  int32_t status = 0;
  e = hipMemcpy(&status, ws, sizeof status, hipMemcpyDeviceToHost);   // status is the first field
  if (e != hipSuccess) return hip_fail(e, "status copy");
  return status;
}

const char* mkv_status_string(int status) {
  switch (status) {
    case MKV_OK: return "ok";
    case MKV_ERR_NULL: return "null pointer";
    case MKV_ERR_SHAPE: return "unsupported shape";
    case MKV_ERR_ALIGN: return "misaligned pointer";
    case MKV_ERR_WORKSPACE: return "workspace too small";
    case MKV_ERR_RANGE: return "value out of range";
    case MKV_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* mkv_last_error(void) { return g_err; }

int mkv_set_partial_kind(int32_t kind) {
  if (kind != 0 && kind != 1) return fail(MKV_ERR_RANGE, "kind %d", kind);
  g_partial_kind.store(kind, std::memory_order_relaxed);
  return MKV_OK;
}


// MKV_DEBUG_SYNC=1: every call that enqueues work synchronises its stream and
// checks it before returning (debug_finish).
int mkv_append(const mkv_layout* layout, const mkv_pool* pool, const float* k, const float* v,
               int32_t n_new, const int32_t* bt_offsets, const int32_t* bt_pages,
               const int32_t* pos, const int32_t* counts, int32_t batch, void* stream) {
  return debug_finish(mkv_append_impl(layout, pool, k, v, n_new, bt_offsets, bt_pages, pos, counts, batch, stream), stream, nullptr, "mkv_append");
}

int mkv_demote_pages_layers(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                            const int32_t* src_fp8, const int32_t* dst_tq3, int32_t n, void* stream) {
  return debug_finish(mkv_demote_pages_layers_impl(layout, pools, n_layers, src_fp8, dst_tq3, n, stream), stream, nullptr, "mkv_demote_pages_layers");
}

int mkv_decode_plan(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch,
                    int32_t n_layers, void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_decode_plan_impl(layout, pool, batch, n_layers, ws, ws_bytes, stream), stream, ws, "mkv_decode_plan");
}

int mkv_attend_fp8(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                   size_t ws_bytes, void* stream) {
  return debug_finish(mkv_attend_fp8_impl(layout, pools, n_layers, batch, q, sm_scale, ws, ws_bytes, stream), stream, ws, "mkv_attend_fp8");
}

int mkv_attend_tq3(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                   const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                   size_t ws_bytes, void* stream) {
  return debug_finish(mkv_attend_tq3_impl(layout, pools, n_layers, batch, q, sm_scale, ws, ws_bytes, stream), stream, ws, "mkv_attend_tq3");
}

int mkv_attend_partials(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                        const mkv_batch* batch, const float* q, float sm_scale, void* ws,
                        size_t ws_bytes, void* stream) {
  return debug_finish(mkv_attend_partials_impl(layout, pools, n_layers, batch, q, sm_scale, ws, ws_bytes, stream), stream, ws, "mkv_attend_partials");
}

int mkv_merge(const mkv_layout* layout, int32_t n_layers, const mkv_batch* batch, float* out,
              float* lse, void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_merge_impl(layout, n_layers, batch, out, lse, ws, ws_bytes, stream), stream, ws, "mkv_merge");
}

int mkv_attend(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
               const mkv_batch* batch, const float* q, float sm_scale, float* out, float* lse,
               void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_attend_impl(layout, pools, n_layers, batch, q, sm_scale, out, lse, ws, ws_bytes, stream), stream, ws, "mkv_attend");
}

int mkv_append_attend(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                      const mkv_batch* batch, const float* k_new, const float* v_new,
                      const float* q, float sm_scale, float* out, float* lse,
                      void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_append_attend_impl(layout, pools, n_layers, batch, k_new, v_new, q, sm_scale, out, lse, ws, ws_bytes, stream), stream, ws, "mkv_append_attend");
}

int mkv_decode_attn_layers(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                           const mkv_batch* batch, const float* q, float sm_scale, float* out,
                           float* lse, void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_decode_attn_layers_impl(layout, pools, n_layers, batch, q, sm_scale, out, lse, ws, ws_bytes, stream), stream, ws, "mkv_decode_attn_layers");
}

int mkv_decode_attn_multi(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                          const mkv_batch* batch, int32_t n_query, const float* q, float sm_scale,
                          float* out, float* lse, void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_decode_attn_multi_impl(layout, pools, n_layers, batch, n_query, q, sm_scale, out, lse, ws, ws_bytes, stream), stream, ws, "mkv_decode_attn_multi");
}

int mkv_debug_gather(const mkv_layout* layout, const mkv_pool* pool, const int32_t* bt_offsets,
                     const int32_t* bt_pages, int32_t b, int32_t n_pages, uint8_t* out, void* stream) {
  return debug_finish(mkv_debug_gather_impl(layout, pool, bt_offsets, bt_pages, b, n_pages, out, stream), stream, nullptr, "mkv_debug_gather");
}

int mkv_stream_read(const void* src, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
  return debug_finish(mkv_stream_read_impl(src, bytes, sink, sink_words, stream), stream, nullptr, "mkv_stream_read");
}

int mkv_debug_item_trace(uint64_t* host, size_t words) {
  return debug_finish(mkv_debug_item_trace_impl(host, words), nullptr, nullptr, "mkv_debug_item_trace");
}

int mkv_materialize(const mkv_layout* layout, const mkv_pool* pool, const mkv_batch* batch, int32_t b,
                    int32_t page_lo, int32_t n_pages, uint16_t* k_out, uint16_t* v_out, void* stream) {
  return debug_finish(mkv_materialize_impl(layout, pool, batch, b, page_lo, n_pages, k_out, v_out, stream), stream, nullptr, "mkv_materialize");
}

int mkv_lifecycle_step(const mkv_layout* layout, const mkv_pool* pools, int32_t n_layers,
                       const int32_t* bt_offsets, int32_t* bt_pages, int32_t* seq_lens, int32_t batch,
                       int32_t bt_capacity, uint8_t* tier, int32_t* fp8_free, int32_t* tq3_free,
                       int32_t* free_tops, int32_t recent_pages, void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_lifecycle_step_impl(layout, pools, n_layers, bt_offsets, bt_pages, seq_lens, batch, bt_capacity, tier, fp8_free, tq3_free, free_tops, recent_pages, ws, ws_bytes, stream), stream, ws, "mkv_lifecycle_step");
}

int mkv_lifecycle_release(const mkv_layout* layout, const mkv_pool* pool, const int32_t* bt_offsets,
                          const int32_t* bt_pages, int32_t* seq_lens, int32_t batch, int32_t bt_capacity,
                          uint8_t* tier, int32_t* fp8_free, int32_t* tq3_free, int32_t* free_tops,
                          const int32_t* requests, int32_t n_req, void* ws, size_t ws_bytes, void* stream) {
  return debug_finish(mkv_lifecycle_release_impl(layout, pool, bt_offsets, bt_pages, seq_lens, batch, bt_capacity, tier, fp8_free, tq3_free, free_tops, requests, n_req, ws, ws_bytes, stream), stream, ws, "mkv_lifecycle_release");
}

}  // extern "C"
