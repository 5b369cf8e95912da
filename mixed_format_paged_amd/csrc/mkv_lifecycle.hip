// mkv_lifecycle.hip -- the per-step page lifecycle on the device.
//
// Minima-KV keeps Recent and protected Anchor pages in FP8 and moves older
// non-anchor pages to packed TQ3 while every live-request page stays
// addressable (arXiv 2608.23834, page 1, Abstract).  The pages describe no
// allocator; the readings implemented here (the caller owns the policy of
// which pages are Anchors, by writing tier A):
//
//  * Free FP8 and TQ3 ids are kept in two stacks (fp8_free[0 .. top_f),
//    tq3_free[0 .. top_t)); a pop takes the top entry.
//  * One decode step adds one token per request.  A request whose seq_len is
//    a multiple of 16 needs a new logical page: it pops an FP8 id, which
//    becomes Recent.  When the number of pages n grows past the Recent window
//    of R pages, page n - R - 1 leaves the window: if its tier is Recent it
//    pops a TQ3 id and is demoted in every layer (an Anchor stays FP8; any
//    other tier is left alone).
//  * Pops are made in request order (request b's pops follow those of the
//    requests before it), the freed FP8 ids are pushed in the same order
//    after the pops, so the whole step is deterministic.
//  * The step is all or nothing: a request whose block-table row is full, an
//    id outside the pool, a tier that contradicts an id, too few free ids or
//    stack tops outside their arrays set MKV_DEV_* bits in the workspace
//    status and change nothing.
//
// Launches: lifecycle_plan (one workgroup: checks, prefix sums, pops, block
// table and seq_len updates, the list of pages to demote), then the demote
// kernel over that list, which also rewrites each demoted page's block-table
// entry, tier bytes and free-stack slot.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

constexpr int kPlanThreads = 1024;

// Exclusive scan of a pair of counts packed in 64 bits over the workgroup.
__device__ uint64_t scan_pairs(uint64_t v, uint64_t* total, uint64_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint64_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint64_t w = lane < kPlanThreads / 64 ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < kPlanThreads / 64; o <<= 1) {
      const uint64_t y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < kPlanThreads / 64) sh[64 + lane] = w;
  }
  __syncthreads();
  const uint64_t before = wave ? sh[64 + wave - 1] : 0;
  *total = sh[64 + kPlanThreads / 64 - 1];
  __syncthreads();
  return before + x - v;
}

__device__ inline uint64_t pair(int a, int b) { return (uint64_t)(uint32_t)a | ((uint64_t)(uint32_t)b << 32); }

// One request's needs this step.
struct Need {
  int new_page;    // 1: logical page n (its first token) is allocated
  int demote;      // 1: logical page `aged` leaves the window as a Recent page
  int aged;        // logical index of the page leaving the window
  int aged_id;
  int err;
};

__device__ Need request_need(int b, const int32_t* bt_offsets, const int32_t* bt_pages, const int32_t* seq_lens,
                             int bt_capacity, const uint8_t* tier, int n_fp8, int n_tq3, int recent) {
  Need r{0, 0, -1, -1, 0};
  const int off0 = bt_offsets[b], off1 = bt_offsets[b + 1];
  const int sl = seq_lens[b];
  if (sl < 0 || off0 < 0 || off1 < off0 || off1 > bt_capacity) { r.err = kDevBadSeqLen; return r; }
  const int n = (sl + kPage - 1) / kPage;              // pages before the step
  if (n > off1 - off0) { r.err = kDevBadSeqLen; return r; }
  if (sl % kPage != 0) return r;                        // the token fits the last page
  r.new_page = 1;
  if (n + 1 > off1 - off0) { r.err = kDevBadSeqLen; return r; }   // the row is full
  r.aged = n - recent;                                  // pages are n + 1 after the step
  if (r.aged < 0) return r;
  r.aged_id = bt_pages[off0 + r.aged];
  if (r.aged_id < 0 || r.aged_id >= n_fp8 + n_tq3) { r.err = kDevBadPageId; return r; }
  const int t = tier[r.aged_id];
  if (t == kTierRecent) {
    if (r.aged_id >= n_fp8) { r.err = kDevBadTier; return r; }
    r.demote = 1;
  }
  return r;
}

}  // namespace

// ws layout (int32): [0] status, [1] pages to demote, [2] first free-stack slot
// of the pushes, [3] unused, then src[batch], dst[batch], entry[batch].
__global__ void __launch_bounds__(kPlanThreads) lifecycle_plan(
    const int32_t* __restrict__ bt_offsets, int32_t* __restrict__ bt_pages, int32_t* __restrict__ seq_lens,
    int batch, int bt_capacity, uint8_t* __restrict__ tier, int n_fp8, int n_tq3,
    const int32_t* __restrict__ fp8_free, const int32_t* __restrict__ tq3_free, int32_t* __restrict__ tops,
    int recent, int32_t* __restrict__ ws) {
  __shared__ uint64_t sh[128];
  const int tid = threadIdx.x;
  const int top_f = tops[0], top_t = tops[1];
  const bool stacks_ok = top_f >= 0 && top_f <= n_fp8 && top_t >= 0 && top_t <= n_tq3;
  int32_t* src = ws + 4;
  int32_t* dst = src + batch;
  int32_t* entry = dst + batch;
  // pass 1: needs, errors and the ids the pops would take
  int err = 0;
  int carry_f = 0, carry_t = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + tid;
    Need r{0, 0, -1, -1, 0};
    if (b < batch) r = request_need(b, bt_offsets, bt_pages, seq_lens, bt_capacity, tier, n_fp8, n_tq3, recent);
    uint64_t tot;
    const uint64_t ex = scan_pairs(pair(r.new_page, r.demote), &tot, sh);
    const int pf = carry_f + (int)(uint32_t)ex, pt = carry_t + (int)(ex >> 32);
    err |= r.err;
    if (r.new_page && stacks_ok && pf < top_f) {
      const int id = fp8_free[top_f - 1 - pf];
      if (id < 0 || id >= n_fp8) err |= kDevBadPageId;
      else if (tier[id] != kTierFree) err |= kDevBadTier;
    }
    if (r.demote && stacks_ok && pt < top_t) {
      const int id = tq3_free[top_t - 1 - pt];
      if (id < n_fp8 || id >= n_fp8 + n_tq3) err |= kDevBadPageId;
      else if (tier[id] != kTierFree) err |= kDevBadTier;
    }
    carry_f += (int)(uint32_t)tot;
    carry_t += (int)(tot >> 32);
  }
  // enough free ids, and room for the pushes of the demoted FP8 ids
  if (!stacks_ok || carry_f > top_f || carry_t > top_t || top_f - carry_f + carry_t > n_fp8) err |= kDevNoFreePage;
  err = (__syncthreads_or(err & kDevBadPageId) ? kDevBadPageId : 0) |
        (__syncthreads_or(err & kDevBadTier) ? kDevBadTier : 0) |
        (__syncthreads_or(err & kDevBadSeqLen) ? kDevBadSeqLen : 0) |
        (__syncthreads_or(err & kDevNoFreePage) ? kDevNoFreePage : 0);
  if (err) {
    if (tid == 0) { ws[0] = err; ws[1] = 0; ws[2] = 0; }
    return;
  }
  // pass 2: pops in request order, new pages, seq_lens, the demotion list
  const int total_f = carry_f, total_t = carry_t;
  carry_f = 0;
  carry_t = 0;
  for (int base = 0; base < batch; base += kPlanThreads) {
    const int b = base + tid;
    Need r{0, 0, -1, -1, 0};
    if (b < batch) r = request_need(b, bt_offsets, bt_pages, seq_lens, bt_capacity, tier, n_fp8, n_tq3, recent);
    uint64_t tot;
    const uint64_t ex = scan_pairs(pair(r.new_page, r.demote), &tot, sh);
    const int pf = carry_f + (int)(uint32_t)ex, pt = carry_t + (int)(ex >> 32);
    if (b < batch) {
      const int off0 = bt_offsets[b], sl = seq_lens[b];
      if (r.new_page) {
        const int id = fp8_free[top_f - 1 - pf];
        bt_pages[off0 + sl / kPage] = id;
        tier[id] = kTierRecent;
      }
      if (r.demote) {
        src[pt] = r.aged_id;
        dst[pt] = tq3_free[top_t - 1 - pt];
        entry[pt] = off0 + r.aged;
      }
      seq_lens[b] = sl + 1;
    }
    carry_f += (int)(uint32_t)tot;
    carry_t += (int)(tot >> 32);
    __syncthreads();      // this block's reads of the tables are done before the next block writes
  }
  if (tid == 0) {
    ws[0] = 0;
    ws[1] = total_t;
    ws[2] = top_f - total_f;                 // the demoted FP8 ids are pushed from here
    tops[0] = top_f - total_f + total_t;
    tops[1] = top_t - total_t;
  }
}

// Release: every live page of the listed requests goes back to its free
// stack (FP8 and TQ3 ids pushed in list order, then logical order), its tier
// byte becomes free and the request's seq_len 0.  The block-table entries
// keep their stale ids; only seq_len decides which entries are live.
__global__ void __launch_bounds__(kPlanThreads) lifecycle_release(
    const int32_t* __restrict__ bt_offsets, const int32_t* __restrict__ bt_pages, int32_t* __restrict__ seq_lens,
    int batch, int bt_capacity, uint8_t* __restrict__ tier, int n_fp8, int n_tq3, int32_t* __restrict__ fp8_free,
    int32_t* __restrict__ tq3_free, int32_t* __restrict__ tops, const int32_t* __restrict__ requests, int n_req,
    int32_t* __restrict__ ws) {
  __shared__ uint64_t sh[128];
  const int tid = threadIdx.x;
  int top_f = tops[0], top_t = tops[1];
  int err = 0;
  // checks first: every listed request is valid, its pages are live ids, and
  // the stacks have room for them
  int sf = 0, st = 0;
  for (int i = tid; i < n_req; i += kPlanThreads) {
    const int b = requests[i];
    if (b < 0 || b >= batch) { err |= kDevBadSeqLen; continue; }
    const int off0 = bt_offsets[b], off1 = bt_offsets[b + 1], sl = seq_lens[b];
    const int n = (sl + kPage - 1) / kPage;
    if (sl < 0 || off0 < 0 || off1 < off0 || off1 > bt_capacity || n > off1 - off0) { err |= kDevBadSeqLen; continue; }
    for (int lp = 0; lp < n; ++lp) {
      const int id = bt_pages[off0 + lp];
      if (id < 0 || id >= n_fp8 + n_tq3) err |= kDevBadPageId;
      else if (tier[id] == kTierFree) err |= kDevBadTier;
      else if (id < n_fp8) ++sf;
      else ++st;
    }
  }
  uint64_t need;
  scan_pairs(pair(sf, st), &need, sh);
  if (top_f < 0 || top_t < 0 || top_f + (int)(uint32_t)need > n_fp8 || top_t + (int)(need >> 32) > n_tq3)
    err |= kDevNoFreePage;
  err = (__syncthreads_or(err & kDevBadPageId) ? kDevBadPageId : 0) |
        (__syncthreads_or(err & kDevBadTier) ? kDevBadTier : 0) |
        (__syncthreads_or(err & kDevBadSeqLen) ? kDevBadSeqLen : 0) |
        (__syncthreads_or(err & kDevNoFreePage) ? kDevNoFreePage : 0);
  if (err) {
    if (tid == 0) ws[0] = err;
    return;
  }
  // one listed request per thread per block of the list; its pages in logical order
  for (int base = 0; base < n_req; base += kPlanThreads) {
    const int i = base + tid;
    int nf = 0, nt = 0, b = -1, n = 0, off0 = 0;
    if (i < n_req) {
      b = requests[i];
      off0 = bt_offsets[b];
      n = (seq_lens[b] + kPage - 1) / kPage;
      for (int lp = 0; lp < n; ++lp) (bt_pages[off0 + lp] < n_fp8 ? nf : nt)++;
    }
    uint64_t tot;
    const uint64_t ex = scan_pairs(pair(nf, nt), &tot, sh);
    int pf = top_f + (int)(uint32_t)ex, pt = top_t + (int)(ex >> 32);
    for (int lp = 0; lp < n; ++lp) {
      const int id = bt_pages[off0 + lp];
      if (id < n_fp8) fp8_free[pf++] = id; else tq3_free[pt++] = id;
      tier[id] = kTierFree;
    }
    if (i < n_req) seq_lens[b] = 0;
    top_f += (int)(uint32_t)tot;
    top_t += (int)(tot >> 32);
  }
  if (tid == 0) {
    ws[0] = 0;
    tops[0] = top_f;
    tops[1] = top_t;
  }
}

hipError_t launch_lifecycle_step(const Geometry& g, const LayerTable& lt, int n_layers, const int32_t* bt_offsets,
                                 int32_t* bt_pages, int32_t* seq_lens, int batch, int bt_capacity, uint8_t* tier,
                                 int32_t* fp8_free, int32_t* tq3_free, int32_t* tops, int recent, int32_t* ws,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(lifecycle_plan, dim3(1), dim3(kPlanThreads), 0, stream, bt_offsets, bt_pages, seq_lens, batch,
                     bt_capacity, tier, g.n_fp8, g.n_tq3, fp8_free, tq3_free, tops, recent, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const TableUpdate upd{bt_pages, tier, fp8_free, ws + 4 + 2 * batch, ws + 2};
  return launch_demote_listed(g, lt, n_layers, ws + 4, ws + 4 + batch, batch, ws + 1, &upd, stream);
}

hipError_t launch_lifecycle_release(const Geometry& g, const int32_t* bt_offsets, const int32_t* bt_pages,
                                    int32_t* seq_lens, int batch, int bt_capacity, uint8_t* tier, int32_t* fp8_free,
                                    int32_t* tq3_free, int32_t* tops, const int32_t* requests, int n_req, int32_t* ws,
                                    hipStream_t stream) {
  hipLaunchKernelGGL(lifecycle_release, dim3(1), dim3(kPlanThreads), 0, stream, bt_offsets, bt_pages, seq_lens, batch,
                     bt_capacity, tier, g.n_fp8, g.n_tq3, fp8_free, tq3_free, tops, requests, n_req, ws);
  return hipGetLastError();
}

}  // namespace mkv
