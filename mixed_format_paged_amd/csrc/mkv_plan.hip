// mkv_plan.hip -- split-K plan for mixed-format decode, computed on device.
//
// The pages route each page to the kernel of its format (arXiv 2608.23834,
// page 1, Abstract: format-specific kernels compute partial attention
// states).  For one decode step (shared by every layer, since all layers use
// the same tier map and block tables):
//   plan_classify  (one workgroup per request): walk the request's logical
//                  pages, check ids and tiers, and compact them into an FP8
//                  list (tier R/A) and a TQ3 list (tier S) in logical order,
//                  stored in the request's own CSR range.
//   plan_chunks    (one workgroup): choose one pages-per-chunk for both
//                  formats so that the whole batch yields about kTargetItems
//                  work items (one per workgroup slot of the GPU), prefix-sum
//                  chunk and partial counts over requests and write the chunk
//                  tables.
// Device-data errors set MKV_DEV_* bits and mark the request invalid (its
// outputs become NaN); nothing is ever read out of bounds.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

// Exclusive scan of one int per thread over a block of BLOCK threads.
template <int BLOCK>
__device__ int block_exclusive_scan(int v, int* total, int* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < BLOCK; off <<= 1) {
    int add = (tid >= off) ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[BLOCK - 1];
  __syncthreads();
  return incl - v;
}

__device__ inline int* req_row(const Plan& p, int field) { return p.req + (size_t)field * (p.batch + 1); }

}  // namespace

__global__ void __launch_bounds__(256) plan_classify(
    const uint8_t* __restrict__ tier, int n_fp8, int n_tq3, const int32_t* __restrict__ bt_offsets,
    const int32_t* __restrict__ bt_pages, const int32_t* __restrict__ seq_lens, Plan plan) {
  __shared__ int sh[256];
  __shared__ int s_last;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int off0 = bt_offsets[b], off1 = bt_offsets[b + 1];
  const int sl = seq_lens[b];
  const int n = (sl + 15) >> 4;
  const bool bad = sl < 0 || off0 < 0 || off1 < off0 || off1 > plan.bt_capacity || n > off1 - off0;
  if (bad) {
    if (tid == 0) {
      req_row(plan, R_NF)[b] = 0;
      req_row(plan, R_NT)[b] = 0;
      req_row(plan, R_TAIL)[b] = 0;
      req_row(plan, R_LASTFMT)[b] = -1;
      req_row(plan, R_INVALID)[b] = kDevBadSeqLen;
    }
    return;
  }
  if (tid == 0) s_last = -1;
  int nf = 0;      // FP8 pages so far (block-uniform)
  int err = 0;     // per-thread error bits
  for (int base = 0; base < n; base += 256) {
    const int lp = base + tid;
    int is_f = 0, id = -1;
    if (lp < n) {
      id = bt_pages[off0 + lp];
      if (id < 0 || id >= n_fp8 + n_tq3) {
        err |= kDevBadPageId;
      } else {
        const int tr = tier[id];
        if (tr == kTierRecent || tr == kTierAnchor) {
          if (id < n_fp8) is_f = 1; else err |= kDevBadTier;
        } else if (tr == kTierStale) {
          if (id < n_fp8) err |= kDevBadTier;
        } else {
          err |= kDevBadTier;
        }
      }
    }
    int tot;
    const int fpos = block_exclusive_scan<256>(is_f, &tot, sh);
    if (lp < n) {
      if (is_f) plan.list_f[off0 + nf + fpos] = id;
      else plan.list_t[off0 + (lp - nf - fpos)] = id - n_fp8;
      if (lp == n - 1) s_last = is_f ? 0 : 1;
    }
    nf += tot;
  }
  // block OR of the error bits
  sh[tid] = err;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) sh[tid] |= sh[tid + s];
    __syncthreads();
  }
  if (tid == 0) {
    const int e = sh[0];
    req_row(plan, R_NF)[b] = e ? 0 : nf;
    req_row(plan, R_NT)[b] = e ? 0 : n - nf;
    req_row(plan, R_TAIL)[b] = n ? sl - 16 * (n - 1) : 0;
    req_row(plan, R_LASTFMT)[b] = e ? -1 : s_last;
    req_row(plan, R_INVALID)[b] = e;
  }
}

__global__ void __launch_bounds__(1024) plan_chunks(const int32_t* __restrict__ bt_offsets, Plan plan) {
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  const int B = plan.batch;
  int* nf_row = req_row(plan, R_NF);
  int* nt_row = req_row(plan, R_NT);
  // totals of pages per format, and the OR of every request's error bits
  int sf = 0, st = 0, serr = 0;
  for (int b = tid; b < B; b += 1024) {
    sf += nf_row[b];
    st += nt_row[b];
    serr |= req_row(plan, R_INVALID)[b];
  }
  int TF, TT;
  block_exclusive_scan<1024>(sf, &TF, sh);
  block_exclusive_scan<1024>(st, &TT, sh);
  sh[tid] = serr;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) sh[tid] |= sh[tid + s];
    __syncthreads();
  }
  const int status = sh[0];
  __syncthreads();
  // One chunk size for both formats, so the work items of a launch are of
  // equal size whatever the mix: about chunks_target chunks in all, less one
  // tail chunk per request and format, so the items fill one wave of
  // workgroups.
  const int tgt = max(1, plan.chunks_target - 2 * B);
  const int ppf = min(kMaxChunkPages, max(kMinChunkPages, (TF + TT + tgt - 1) / tgt));
  const int ppt = ppf;
  // per-request counts and their prefix sums
  int carry_f = 0, carry_t = 0, carry_p = 0;
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    int nfc = 0, ntc = 0, np = 0;
    if (b < B) {
      nfc = (nf_row[b] + ppf - 1) / ppf;
      ntc = (nt_row[b] + ppt - 1) / ppt;
      np = nfc + ntc;
    }
    int tf, tt, tp;
    const int ef = block_exclusive_scan<1024>(nfc, &tf, sh);
    const int et = block_exclusive_scan<1024>(ntc, &tt, sh);
    const int ep = block_exclusive_scan<1024>(np, &tp, sh);
    if (b < B) {
      req_row(plan, R_CF_OFF)[b] = carry_f + ef;   // chunk offsets (exclusive) per format
      req_row(plan, R_CT_OFF)[b] = carry_t + et;
      req_row(plan, R_POFF)[b] = carry_p + ep;
    }
    carry_f += tf; carry_t += tt; carry_p += tp;
  }
  // Chunk counts cannot exceed the capacity for valid CSR offsets; guard anyway.
  const bool over = carry_f > plan.table_cap || carry_t > plan.table_cap;
  if (over) { carry_f = 0; carry_t = 0; carry_p = 0; }
  if (tid == 0) {
    plan.status[0] = status | (over ? kDevBadSeqLen : 0);
    req_row(plan, R_CF_OFF)[B] = carry_f;
    req_row(plan, R_CT_OFF)[B] = carry_t;
    req_row(plan, R_POFF)[B] = carry_p;
    plan.totals[T_NCF] = carry_f;
    plan.totals[T_NCT] = carry_t;
    plan.totals[T_NP] = carry_p;
    plan.totals[T_PPF] = ppf;
    plan.totals[T_PPT] = ppt;
  }
  __syncthreads();
  const int* cf = req_row(plan, R_CF_OFF);
  const int* ct = req_row(plan, R_CT_OFF);
  const int* po = req_row(plan, R_POFF);
  const int* tail = req_row(plan, R_TAIL);
  const int* lastfmt = req_row(plan, R_LASTFMT);
  // chunk tables, one thread per chunk; the owning request by binary search
  for (int fmt = 0; fmt < 2; ++fmt) {
    const int* co = fmt ? ct : cf;
    const int total = co[B];
    const int pp = fmt ? ppt : ppf;
    const int* cnt = fmt ? nt_row : nf_row;
    int4* out = fmt ? plan.chunks_t : plan.chunks_f;
    for (int c = tid; c < total && c < plan.table_cap; c += 1024) {
      int lo = 0, hi = B - 1;                 // last b with co[b] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (co[mid] <= c) lo = mid; else hi = mid - 1;
      }
      const int b = lo;
      const int local = c - co[b];
      const int nchunks = co[b + 1] - co[b];
      const int start = local * pp;
      const int count = min(pp, cnt[b] - start);
      const int last_tok = (local == nchunks - 1 && lastfmt[b] == fmt) ? tail[b] : 16;
      const int pidx = po[b] + (fmt ? (cf[b + 1] - cf[b]) : 0) + local;
      out[c] = make_int4(b, bt_offsets[b] + start, count | (last_tok << 16), pidx);
    }
  }
}

hipError_t launch_plan(const Geometry& g, const uint8_t* tier, const int32_t* bt_offsets,
                       const int32_t* bt_pages, const int32_t* seq_lens, const Plan& plan,
                       hipStream_t stream) {
  hipError_t e;
  if (plan.batch > 0) {
    hipLaunchKernelGGL(plan_classify, dim3(plan.batch), dim3(256), 0, stream, tier, g.n_fp8,
                       g.n_tq3, bt_offsets, bt_pages, seq_lens, plan);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_chunks, dim3(1), dim3(1024), 0, stream, bt_offsets, plan);
  return hipGetLastError();
}

}  // namespace mkv
