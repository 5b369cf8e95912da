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

// Exclusive scan of one value per thread over a block of BLOCK threads (T is
// int or a pair of int counts packed in a 64-bit word, which add field-wise
// as long as each field's total stays below 2^32).  Each wave scans its 64
// values with shuffles, one wave scans the wave totals, two barriers in all.
template <int BLOCK, typename T>
__device__ T block_exclusive_scan(T v, T* total, T* sh) {
  static_assert(BLOCK % 64 == 0 && BLOCK / 64 <= 64, "block of whole waves");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  T x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const T y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = lane < BLOCK / 64 ? sh[lane] : T(0);
#pragma unroll
    for (int o = 1; o < BLOCK / 64; o <<= 1) {
      const T y = __shfl_up(w, o);
      if (lane >= o) w += y;
    }
    if (lane < BLOCK / 64) sh[64 + lane] = w;                       // inclusive wave prefix
  }
  __syncthreads();
  const T before = wave ? sh[64 + wave - 1] : T(0);
  *total = sh[64 + BLOCK / 64 - 1];
  __syncthreads();                                              // sh is reused by the caller
  return before + x - v;
}

// Bitwise OR of the MKV_DEV_* bits over the block (__syncthreads_or is a
// logical OR, so one call per bit).
__device__ inline int block_or_bits(int v) {
  return (__syncthreads_or(v & kDevBadPageId) ? kDevBadPageId : 0) |
         (__syncthreads_or(v & kDevBadTier) ? kDevBadTier : 0) |
         (__syncthreads_or(v & kDevBadSeqLen) ? kDevBadSeqLen : 0);
}

__device__ inline uint64_t pack2(int a, int b) { return (uint64_t)(uint32_t)a | ((uint64_t)(uint32_t)b << 32); }
__device__ inline int lo32(uint64_t x) { return (int)(uint32_t)x; }
__device__ inline int hi32(uint64_t x) { return (int)(uint32_t)(x >> 32); }

__device__ inline int* req_row(const Plan& p, int field) { return p.req + (size_t)field * (p.batch + 1); }

constexpr int kClassifyThreads = 1024;
constexpr int kPlanLdsRows = 1025;                  // per-request rows of batches up to 1024 go to LDS
constexpr int kClassifyPages = 8;

}  // namespace

__global__ void __launch_bounds__(kClassifyThreads) plan_classify(
    const uint8_t* __restrict__ tier, int n_fp8, int n_tq3, const int32_t* __restrict__ bt_offsets,
    const int32_t* __restrict__ bt_pages, const int32_t* __restrict__ seq_lens, Plan plan) {
  constexpr int P = kClassifyPages;                 // consecutive logical pages per thread
  constexpr int SUPER = kClassifyThreads * P;
  __shared__ int sh[128];
  __shared__ int s_last, s_prev_fmt, s_prev_idx;
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
      req_row(plan, R_PREVFMT)[b] = -1;
      req_row(plan, R_PREVIDX)[b] = -1;
    }
    return;
  }
  if (tid == 0) { s_last = -1; s_prev_fmt = -1; s_prev_idx = -1; }
  int nf = 0;      // FP8 pages before the current super-block (block-uniform)
  int err = 0;     // per-thread error bits
  for (int base = 0; base < n; base += SUPER) {
    const int lp0 = base + tid * P;
    // every id first, then every tier byte: two dependent round trips per super-block
    int id[P];
#pragma unroll
    for (int k = 0; k < P; ++k) id[k] = lp0 + k < n ? bt_pages[off0 + lp0 + k] : -1;
    int isf = 0, cnt = 0;                          // bit k: page k is FP8
#pragma unroll
    for (int k = 0; k < P; ++k) {
      if (lp0 + k >= n) continue;
      if (id[k] < 0 || id[k] >= n_fp8 + n_tq3) {
        err |= kDevBadPageId;
        continue;
      }
      const int tr = tier[id[k]];
      if (tr == kTierRecent || tr == kTierAnchor) {
        if (id[k] < n_fp8) { isf |= 1 << k; ++cnt; } else err |= kDevBadTier;
      } else if (tr == kTierStale) {
        if (id[k] < n_fp8) err |= kDevBadTier;
      } else {
        err |= kDevBadTier;
      }
    }
    int tot;
    const int fpos = block_exclusive_scan<kClassifyThreads>(cnt, &tot, sh);
    int fb = 0;                                    // FP8 pages before page k within this thread
#pragma unroll
    for (int k = 0; k < P; ++k) {
      const int lp = lp0 + k;
      if (lp >= n) continue;
      const bool f = (isf >> k) & 1;
      const int at = f ? off0 + nf + fpos + fb : off0 + (lp - nf - fpos - fb);
      if (f) plan.list_f[at] = id[k];
      else plan.list_t[at] = id[k] - n_fp8;
      fb += f;
      if (lp == n - 1) s_last = f ? 0 : 1;
      if (lp == n - 2) { s_prev_fmt = f ? 0 : 1; s_prev_idx = at; }
    }
    nf += tot;
  }
  const int e = block_or_bits(err);
  if (tid == 0) {
    req_row(plan, R_NF)[b] = e ? 0 : nf;
    req_row(plan, R_NT)[b] = e ? 0 : n - nf;
    req_row(plan, R_TAIL)[b] = n ? sl - 16 * (n - 1) : 0;
    req_row(plan, R_LASTFMT)[b] = e ? -1 : s_last;
    req_row(plan, R_INVALID)[b] = e;
    req_row(plan, R_PREVFMT)[b] = e ? -1 : s_prev_fmt;
    req_row(plan, R_PREVIDX)[b] = e ? -1 : s_prev_idx;
  }
}

// The per-request rows in LDS (batches up to kPlanLdsRows - 1 requests):
// counts, error bits, tail, last page's format, block-table offset, then the
// chunk and partial offsets the kernel computes.
enum { L_NF, L_NT, L_INVAL, L_TAIL, L_LAST, L_BTO, L_CF, L_CT, L_PO, kLdsRowCount };

__global__ void __launch_bounds__(1024) plan_chunks(const int32_t* __restrict__ bt_offsets, Plan plan) {
  __shared__ uint64_t sh[128];
  __shared__ int s_rows[kLdsRowCount][kPlanLdsRows];
  const int tid = threadIdx.x;
  const int B = plan.batch;
  // One round of loads up front: the per-request rows plan_classify wrote;
  // everything after reads them, and the offsets computed here, from LDS
  // (with a batch past kPlanLdsRows - 1, from global memory as written).  The
  // page lists stay in global memory: the tables read 12 ids per chunk.
  const bool rows_lds = B + 1 <= kPlanLdsRows;            // uniform
  if (rows_lds) {
    for (int b = tid; b < B; b += 1024) {
      s_rows[L_NF][b] = req_row(plan, R_NF)[b];
      s_rows[L_NT][b] = req_row(plan, R_NT)[b];
      s_rows[L_INVAL][b] = req_row(plan, R_INVALID)[b];
      s_rows[L_TAIL][b] = req_row(plan, R_TAIL)[b];
      s_rows[L_LAST][b] = req_row(plan, R_LASTFMT)[b];
      s_rows[L_BTO][b] = bt_offsets[b];
    }
  }
  __syncthreads();
  const int* nf_row = rows_lds ? s_rows[L_NF] : req_row(plan, R_NF);
  const int* nt_row = rows_lds ? s_rows[L_NT] : req_row(plan, R_NT);
  const int* inval = rows_lds ? s_rows[L_INVAL] : req_row(plan, R_INVALID);
  // totals of pages per format, and the OR of every request's error bits
  int sf = 0, st = 0, serr = 0;
  for (int b = tid; b < B; b += 1024) {
    sf += nf_row[b];
    st += nt_row[b];
    serr |= inval[b];
  }
  uint64_t tot2;
  block_exclusive_scan<1024>(pack2(sf, st), &tot2, sh);
  const int TF = lo32(tot2), TT = hi32(tot2);
  const int status = block_or_bits(serr);
  // Chunk size: every (request, format) segment is cut into chunks of
  // balanced size (floor or ceil of n / chunks): a TQ3 segment of n pages
  // into ceil(n / P), an FP8 one into fp8_chunk_count(n, P) (its pages weigh
  // 4/3), with P the smallest size (at least kMinChunkPages) that keeps the
  // chunk count within chunks_target, so the items fill the CUs once with the
  // least work per item.  P = ceil(W / (target - 2 B)), W the weighted page
  // total, always fits (each segment adds at most one part-filled chunk); a
  // binary search below it finds the smallest.  Past kMaxChunkPages pages per
  // chunk, longer contexts get more chunks than the target instead.
  const int target = plan.chunks_target;
  const int tgt = max(1, target - 2 * B);
  const long long W = (long long)TT + ((long long)TF * kFp8WeightNum + kFp8WeightDen - 1) / kFp8WeightDen;
  auto size_for = [&](long long div) {
    const long long p = (W + div - 1) / div;
    return (int)(p < kMinChunkPages ? kMinChunkPages : (p > kMaxChunkPages ? kMaxChunkPages : p));
  };
  int p_hi = size_for(tgt);
  int p_lo = min(p_hi, size_for(max(1, target)));
  while (p_lo < p_hi) {                                   // uniform over the block
    const int mid = (p_lo + p_hi) >> 1;
    int c = 0;
    for (int b = tid; b < B; b += 1024) c += fp8_chunk_count(nf_row[b], mid) + (nt_row[b] + mid - 1) / mid;
    int tot;
    block_exclusive_scan<1024>(c, &tot, reinterpret_cast<int*>(sh));
    if (tot <= target) p_hi = mid; else p_lo = mid + 1;
  }
  const int ppt = p_hi;
  // per-request counts and their prefix sums
  int carry_f = 0, carry_t = 0, carry_p = 0;
  for (int base = 0; base < B; base += 1024) {
    const int b = base + tid;
    int nfc = 0, ntc = 0;
    if (b < B) {
      nfc = fp8_chunk_count(nf_row[b], ppt);
      ntc = (nt_row[b] + ppt - 1) / ppt;
    }
    uint64_t t2;
    const uint64_t e2 = block_exclusive_scan<1024>(pack2(nfc, ntc), &t2, sh);
    const int ef = lo32(e2), et = hi32(e2), ep = ef + et;
    const int tf = lo32(t2), tt = hi32(t2), tp = tf + tt;
    if (b < B) {
      req_row(plan, R_CF_OFF)[b] = carry_f + ef;   // chunk offsets (exclusive) per format
      req_row(plan, R_CT_OFF)[b] = carry_t + et;
      req_row(plan, R_POFF)[b] = carry_p + ep;
      if (rows_lds) {
        s_rows[L_CF][b] = carry_f + ef;
        s_rows[L_CT][b] = carry_t + et;
        s_rows[L_PO][b] = carry_p + ep;
      }
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
    plan.totals[T_PPF] = ppt;
    plan.totals[T_PPT] = ppt;
    plan.totals[T_STAMP] = plan_stamp(plan);
    if (rows_lds) {
      s_rows[L_CF][B] = carry_f;
      s_rows[L_CT][B] = carry_t;
      s_rows[L_PO][B] = carry_p;
    }
  }
  __syncthreads();
  const int* cf = rows_lds ? s_rows[L_CF] : req_row(plan, R_CF_OFF);
  const int* ct = rows_lds ? s_rows[L_CT] : req_row(plan, R_CT_OFF);
  const int* po = rows_lds ? s_rows[L_PO] : req_row(plan, R_POFF);
  const int* tail = rows_lds ? s_rows[L_TAIL] : req_row(plan, R_TAIL);
  const int* lastfmt = rows_lds ? s_rows[L_LAST] : req_row(plan, R_LASTFMT);
  const int* bto = rows_lds ? s_rows[L_BTO] : bt_offsets;
  // chunk tables, one thread per chunk; the owning request by binary search
  for (int fmt = 0; fmt < 2; ++fmt) {
    const int* co = fmt ? ct : cf;
    const int total = co[B];
    const int* cnt = fmt ? nt_row : nf_row;
    const int* lst = fmt ? plan.list_t : plan.list_f;
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
      // balanced cut of the segment's n pages into nchunks chunks
      const int n_seg = cnt[b];
      const int start = (int)((int64_t)local * n_seg / nchunks);
      const int count = (int)((int64_t)(local + 1) * n_seg / nchunks) - start;
      const bool holds_tail = local == nchunks - 1 && lastfmt[b] == fmt;
      const int last_tok = holds_tail ? tail[b] : 16;
      const int pidx = po[b] + (fmt ? (cf[b + 1] - cf[b]) : 0) + local;
      const int first = bto[b] + start;
      int4* const ent = out + (kChunkInts / 4) * c;
      ent[0] = make_int4(b, first, count | (last_tok << 16) | (holds_tail ? kChunkHoldsTail : 0), pidx);
      int fid[kItemWaves];
#pragma unroll
      for (int w = 0; w < kItemWaves; ++w) fid[w] = lst[first + chunk_order(min(w, count - 1), count, holds_tail)];
#pragma unroll
      for (int q = 0; q < kItemWaves / 4; ++q) ent[1 + q] = make_int4(fid[4 * q], fid[4 * q + 1], fid[4 * q + 2], fid[4 * q + 3]);
    }
  }
}

hipError_t launch_plan(const Geometry& g, const uint8_t* tier, const int32_t* bt_offsets,
                       const int32_t* bt_pages, const int32_t* seq_lens, const Plan& plan,
                       hipStream_t stream) {
  hipError_t e;
  if (plan.batch > 0) {
    hipLaunchKernelGGL(plan_classify, dim3(plan.batch), dim3(kClassifyThreads), 0, stream, tier, g.n_fp8,
                       g.n_tq3, bt_offsets, bt_pages, seq_lens, plan);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(plan_chunks, dim3(1), dim3(1024), 0, stream, bt_offsets, plan);
  return hipGetLastError();
}

}  // namespace mkv
