// mkv_merge.hip -- globally normalised log-sum-exp merge of partial states.
//
// Minima-KV combines the format-specific partial attention states through a
// globally normalised online-softmax merge (arXiv 2608.23834, page 1,
// Abstract): with partials (m_p, l_p, acc_p) in log2 units,
//   M = max_p m_p,  w_p = 2^(m_p - M),  L = sum_p l_p w_p,
//   o = sum_p acc_p w_p / L,  lse = (M + log2 L) * ln 2.
// One launch merges any number of partials per request.  A workgroup takes
// (layer, request, KV head, group of up to 8 query rows, slice of 32
// channels), 256 threads (a KV head has R = T G rows: T query tokens per
// request times G heads; row r = t G + g goes to out[b][t][h G + g]):
//   1. each (row, 4-channel column) of the slice is shared by kSubs threads,
//      each taking every kSubs-th partial: its (m, l) pairs and states are
//      requested in one go, kReg at a time;
//   2. the thread folds them with its own running maximum (the same merge,
//      applied to its share): Mt, Lt and its weighted sum;
//   3. the kSubs shares of a (row, column) are merged through LDS in a fixed
//      order: M = max Mt, L = sum Lt 2^(Mt - M), o = sum at 2^(Mt - M) / L.
// The order of every sum is fixed, so results are bitwise reproducible, and
// there is one workgroup barrier per item.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

__device__ inline const int* req_row(const Plan& p, int field) { return p.req + (size_t)field * (p.batch + 1); }

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kSliceC = kStateSlice;             // channels per workgroup: one slice of the state layout
constexpr int kQuads = kSliceC / 4;              // float4 columns of a slice
constexpr int kSubs = kThreads / (kMaxG * kQuads);   // threads sharing one (head, float4 column)
constexpr int kReg = 16;                         // partial states (float4) a thread requests at once

}  // namespace

// Thread t takes float4 column q = t % kQuads of the slice, query row
// i = (t / kQuads) % kMaxG of the row group (idle past its rows) and every kSubs-th partial from
// sub = t / (kQuads kMaxG): its loads are 16-byte vectors, and the kQuads
// threads of one (partial, row) read one contiguous 128-byte line; in the
// state layout (part_acc_index) the rows and then the partials of a request
// follow one another, so a workgroup's states are one contiguous run.
// appended: the partial states come from a launch that appended each
// request's new token to its last logical page (mkv_append_attend).  That page
// must be FP8; a request whose last page is TQ3 could not take the token, so
// its outputs are NaN and the status gets MKV_DEV_BAD_TIER.
template <int D>
__global__ void __launch_bounds__(kThreads) merge_kernel(int n_layers, int hkv, int Gh, Plan plan,
                                                         float* __restrict__ out, float* __restrict__ lse,
                                                         size_t out_ls, size_t lse_ls, int appended) {
  constexpr int NS = D / kSliceC;
  const int T = plan.n_query;
  const int R = T * Gh;                                     // rows per KV head
  const int NRG = (R + kMaxG - 1) / kMaxG;                  // row groups
  __shared__ f4v sa[kThreads];                  // per-thread weighted sums, [sub][i][q]
  __shared__ float sm[kThreads], sl[kThreads];  // per-thread maxima and denominators
  const int B = plan.batch;
  // per-request plan fields through the constant address space: (uniform)
  // scalar loads, requested together
  typedef const __attribute__((address_space(4))) int* cptr;
  const cptr poff = (cptr)req_row(plan, R_POFF);
  const cptr inval = (cptr)req_row(plan, R_INVALID);
  const cptr lastfmt = (cptr)req_row(plan, R_LASTFMT);
  const int hq = hkv * Gh;
  const int tid = threadIdx.x;
  // a workspace without this batch's plan is refused (NaN outputs), not read
  const bool planned = plan.totals[T_STAMP] == plan_stamp(plan);
  if (!planned && blockIdx.x == 0 && tid == 0) atomicOr(plan.status, kDevNoPlan);
  const int qc = tid % kQuads, pi = (tid / kQuads) % kMaxG, sub = tid / (kQuads * kMaxG);
  // 32-bit unsigned item arithmetic (far below 2^31 items per launch)
  const unsigned items = (unsigned)(n_layers * B * hkv * NRG * NS);
  // output element of row r of request b, KV head h
  auto out_at = [&](int layer, int b, int h, int r) {
    const int t = r / Gh;
    return ((size_t)(b * T + t) * hq + (size_t)h * Gh + (r - t * Gh));
  };
  for (unsigned item = blockIdx.x; item < items; item += gridDim.x) {
    const int cs = (int)(item % NS);
    const unsigned irg = item / NS;
    const int rg = (int)(irg % (unsigned)NRG);
    const unsigned ih = irg / (unsigned)NRG;
    const int h = (int)(ih % (unsigned)hkv);
    const unsigned ib = ih / (unsigned)hkv;
    const int b = (int)(ib % (unsigned)B);
    const int layer = (int)(ib / (unsigned)B);
    const int r0 = rg * kMaxG;
    const int G = R - r0 < kMaxG ? R - r0 : kMaxG;          // rows of this group
    const bool live = pi < G;
    const int p0 = planned ? poff[b] : 0, np = planned ? poff[b + 1] - p0 : 0;
    const int bad_append = (planned && appended && lastfmt[b] == 1) ? kDevBadTier : 0;
    const int bad = planned ? (inval[b] | bad_append) : kDevNoPlan;
    if (bad_append && layer == 0 && h == 0 && rg == 0 && cs == 0 && tid == 0) atomicOr(plan.status, bad_append);
    float* out_row = out + layer * out_ls + out_at(layer, b, h, r0 + (live ? pi : 0)) * D + cs * kSliceC;
    float* lse_l = lse ? lse + layer * lse_ls : nullptr;
    if (bad || np == 0 || p0 + np > plan.np_cap) {   // uniform per workgroup
      const bool nan = bad != 0 || np != 0;
      if (sub == 0 && live)
        *reinterpret_cast<f4v*>(out_row + 4 * qc) = nan ? f4v{NAN, NAN, NAN, NAN} : f4v{0.0f, 0.0f, 0.0f, 0.0f};
      if (cs == 0 && lse_l && tid < G) lse_l[out_at(layer, b, h, r0 + tid)] = nan ? __int_as_float(0x7fc00000) : -INFINITY;
      continue;
    }
    // a request's partials are consecutive: R rows of (m, l) and R * 32 floats of
    // the slice's states per partial, one contiguous run
    const int row = r0 + (live ? pi : 0);
    const float* ml = plan.part_ml + part_ml_index(plan.np_cap, hkv, R, layer, h, p0, row);
    const float* acc = plan.part_acc + part_acc_index(plan.np_cap, hkv, D, R, layer, h, p0, row, cs * kSliceC + 4 * qc);
    // 1 + 2: this thread's share, partials sub, sub + kSubs, ..., kReg at a time
    float Mt = -INFINITY, Lt = 0.0f;
    f4v at = f4v{0.0f, 0.0f, 0.0f, 0.0f};
    const int mine = live ? (np - sub + kSubs - 1) / kSubs : 0;
    for (int k0 = 0; k0 < mine; k0 += kReg) {
      const int cnt = mine - k0 < kReg ? mine - k0 : kReg;
      f4v av[kReg];
      float mv[kReg], lv[kReg];
#pragma unroll
      for (int k = 0; k < kReg; ++k) {
        const size_t p = (size_t)(sub + (k0 + k) * kSubs);
        if (k < cnt) {
          av[k] = *reinterpret_cast<const f4v*>(acc + p * R * kSliceC);
          const float2 m_l = *reinterpret_cast<const float2*>(ml + p * R * 2);
          mv[k] = m_l.x;
          lv[k] = m_l.y;
        } else {
          av[k] = f4v{0.0f, 0.0f, 0.0f, 0.0f};
          mv[k] = -INFINITY;
          lv[k] = 0.0f;
        }
      }
      float mx = Mt;
#pragma unroll
      for (int k = 0; k < kReg; ++k) mx = fmaxf(mx, mv[k]);
      if (mx > Mt) {                                        // Mt = -inf: nothing to rescale yet
        const float sc = Mt == -INFINITY ? 0.0f : exp2f(Mt - mx);
        at *= sc;
        Lt *= sc;
        Mt = mx;
      }
#pragma unroll
      for (int k = 0; k < kReg; ++k) {
        const float w = mv[k] == -INFINITY ? 0.0f : exp2f(mv[k] - Mt);
        at += w * av[k];
        Lt += w * lv[k];
      }
    }
    // 3. the kSubs shares of (pi, qc), in sub order
    sa[tid] = at;
    sm[tid] = Mt;
    sl[tid] = Lt;
    __syncthreads();
    if (sub == 0 && live) {
      float M = -INFINITY;
      for (int s2 = 0; s2 < kSubs; ++s2) M = fmaxf(M, sm[s2 * kQuads * kMaxG + tid]);
      f4v o = f4v{0.0f, 0.0f, 0.0f, 0.0f};
      float L = 0.0f;
      for (int s2 = 0; s2 < kSubs; ++s2) {
        const int t2 = s2 * kQuads * kMaxG + tid;
        const float w = sm[t2] == -INFINITY ? 0.0f : exp2f(sm[t2] - M);
        o += w * sa[t2];
        L += w * sl[t2];
      }
      *reinterpret_cast<f4v*>(out_row + 4 * qc) = L > 0.0f ? o / L : f4v{0.0f, 0.0f, 0.0f, 0.0f};
      if (cs == 0 && qc == 0 && lse_l)
        lse_l[out_at(layer, b, h, r0 + pi)] = L > 0.0f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    }
    __syncthreads();
  }
}

hipError_t launch_merge(const Geometry& g, int n_layers, const Plan& plan, float* out, float* lse,
                        size_t out_ls, size_t lse_ls, hipStream_t stream, bool appended) {
  const int R = plan.n_query * g.G;
  const long cap = (long)n_layers * plan.batch * g.hkv * ((R + kMaxG - 1) / kMaxG) * (g.d / kSliceC);
  const dim3 grid((unsigned)(cap < 4096 ? (cap > 0 ? cap : 1) : 4096));
  if (g.d == 256)
    hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(kThreads), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls,
                       appended ? 1 : 0);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kThreads), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls,
                       appended ? 1 : 0);
  return hipGetLastError();
}

}  // namespace mkv
