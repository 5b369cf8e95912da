// mkv_merge.hip -- globally normalised log-sum-exp merge of partial states.
//
// Minima-KV combines the format-specific partial attention states through a
// globally normalised online-softmax merge (arXiv 2608.23834, page 1,
// Abstract): with partials (m_p, l_p, acc_p) in log2 units,
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  o = sum_p acc_p 2^(m_p - M) / L,
//   lse = (M + log2 L) * ln 2.
// merge1: one item per (layer, KV head, group of <= kMergeFan partials of a
//         request); a request with <= kMergeFan partials is finished here,
//         a longer one leaves one intermediate state per group.
// merge2: one item per (layer, KV head, request) with > kMergeFan partials,
//         merging its intermediates.  The order of summation is fixed, so
//         results are bitwise reproducible run to run.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

__device__ inline const int* req_row(const Plan& p, int field) { return p.req + (size_t)field * (p.batch + 1); }

__device__ inline int find_owner(const int* offs, int B, int x) {   // last b with offs[b] <= x
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int kTile = 64;

// Merge `count` states starting at state index `first` of (ml, acc) with
// [state][hkv][G] layout, for KV head h.  Writes either a final output
// (out != nullptr) or one intermediate state (dst_ml / dst_acc).
template <int D>
__device__ void merge_states(const float* __restrict__ ml, const float* __restrict__ acc,
                             int first, int count, int hkv, int h, int G,
                             float* out_row, float* lse_row, float* dst_ml, float* dst_acc,
                             float (*w)[kMaxG], float* sM, float* sL) {
  constexpr int kPer = kMaxG * D / 256;
  const int tid = threadIdx.x;
  if (tid < G) {
    float M = -INFINITY;
    for (int p = 0; p < count; ++p) M = fmaxf(M, ml[(((size_t)(first + p) * hkv + h) * G + tid) * 2]);
    float L = 0.0f;
    if (M != -INFINITY)
      for (int p = 0; p < count; ++p) {
        const float* e = ml + (((size_t)(first + p) * hkv + h) * G + tid) * 2;
        if (e[0] != -INFINITY) L += e[1] * exp2f(e[0] - M);
      }
    sM[tid] = M;
    sL[tid] = L;
  }
  float a[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) a[k] = 0.0f;
  __syncthreads();
  for (int t0 = 0; t0 < count; t0 += kTile) {
    const int n = min(kTile, count - t0);
    for (int e = tid; e < n * G; e += 256) {
      const int p = e / G, i = e % G;
      const float m = ml[(((size_t)(first + t0 + p) * hkv + h) * G + i) * 2];
      w[p][i] = (m == -INFINITY) ? 0.0f : exp2f(m - sM[i]);
    }
    __syncthreads();
    for (int p = 0; p < n; ++p) {
      const float* src = acc + (((size_t)(first + t0 + p) * hkv + h) * G) * D;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int idx = tid + 256 * k;
        if (idx < G * D) a[k] = fmaf(w[p][idx / D], src[idx], a[k]);
      }
    }
    __syncthreads();
  }
  if (out_row) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = tid + 256 * k;
      if (idx < G * D) {
        const float L = sL[idx / D];
        out_row[idx] = (L > 0.0f) ? a[k] / L : 0.0f;
      }
    }
    if (lse_row && tid < G)
      lse_row[tid] = (sL[tid] > 0.0f) ? (sM[tid] + log2f(sL[tid])) * 0.69314718055994531f : -INFINITY;
  } else {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = tid + 256 * k;
      if (idx < G * D) dst_acc[idx] = a[k];
    }
    if (tid < G) { dst_ml[2 * tid] = sM[tid]; dst_ml[2 * tid + 1] = sL[tid]; }
  }
  __syncthreads();
}

template <int D>
__device__ void write_special(float* out_row, float* lse_row, int G, bool invalid) {
  const int tid = threadIdx.x;
  for (int idx = tid; idx < G * D; idx += 256) out_row[idx] = invalid ? __int_as_float(0x7fc00000) : 0.0f;
  if (lse_row && tid < G) lse_row[tid] = invalid ? __int_as_float(0x7fc00000) : -INFINITY;
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(256) merge1_kernel(int n_layers, int hkv, int G, Plan plan,
                                                     float* __restrict__ out, float* __restrict__ lse,
                                                     size_t out_ls, size_t lse_ls) {
  __shared__ float w[kTile][kMaxG];
  __shared__ float sM[kMaxG], sL[kMaxG];
  const int B = plan.batch;
  const int nm1 = plan.totals[T_NM1];
  const int* m1off = req_row(plan, R_M1OFF);
  const int* poff = req_row(plan, R_POFF);
  const int* ioff = req_row(plan, R_IOFF);
  const int* inval = req_row(plan, R_INVALID);
  const int hq = hkv * G;
  const long items = (long)n_layers * hkv * nm1;
  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int m1 = (int)(item % nm1);
    const int h = (int)((item / nm1) % hkv);
    const int layer = (int)(item / ((long)nm1 * hkv));
    const int b = find_owner(m1off, B, m1);
    const int k = m1 - m1off[b];
    const int p0 = poff[b], np = poff[b + 1] - poff[b];
    float* out_row = out + layer * out_ls + ((size_t)b * hq + (size_t)h * G) * D;
    float* lse_row = lse ? lse + layer * lse_ls + (size_t)b * hq + (size_t)h * G : nullptr;
    const float* ml = plan.part_ml + (size_t)layer * plan.np_cap * hkv * G * 2;
    const float* acc = plan.part_acc + (size_t)layer * plan.np_cap * hkv * G * D;
    const bool over = p0 + np > plan.np_cap || (np > kMergeFan && ioff[b] + k >= plan.ni_cap);
    if (over && threadIdx.x == 0) atomicOr(plan.status, kDevBadSeqLen);
    if (inval[b] || np == 0 || over) {
      write_special<D>(out_row, lse_row, G, inval[b] != 0 || over);
    } else if (np <= kMergeFan) {
      merge_states<D>(ml, acc, p0, np, hkv, h, G, out_row, lse_row, nullptr, nullptr, w, sM, sL);
    } else {
      const int first = p0 + k * kMergeFan;
      const int cnt = min(kMergeFan, np - k * kMergeFan);
      const size_t slot = ((size_t)layer * plan.ni_cap + ioff[b] + k) * hkv + h;
      merge_states<D>(ml, acc, first, cnt, hkv, h, G, nullptr, nullptr,
                      plan.inter_ml + slot * G * 2, plan.inter_acc + slot * G * D, w, sM, sL);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256) merge2_kernel(int n_layers, int hkv, int G, Plan plan,
                                                     float* __restrict__ out, float* __restrict__ lse,
                                                     size_t out_ls, size_t lse_ls) {
  __shared__ float w[kTile][kMaxG];
  __shared__ float sM[kMaxG], sL[kMaxG];
  const int B = plan.batch;
  const int* m1off = req_row(plan, R_M1OFF);
  const int* poff = req_row(plan, R_POFF);
  const int* ioff = req_row(plan, R_IOFF);
  const int* inval = req_row(plan, R_INVALID);
  const int hq = hkv * G;
  const long items = (long)n_layers * hkv * B;
  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int b = (int)(item % B);
    const int h = (int)((item / B) % hkv);
    const int layer = (int)(item / ((long)B * hkv));
    const int np = poff[b + 1] - poff[b];
    const int cnt = m1off[b + 1] - m1off[b];
    if (inval[b] || np <= kMergeFan || poff[b + 1] > plan.np_cap || ioff[b] + cnt > plan.ni_cap)
      continue;                                               // uniform per block
    float* out_row = out + layer * out_ls + ((size_t)b * hq + (size_t)h * G) * D;
    float* lse_row = lse ? lse + layer * lse_ls + (size_t)b * hq + (size_t)h * G : nullptr;
    merge_states<D>(plan.inter_ml + (size_t)layer * plan.ni_cap * hkv * G * 2,
                    plan.inter_acc + (size_t)layer * plan.ni_cap * hkv * G * D, ioff[b], cnt, hkv, h,
                    G, out_row, lse_row, nullptr, nullptr, w, sM, sL);
  }
}

hipError_t launch_merge(const Geometry& g, int n_layers, const Plan& plan, float* out, float* lse,
                        size_t out_ls, size_t lse_ls, hipStream_t stream) {
  const long m1_cap = (long)n_layers * g.hkv * (plan.np_cap / kMergeFan + plan.batch + 1);
  const long m2_cap = (long)n_layers * g.hkv * plan.batch;
  const dim3 g1((unsigned)(m1_cap < 2048 ? m1_cap : 2048)), g2((unsigned)(m2_cap < 1024 ? m2_cap : 1024));
  if (g.d == 256) {
    hipLaunchKernelGGL(merge1_kernel<256>, g1, dim3(256), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
    hipLaunchKernelGGL(merge2_kernel<256>, g2, dim3(256), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
  } else {
    hipLaunchKernelGGL(merge1_kernel<128>, g1, dim3(256), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
    hipLaunchKernelGGL(merge2_kernel<128>, g2, dim3(256), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
  }
  return hipGetLastError();
}

}  // namespace mkv
