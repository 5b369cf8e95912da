// mkv_merge.hip -- globally normalised log-sum-exp merge of partial states.
//
// Minima-KV combines the format-specific partial attention states through a
// globally normalised online-softmax merge (arXiv 2608.23834, page 1,
// Abstract): with partials (m_p, l_p, acc_p) in log2 units,
//   M = max_p m_p,  L = sum_p l_p 2^(m_p - M),  o = sum_p acc_p 2^(m_p - M) / L,
//   lse = (M + log2 L) * ln 2.
// The order of summation is fixed (partial index order), so results are
// bitwise reproducible run to run.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {
__device__ inline const int* req_row(const Plan& p, int field) { return p.req + (size_t)field * (p.batch + 1); }
}  // namespace

// Single-launch merge: one workgroup per (layer, request, KV head, slice of
// kSliceC channels).  Waves reduce M and L per query head over all the
// request's partials (both formats); each thread then accumulates one
// (head, channel) output over the partials in index order.  No intermediate
// states and no second launch, whatever the number of partials.
constexpr int kSliceC = 32;

template <int D>
__global__ void __launch_bounds__(256) merge_slices_kernel(int n_layers, int hkv, int G, Plan plan,
                                                           float* __restrict__ out, float* __restrict__ lse,
                                                           size_t out_ls, size_t lse_ls) {
  constexpr int NS = D / kSliceC;
  __shared__ float sM[kMaxG], sL[kMaxG];
  const int B = plan.batch;
  const int* poff = req_row(plan, R_POFF);
  const int* inval = req_row(plan, R_INVALID);
  const int hq = hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long items = (long)n_layers * B * hkv * NS;
  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int cs = (int)(item % NS);
    const int h = (int)((item / NS) % hkv);
    const int b = (int)((item / ((long)NS * hkv)) % B);
    const int layer = (int)(item / ((long)NS * hkv * B));
    const int p0 = poff[b], np = poff[b + 1] - poff[b];
    float* out_row = out + layer * out_ls + ((size_t)b * hq + (size_t)h * G) * D;
    float* lse_row = lse ? lse + layer * lse_ls + (size_t)b * hq + (size_t)h * G : nullptr;
    if (inval[b] || np == 0 || p0 + np > plan.np_cap) {   // uniform per block
      const bool nan = inval[b] != 0 || np != 0;
      for (int idx = tid; idx < G * kSliceC; idx += 256)
        out_row[(idx / kSliceC) * D + cs * kSliceC + idx % kSliceC] = nan ? __int_as_float(0x7fc00000) : 0.0f;
      if (cs == 0 && lse_row && tid < G) lse_row[tid] = nan ? __int_as_float(0x7fc00000) : -INFINITY;
      continue;
    }
    const size_t sstride = (size_t)hkv * G;                 // states between consecutive partials
    const float* ml = plan.part_ml + ((size_t)layer * plan.np_cap * hkv + (size_t)p0 * hkv + h) * G * 2;
    const float* acc = plan.part_acc + ((size_t)layer * plan.np_cap * hkv + (size_t)p0 * hkv + h) * G * D;
    // M and L of head i by wave i % 4, lanes strided over the partials
    for (int i = wave; i < G; i += 4) {
      float M = -INFINITY;
      for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[(p * sstride + i) * 2]);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
      float L = 0.0f;
      if (M != -INFINITY)
        for (int p = lane; p < np; p += 64) {
          const float m = ml[(p * sstride + i) * 2];
          if (m != -INFINITY) L += ml[(p * sstride + i) * 2 + 1] * exp2f(m - M);
        }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) L += __shfl_xor(L, o);
      if (lane == 0) { sM[i] = M; sL[i] = L; }
    }
    __syncthreads();
    if (tid < G * kSliceC) {
      const int i = tid / kSliceC, c = cs * kSliceC + tid % kSliceC;
      const float M = sM[i];
      const float* ap = acc + (size_t)i * D + c;
      const float* mp = ml + (size_t)i * 2;
      float a = 0.0f;
#pragma unroll 8
      for (int p = 0; p < np; ++p) {
        const float m = mp[p * sstride * 2];
        const float v = ap[p * sstride * D];
        a = fmaf(m == -INFINITY ? 0.0f : exp2f(m - M), v, a);
      }
      const float L = sL[i];
      out_row[(size_t)i * D + c] = L > 0.0f ? a / L : 0.0f;
    }
    if (cs == 0 && lse_row && tid < G)
      lse_row[tid] = sL[tid] > 0.0f ? (sM[tid] + log2f(sL[tid])) * 0.69314718055994531f : -INFINITY;
    __syncthreads();
  }
}

hipError_t launch_merge(const Geometry& g, int n_layers, const Plan& plan, float* out, float* lse,
                        size_t out_ls, size_t lse_ls, hipStream_t stream) {
  const long cap = (long)n_layers * plan.batch * g.hkv * (g.d / kSliceC);
  const dim3 grid((unsigned)(cap < 4096 ? (cap > 0 ? cap : 1) : 4096));
  if (g.d == 256)
    hipLaunchKernelGGL(merge_slices_kernel<256>, grid, dim3(256), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
  else
    hipLaunchKernelGGL(merge_slices_kernel<128>, grid, dim3(256), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
  return hipGetLastError();
}

}  // namespace mkv
