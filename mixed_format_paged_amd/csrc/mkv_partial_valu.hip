// mkv_partial_valu.hip -- plain VALU partial-attention kernels (FP8 and TQ3).
//
// The format-specific kernels of Minima-KV compute partial attention states
// over the pages of one format (arXiv 2608.23834, page 1, Abstract).  This is
// the straightforward vector-ALU formulation, kept as the measured baseline
// for the matrix-core kernels in mkv_partial_mfma.hip:
//   one workgroup per (layer, chunk, KV head) work item; per page the
//   workgroup dequantises the page's K and V rows of that head into LDS as
//   fp32, forms the G x 16 scores in fp32, runs the online-softmax update
//   (running max m, denominator l, in log2 units) and accumulates P V.
// The partial state (m, l, unnormalised acc) is written per work item.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

template <int D>
__device__ inline float tq3_value(const uint8_t* blk, int kv, int t, int c) {
  int slot;
  const int off = kv ? tq3_v_triple(D, t, c, &slot) : tq3_k_triple(D, t, c, &slot);
  const uint32_t w = (uint32_t)blk[off] | ((uint32_t)blk[off + 1] << 8) | ((uint32_t)blk[off + 2] << 16);
  const int u = (int)((w >> (3 * slot)) & 7u);
  const uint16_t sb = *reinterpret_cast<const uint16_t*>(blk + tq3_scale_off(D, kv, t, c >> 5));
  return (float)(u - 4) * half_bits_to_float(sb);
}

}  // namespace

template <bool TQ3, int D>
__global__ void __launch_bounds__(256) partial_valu_kernel(
    LayerTable lt, int n_layers, int hkv, int G, const float* __restrict__ q,
    size_t q_layer_stride, float qscale, Plan plan) {
  __shared__ float Ks[kPage][D];
  __shared__ float Vs[kPage][D];
  __shared__ float Qs[kMaxGroup][D];
  __shared__ float S[kMaxGroup][kPage];
  __shared__ float alpha_s[kMaxGroup], m_s[kMaxGroup], l_s[kMaxGroup];
  constexpr int kPer = kMaxGroup * D / 256;
  const int tid = threadIdx.x;
  // a workspace without this batch's plan is refused, not read
  if (plan.totals[T_STAMP] != plan_stamp(plan)) {
    if (blockIdx.x == 0 && tid == 0) atomicOr(plan.status, kDevNoPlan);
    return;
  }
  const int n_chunks = plan.totals[TQ3 ? T_NCT : T_NCF];
  const int4* chunks = TQ3 ? plan.chunks_t : plan.chunks_f;
  const int32_t* list = TQ3 ? plan.list_t : plan.list_f;
  const int hq = hkv * G;
  const long items = (long)n_layers * hkv * n_chunks;
  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int h = (int)(item % hkv);
    const int chunk = (int)((item / hkv) % n_chunks);
    const int layer = (int)(item / ((long)hkv * n_chunks));
    const int4 cd = chunks[(kChunkInts / 4) * chunk];
    const int b = cd.x, start = cd.y, count = chunk_pages(cd.z), last_tok = chunk_last_tok(cd.z), pidx = cd.w;
    if (pidx >= plan.np_cap) {                 // plan made for more layers than this call
      if (tid == 0) atomicOr(plan.status, kDevBadSeqLen);
      continue;
    }
    const float* qb = q + layer * q_layer_stride + ((size_t)b * hq + (size_t)h * G) * D;
    for (int idx = tid; idx < G * D; idx += 256) Qs[idx / D][idx % D] = qb[idx] * qscale;
    if (tid < G) { m_s[tid] = -INFINITY; l_s[tid] = 0.0f; }
    float acc[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) acc[k] = 0.0f;
    const float ks = TQ3 ? 1.0f : lt.k_scale[layer];
    const float vs = TQ3 ? 1.0f : lt.v_scale[layer];
    __syncthreads();
    for (int e = 0; e < count; ++e) {
      const int pid = list[start + e];
      const int ntok = (e == count - 1) ? last_tok : kPage;
      if (TQ3) {
        const uint8_t* blk = lt.tq3[layer] + (size_t)pid * tq3_page_bytes(hkv, D) + (size_t)h * tq3_head_bytes(D);
        for (int idx = tid; idx < kPage * D; idx += 256) {
          const int t = idx / D, c = idx % D;
          Ks[t][c] = tq3_value<D>(blk, 0, t, c);
          Vs[t][c] = tq3_value<D>(blk, 1, t, c);
        }
      } else {
        const uint8_t* pg = lt.fp8[layer] + (size_t)pid * fp8_page_bytes(hkv, D) + (size_t)h * 2 * kPage * D;
        for (int idx = tid; idx < kPage * D; idx += 256) {
          const int t = idx / D, c = idx % D;
          Ks[t][c] = e4m3_decode(pg[idx]) * ks;
          Vs[t][c] = e4m3_decode(pg[kPage * D + idx]) * vs;
        }
      }
      __syncthreads();
      for (int idx = tid; idx < G * kPage; idx += 256) {
        const int i = idx / kPage, t = idx % kPage;
        float s = 0.0f;
        for (int c = 0; c < D; ++c) s = fmaf(Qs[i][c], Ks[t][c], s);
        S[i][t] = (t < ntok) ? s : -INFINITY;
      }
      __syncthreads();
      if (tid < G) {
        float pm = -INFINITY;
        for (int t = 0; t < kPage; ++t) pm = fmaxf(pm, S[tid][t]);
        const float mn = fmaxf(m_s[tid], pm);
        const float a = exp2f(m_s[tid] - mn);
        float l = l_s[tid] * a;
        for (int t = 0; t < kPage; ++t) {
          const float p = exp2f(S[tid][t] - mn);
          S[tid][t] = p;
          l += p;
        }
        l_s[tid] = l;
        m_s[tid] = mn;
        alpha_s[tid] = a;
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int idx = tid + 256 * k;
        if (idx < G * D) {
          const int i = idx / D, c = idx % D;
          float a = acc[k] * alpha_s[i];
          for (int t = 0; t < kPage; ++t) a = fmaf(S[i][t], Vs[t][c], a);
          acc[k] = a;
        }
      }
      __syncthreads();
    }
    float* ml = plan.part_ml + part_ml_index(plan.np_cap, hkv, G, layer, h, pidx, 0);
    if (tid < G) { ml[2 * tid] = m_s[tid]; ml[2 * tid + 1] = l_s[tid]; }
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int idx = tid + 256 * k;
      if (idx < G * D) plan.part_acc[part_acc_index(plan.np_cap, hkv, D, G, layer, h, pidx, idx / D, idx % D)] = acc[k];
    }
    __syncthreads();
  }
}

static int grid_for(int items_cap) { return items_cap < 2048 ? (items_cap > 0 ? items_cap : 1) : 2048; }

hipError_t launch_partial_valu(bool tq3, const Geometry& g, const LayerTable& lt, int n_layers,
                               const float* q, size_t q_layer_stride, float qscale,
                               const Plan& plan, hipStream_t stream) {
  const dim3 grid(grid_for(n_layers * g.hkv * plan.np_cap / 2)), block(256);
  if (tq3) {
    if (g.d == 256)
      hipLaunchKernelGGL((partial_valu_kernel<true, 256>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
    else
      hipLaunchKernelGGL((partial_valu_kernel<true, 128>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
  } else {
    if (g.d == 256)
      hipLaunchKernelGGL((partial_valu_kernel<false, 256>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
    else
      hipLaunchKernelGGL((partial_valu_kernel<false, 128>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
  }
  return hipGetLastError();
}

}  // namespace mkv
