// mkv_append.hip -- quantise new tokens to FP8 E4M3 on Recent pages.
//
// Minima-KV keeps Recent pages in FP8 (arXiv 2608.23834, page 1, Abstract).
// One workgroup per (request, new token); each thread converts 4 consecutive
// channels and stores them as one 32-bit word.  Byte = e4m3_RNE_sat(x / scale).
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

__global__ void __launch_bounds__(256) append_kernel(
    uint8_t* __restrict__ fp8_slab, int n_fp8, int hkv, int d, float k_scale, float v_scale,
    const float* __restrict__ k, const float* __restrict__ v, int n_new,
    const int32_t* __restrict__ bt_offsets, const int32_t* __restrict__ bt_pages,
    const int32_t* __restrict__ pos, const int32_t* __restrict__ counts) {
  const int b = blockIdx.x / n_new;
  const int i = blockIdx.x - b * n_new;
  if (counts && i >= counts[b]) return;
  const int p = pos[b] + i;
  if (p < 0) return;
  const int lp = p >> 4, slot = p & 15;
  const int off0 = bt_offsets[b], off1 = bt_offsets[b + 1];
  if (lp >= off1 - off0) return;
  const int pid = bt_pages[off0 + lp];
  if (pid < 0 || pid >= n_fp8) return;
  uint8_t* page = fp8_slab + (size_t)pid * fp8_page_bytes(hkv, d);
  const size_t tok = (size_t)blockIdx.x * hkv * d;          // [b][i] row of k and v
  const int quads = hkv * 2 * d / 4;
  for (int e4 = threadIdx.x; e4 < quads; e4 += blockDim.x) {
    const int e = e4 * 4;
    const int h = e / (2 * d);
    const int kv = (e / d) & 1;
    const int c = e % d;
    const float* src = (kv ? v : k) + tok + (size_t)h * d + c;
    const float4 x = *reinterpret_cast<const float4*>(src);
    const float sc = kv ? v_scale : k_scale;
    uint32_t w = e4m3_encode(__fdiv_rn(x.x, sc)) | (e4m3_encode(__fdiv_rn(x.y, sc)) << 8) |
                 (e4m3_encode(__fdiv_rn(x.z, sc)) << 16) | (e4m3_encode(__fdiv_rn(x.w, sc)) << 24);
    *reinterpret_cast<uint32_t*>(page + ((h * 2 + kv) * kPage + slot) * d + c) = w;
  }
}

hipError_t launch_append(const Geometry& g, uint8_t* fp8_slab, float k_scale, float v_scale,
                         const float* k, const float* v, int n_new, const int32_t* bt_offsets,
                         const int32_t* bt_pages, const int32_t* pos, const int32_t* counts,
                         int batch, hipStream_t stream) {
  if (batch == 0 || n_new == 0) return hipSuccess;
  hipLaunchKernelGGL(append_kernel, dim3(batch * n_new), dim3(256), 0, stream, fp8_slab, g.n_fp8,
                     g.hkv, g.d, k_scale, v_scale, k, v, n_new, bt_offsets, bt_pages, pos, counts);
  return hipGetLastError();
}

}  // namespace mkv
