// mkv_materialize.hip -- dequantise a range of a request's pages to dense BF16.
//
// Minima-KV's quality profile runs on materialised pages (arXiv 2608.23834,
// page 1, Abstract), while its decode path
// reads the mixed pages in place, avoiding the dequantisation of stale pages
// into a dense buffer (page 2, "Technical Deep Dive").  This kernel is that
// dense buffer: the comparison the decode path is measured against, and the
// input a dense-attention consumer would need.
//
// Element values: FP8 page bf16_RNE(fl32(decode(e) * scale)); TQ3 page
// bf16_RNE((u - 4) * s), where (u - 4) * s is exact in fp32 (11 + 3 bits).
// One workgroup per (logical page, KV head): an FP8 page-head converts from
// global memory directly; a TQ3 head block (14 d bytes) is first staged in
// LDS, then each thread writes whole 16-byte chunks of 8 channels of one
// token, so the stores of a workgroup are contiguous rows.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

constexpr int kThreads = 256;

// bf16 bits of a finite fp32 value, round to nearest, ties to even.
__device__ inline uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline uint32_t tq3_code_at(const uint8_t* blk, int off, int slot) {
  const uint32_t w = blk[off] | ((uint32_t)blk[off + 1] << 8) | ((uint32_t)blk[off + 2] << 16);
  return (w >> (3 * slot)) & 7u;
}

}  // namespace

template <int D>
__global__ void __launch_bounds__(kThreads) materialize_kernel(
    const uint8_t* __restrict__ fp8_slab, const uint8_t* __restrict__ tq3_slab, int n_fp8, int n_tq3,
    float k_scale, float v_scale, int hkv, const int32_t* __restrict__ bt_offsets,
    const int32_t* __restrict__ bt_pages, int bt_capacity, int b, int page_lo, int n_pages,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out) {
  constexpr int C8 = D / 8;                          // 16-byte output chunks per token row
  constexpr int kChunks = 2 * kPage * C8;            // K and V chunks of a page-head
  __shared__ __align__(16) uint8_t blk[14 * D];
  const int off0 = bt_offsets[b], off1 = bt_offsets[b + 1];
  const long units = (long)n_pages * hkv;
  for (long unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const int lp = (int)(unit / hkv), h = (int)(unit % hkv);
    const long entry = (long)off0 + page_lo + lp;
    // outside the request's table (or the block-table array): no page
    const bool listed = off0 >= 0 && entry < off1 && entry < bt_capacity;
    const int id = listed ? bt_pages[entry] : -1;
    const bool fp8 = id >= 0 && id < n_fp8;
    const bool tq3 = id >= n_fp8 && id < n_fp8 + n_tq3;
    if (tq3) {                                       // uniform per workgroup
      const uint4* src = reinterpret_cast<const uint4*>(tq3_slab + (size_t)(id - n_fp8) * tq3_page_bytes(hkv, D) +
                                                        (size_t)h * tq3_head_bytes(D));
      for (int e = threadIdx.x; e < 14 * D / 16; e += kThreads) reinterpret_cast<uint4*>(blk)[e] = src[e];
      __syncthreads();
    }
    for (int q = threadIdx.x; q < kChunks; q += kThreads) {
      const int kv = q / (kPage * C8), t = (q / C8) % kPage, c8 = q % C8;
      uint32_t w[4];
      if (fp8) {
        const uint8_t* src = fp8_slab + (size_t)id * fp8_page_bytes(hkv, D) + ((size_t)(h * 2 + kv) * kPage + t) * D + 8 * c8;
        const uint2 e = *reinterpret_cast<const uint2*>(src);
        const float sc = kv ? v_scale : k_scale;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t word = i < 2 ? e.x : e.y;
          const int sh = 16 * (i & 1);
          const float lo = __fmul_rn(e4m3_decode((word >> sh) & 0xffu), sc);
          const float hi = __fmul_rn(e4m3_decode((word >> (sh + 8)) & 0xffu), sc);
          w[i] = bf16_rne(lo) | (bf16_rne(hi) << 16);
        }
      } else if (tq3) {
        const int c0 = 8 * c8;
        const float s = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + tq3_scale_off(D, kv, t, c0 >> 5)));
        float x[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          int slot;
          const int off = kv ? tq3_v_triple(D, t, c0 + k, &slot) : tq3_k_triple(D, t, c0 + k, &slot);
          x[k] = (float)((int)tq3_code_at(blk, off, slot) - 4) * s;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = bf16_rne(x[2 * i]) | (bf16_rne(x[2 * i + 1]) << 16);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = 0x7fc07fc0u;   // bf16 NaN: no page in the pool
      }
      uint16_t* dst = (kv ? v_out : k_out) + ((size_t)(lp * kPage + t) * hkv + h) * D + 8 * c8;
      *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (tq3) __syncthreads();                        // blk is rewritten by the next unit
  }
}

hipError_t launch_materialize(const Geometry& g, const uint8_t* fp8_slab, const uint8_t* tq3_slab,
                              float k_scale, float v_scale, const int32_t* bt_offsets,
                              const int32_t* bt_pages, int bt_capacity, int b, int page_lo,
                              int n_pages, uint16_t* k_out, uint16_t* v_out, hipStream_t stream) {
  const long units = (long)n_pages * g.hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)(units < 8192 ? units : 8192));
  if (g.d == 256)
    hipLaunchKernelGGL(materialize_kernel<256>, grid, dim3(kThreads), 0, stream, fp8_slab, tq3_slab, g.n_fp8,
                       g.n_tq3, k_scale, v_scale, g.hkv, bt_offsets, bt_pages, bt_capacity, b, page_lo, n_pages, k_out,
                       v_out);
  else
    hipLaunchKernelGGL(materialize_kernel<128>, grid, dim3(kThreads), 0, stream, fp8_slab, tq3_slab, g.n_fp8,
                       g.n_tq3, k_scale, v_scale, g.hkv, bt_offsets, bt_pages, bt_capacity, b, page_lo, n_pages, k_out,
                       v_out);
  return hipGetLastError();
}

}  // namespace mkv
