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
// Rotated TQ3 pages (the layer has a sign vector; the codes are those of
// y = c H (signs . x)): per token row, the exact y = (u - 4) s goes through the
// format's fast transform in fp32 (stage s = 0, 1, ... pairs channels i and
// i + 2^s as (a + b, a - b)), and x = signs . (H y) / (c d), c d = 16 (exact),
// then bf16_RNE.
// One workgroup per (logical page, KV head): an FP8 page-head converts from
// global memory directly (hardware E4M3 decode, exact); a TQ3 head block
// (14 d bytes) is first staged in LDS, each thread decodes whole triples (8
// codes, one 3-byte read) into a bf16 tile of the page-head in LDS, and then
// every thread writes whole 16-byte chunks of 8 channels of one token, so the
// stores of a workgroup are contiguous rows.
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

}  // namespace

template <int D, bool ROT>
__global__ void __launch_bounds__(kThreads) materialize_kernel(
    const uint8_t* __restrict__ fp8_slab, const uint8_t* __restrict__ tq3_slab, int n_fp8, int n_tq3,
    float k_scale, float v_scale, int hkv, const int32_t* __restrict__ bt_offsets,
    const int32_t* __restrict__ bt_pages, int bt_capacity, int b, int page_lo, int n_pages,
    uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out, const int8_t* __restrict__ signs) {
  constexpr int C8 = D / 8;                          // 16-byte output chunks per token row
  constexpr int kChunks = 2 * kPage * C8;            // K and V chunks of a page-head
  constexpr int G = D / 32;                          // 32-channel scale groups
  constexpr int NTRI = 2 * D;                        // triples of K (and of V) in a head block
  __shared__ __align__(16) uint8_t blk[14 * D];
  __shared__ __align__(16) uint16_t tile[2][kPage][D];   // bf16 bits of a TQ3 page-head, [K/V][token][channel]
  __shared__ __align__(16) float ftile[ROT ? 2 : 1][ROT ? kPage : 1][ROT ? D : 1];   // rotated: fp32 rows
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
      // one triple (8 codes) per step: K triple x of row t holds channels
      // 32 g + 8 j + e of token t (two scale groups), V triple x holds two
      // channels of one group for the 4 tokens of a quarter (four scales);
      // each value (u - 4) s (exact in fp32) goes to the bf16 tile
      for (int tau = threadIdx.x; tau < 2 * NTRI; tau += kThreads) {
        const bool isv = tau >= NTRI;
        const int x = isv ? tau - NTRI : tau;
        const int o = (isv ? 6 * D : 0) + 3 * x;
        const uint32_t w = blk[o] | ((uint32_t)blk[o + 1] << 8) | ((uint32_t)blk[o + 2] << 16);
        if (!isv) {
          const int t = x / (D / 8), xr = x % (D / 8), j = xr / G, r = xr % G;
          const int g0 = 4 * (r >> 2) + ((r >> 1) & 1), g1 = g0 + 2;     // slots s: group g0 + 2 (s & 1)
          const float s0 = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + tq3_scale_off(D, 0, t, g0)));
          const float s1 = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + tq3_scale_off(D, 0, t, g1)));
          const int cb = 8 * j + 4 * (r & 1);
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) {
            const float v = (float)((int)((w >> (3 * sl)) & 7u) - 4) * ((sl & 1) ? s1 : s0);
            const int c = 32 * ((sl & 1) ? g1 : g0) + cb + (sl >> 1);
            if (ROT)
              ftile[0][t][c] = v;
            else
              tile[0][t][c] = (uint16_t)bf16_rne(v);
          }
        } else {
          const int jq = x / (16 * G), rem = x % (16 * G), n = rem / G, p = rem % G;
          const int c0 = n * (D / 16) + 2 * p, g = c0 / 32;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 4 * jq + r;
            const float sc = half_bits_to_float(*reinterpret_cast<const uint16_t*>(blk + tq3_scale_off(D, 1, t, g)));
#pragma unroll
            for (int ci = 0; ci < 2; ++ci) {
              const int sl = tq3_v_slot(ci, r);
              const float v = (float)((int)((w >> (3 * sl)) & 7u) - 4) * sc;
              if (ROT)
                ftile[1][t][c0 + ci] = v;
              else
                tile[1][t][c0 + ci] = (uint16_t)bf16_rne(v);
            }
          }
        }
      }
      __syncthreads();
      if (ROT) {
        // H y for each of the 2 x 16 rows, stage by stage, then the signs and 1/16
        for (int hs = 1; hs < D; hs <<= 1) {
          for (int pp = threadIdx.x; pp < 2 * kPage * (D / 2); pp += kThreads) {
            const int row = pp / (D / 2), r = pp % (D / 2);
            float* const rr = &ftile[row / kPage][row % kPage][(r / hs) * 2 * hs + r % hs];
            const float a = rr[0], b2 = rr[hs];
            rr[0] = a + b2;
            rr[hs] = a - b2;
          }
          __syncthreads();
        }
        for (int e = threadIdx.x; e < 2 * kPage * D; e += kThreads) {
          const int kv = e / (kPage * D), t = (e / D) % kPage, c = e % D;
          const float v = ftile[kv][t][c] * 0.0625f;
          tile[kv][t][c] = (uint16_t)bf16_rne(signs[c] < 0 ? -v : v);
        }
        __syncthreads();
      }
    }
    for (int q = threadIdx.x; q < kChunks; q += kThreads) {
      const int kv = q / (kPage * C8), t = (q / C8) % kPage, c8 = q % C8;
      uint4 o4;
      if (fp8) {
        // exact E4M3 -> fp32 through the hardware conversion, then the scale
        const uint8_t* src = fp8_slab + (size_t)id * fp8_page_bytes(hkv, D) + ((size_t)(h * 2 + kv) * kPage + t) * D + 8 * c8;
        const uint2 e = *reinterpret_cast<const uint2*>(src);
        const float sc = kv ? v_scale : k_scale;
        const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e.x, 1.0f, false);   // bytes 0, 1
        const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e.x, 1.0f, true);    // bytes 2, 3
        const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e.y, 1.0f, false);
        const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(e.y, 1.0f, true);
        auto pk = [&](float a, float b2) { return bf16_rne(__fmul_rn(a, sc)) | (bf16_rne(__fmul_rn(b2, sc)) << 16); };
        o4 = make_uint4(pk(f0[0], f0[1]), pk(f1[0], f1[1]), pk(f2[0], f2[1]), pk(f3[0], f3[1]));
      } else if (tq3) {
        o4 = *reinterpret_cast<const uint4*>(&tile[kv][t][8 * c8]);
      } else {
        o4 = make_uint4(0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u);   // bf16 NaN: no page in the pool
      }
      uint16_t* dst = (kv ? v_out : k_out) + ((size_t)(lp * kPage + t) * hkv + h) * D + 8 * c8;
      *reinterpret_cast<uint4*>(dst) = o4;
    }
    if (tq3) __syncthreads();                        // blk and tile are rewritten by the next unit
  }
}

hipError_t launch_materialize(const Geometry& g, const uint8_t* fp8_slab, const uint8_t* tq3_slab,
                              float k_scale, float v_scale, const int32_t* bt_offsets,
                              const int32_t* bt_pages, int bt_capacity, int b, int page_lo,
                              int n_pages, uint16_t* k_out, uint16_t* v_out, const int8_t* signs,
                              hipStream_t stream) {
  const long units = (long)n_pages * g.hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)(units < 8192 ? units : 8192));
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, stream, fp8_slab, tq3_slab, g.n_fp8, g.n_tq3, k_scale, v_scale,
                       g.hkv, bt_offsets, bt_pages, bt_capacity, b, page_lo, n_pages, k_out, v_out, signs);
  };
  if (g.d == 256)
    signs ? go(materialize_kernel<256, true>) : go(materialize_kernel<256, false>);
  else
    signs ? go(materialize_kernel<128, true>) : go(materialize_kernel<128, false>);
  return hipGetLastError();
}

}  // namespace mkv
