// mkv_demote.hip -- FP8 -> TQ3 page demotion (the pack).
//
// "Older non-anchor pages move to packed TQ3" (arXiv 2608.23834, page 1,
// Abstract).  One workgroup per (layer, page, KV head):
//   phase 1: one thread per (K/V, token, 32-channel group) decodes the FP8
//            bytes (x = fl32(decode(e) * scale)), takes the absmax, forms the
//            fp16 scale s = fp16_RNE(fl32(a / 3)) and the codes u = q + 4,
//            and leaves codes and scales in LDS;
//   phase 2: each thread assembles four consecutive triples (12 bytes) of the
//            head block from LDS in the documented slot order and stores
//            them as three 32-bit words; scales are stored as fp16.
// The lifecycle's variant takes its page count from device memory and also
// rewrites each demoted page's block-table entry, tier bytes and free-stack
// slot (one workgroup per page does it; nothing else in the launch reads
// them, and the FP8 slot it frees is only reused by a later launch).
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

template <int D>
__global__ void __launch_bounds__(256) demote_kernel(
    LayerTable lt, int n, int n_fp8, int n_tq3, int hkv, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, const int32_t* __restrict__ n_dev, TableUpdate upd) {
  constexpr int G = D / 32;
  __shared__ uint8_t codes[2][kPage][D];
  __shared__ uint16_t scales[2][kPage][G];
  const int layer = blockIdx.x / (n * hkv);
  const int rest = blockIdx.x - layer * n * hkv;
  const int page = rest / hkv;
  const int h = rest - page * hkv;
  const uint8_t* __restrict__ fp8_slab = lt.fp8[layer];
  uint8_t* __restrict__ tq3_slab = lt.tq3[layer];
  const float k_scale = lt.k_scale[layer], v_scale = lt.v_scale[layer];
  if (n_dev && page >= *n_dev) return;                                              // uniform
  const int s_id = src[page];
  const int d_id = dst[page];
  if (s_id < 0 || s_id >= n_fp8 || d_id < n_fp8 || d_id >= n_fp8 + n_tq3) return;   // uniform
  if (upd.bt_pages && layer == 0 && h == 0 && threadIdx.x == 0) {
    upd.bt_pages[upd.entry[page]] = d_id;
    upd.tier[d_id] = kTierStale;
    upd.tier[s_id] = kTierFree;
    upd.fp8_free[*upd.push_base + page] = s_id;
  }
  const uint8_t* in = fp8_slab + (size_t)s_id * fp8_page_bytes(hkv, D) + (size_t)h * 2 * kPage * D;
  uint8_t* out = tq3_slab + (size_t)(d_id - n_fp8) * tq3_page_bytes(hkv, D) + (size_t)h * tq3_head_bytes(D);

  for (int grp = threadIdx.x; grp < 2 * kPage * G; grp += blockDim.x) {
    const int kv = grp / (kPage * G);
    const int t = (grp / G) % kPage;
    const int g = grp % G;
    const float sc = kv ? v_scale : k_scale;
    const uint32_t* row = reinterpret_cast<const uint32_t*>(in + (kv * kPage + t) * D + g * 32);
    float x[32];
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const uint32_t word = row[w];
#pragma unroll
      for (int byte = 0; byte < 4; ++byte) {
        const float val = __fmul_rn(e4m3_decode((word >> (8 * byte)) & 0xffu), sc);
        x[w * 4 + byte] = val;
        a = fmaxf(a, fabsf(val));
      }
    }
    const uint16_t sb = tq3_scale_bits(a);
    const float s = half_bits_to_float(sb);
    scales[kv][t][g] = sb;
#pragma unroll
    for (int c = 0; c < 32; ++c) codes[kv][t][g * 32 + c] = (uint8_t)(tq3_code(x[c], s) + 4);
  }
  __syncthreads();

  // code region: 12 D bytes = 4 D triples; thread handles triples 4 tau .. 4 tau + 3
  for (int tau = threadIdx.x; tau < D; tau += blockDim.x) {
    uint32_t words[3] = {0u, 0u, 0u};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ti = 4 * tau + q;
      uint32_t tw = 0;
      if (ti < 2 * D) {                                  // K triple: row t, triple (j, g)
        const int t = ti / (D / 8);
        const int r = ti - t * (D / 8);
        const int j = r / G, g = r - (r / G) * G;
#pragma unroll
        for (int k = 0; k < 8; ++k) tw |= (uint32_t)codes[0][t][32 * g + 8 * j + k] << (3 * k);
      } else {                                           // V triple: (j, n, p)
        const int tv = ti - 2 * D;
        const int p = tv % G;
        const int jn = tv / G;
        const int n = jn & 15, j = jn >> 4;
        const int a = n * (D / 16) + 2 * p;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          // inverse of the slot table: slot -> (channel-in-pair, token-in-quarter)
          const int ci = (0x3c >> k) & 1;                // slots 2,3,4,5 hold channel b
          const int rr = (0xde18 >> (2 * k)) & 3;        // slot -> r : 0,2,1,0,2,3,1,3
          tw |= (uint32_t)codes[1][4 * j + rr][a + ci] << (3 * k);
        }
      }
      // place the 24-bit triple at byte 3q of the 12-byte window
      const int bit = 24 * q;
      words[bit >> 5] |= tw << (bit & 31);
      if ((bit & 31) > 8) words[(bit >> 5) + 1] |= tw >> (32 - (bit & 31));
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(out + 12 * tau);
    o[0] = words[0];
    o[1] = words[1];
    o[2] = words[2];
  }
  // scales: 2 * 16 * G fp16 values
  for (int e = threadIdx.x; e < 2 * kPage * G; e += blockDim.x) {
    const int kv = e / (kPage * G);
    const int t = (e / G) % kPage;
    const int g = e % G;
    *reinterpret_cast<uint16_t*>(out + tq3_scale_off(D, kv, t, g)) = scales[kv][t][g];
  }
}

hipError_t launch_demote_listed(const Geometry& g, const LayerTable& lt, int n_layers, const int32_t* src,
                                const int32_t* dst, int n, const int32_t* n_dev, const TableUpdate* upd,
                                hipStream_t stream) {
  if (n == 0 || n_layers == 0) return hipSuccess;
  dim3 grid(n_layers * n * g.hkv);
  const TableUpdate u = upd ? *upd : TableUpdate{nullptr, nullptr, nullptr, nullptr, nullptr};
  if (g.d == 256)
    hipLaunchKernelGGL(demote_kernel<256>, grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3,
                       g.hkv, src, dst, n_dev, u);
  else
    hipLaunchKernelGGL(demote_kernel<128>, grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3,
                       g.hkv, src, dst, n_dev, u);
  return hipGetLastError();
}

hipError_t launch_demote(const Geometry& g, const LayerTable& lt, int n_layers,
                         const int32_t* src, const int32_t* dst, int n, hipStream_t stream) {
  return launch_demote_listed(g, lt, n_layers, src, dst, n, nullptr, nullptr, stream);
}

}  // namespace mkv
