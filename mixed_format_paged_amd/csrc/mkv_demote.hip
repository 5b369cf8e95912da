// mkv_demote.hip -- FP8 -> TQ3 page demotion (the pack).
//
// Older non-anchor pages move to packed TQ3 (arXiv 2608.23834, page 1,
// Abstract).  One workgroup per (layer, page, KV head):
//   phase 1: one thread per (K/V, token, 32-channel group) converts its 32 FP8
//            bytes (x = fl32(decode(e) * scale), decode exact through the
//            hardware E4M3 conversion), takes the absmax, forms the fp16
//            scale s = fp16_RNE(fl32(a / 3)) and the codes u = q + 4 (q the
//            nearest integer to x / s, ties to even, from exact fp32
//            thresholds).  A K group's 32 codes are exactly four triples of
//            its token row, packed in registers and stored as triple words;
//            a V group's codes are OR-ed, two channels at a time, into the
//            triple words of their (token quarter, channel pair).
//   phase 2: each thread packs four consecutive triple words into the 12
//            bytes of the head block and stores them with one 12-byte store;
//            the scales follow as 16-byte chunks.
// The lifecycle's variant takes its page count from device memory and also
// rewrites each demoted page's block-table entry, tier bytes and free-stack
// slot (one workgroup per page does it; nothing else in the launch reads
// them, and the FP8 slot it frees is only reused by a later launch).
#include <type_traits>

#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

typedef uint32_t u3v __attribute__((ext_vector_type(3)));

// x of the lane whose index differs in bit gb (1, 2 or 4) within its group of
// 8 lanes, by DPP moves (no LDS): quad permutes for xor 1 and 2; xor 4 is a
// quad permute (xor 3) then a half-row mirror (xor 7).
template <int GB>
__device__ inline float lane_xor(float x) {
  const int v = __builtin_bit_cast(int, x);
  if constexpr (GB == 1) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xf, 0xf, false));
  if constexpr (GB == 2) return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xf, 0xf, false));
  const int t = __builtin_amdgcn_update_dpp(0, v, 0x1B, 0xf, 0xf, false);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, t, 0x141, 0xf, 0xf, false));
}

template <int D, bool ROT = false>
__global__ void __launch_bounds__(256) demote_kernel(
    LayerTable lt, int n, int n_fp8, int n_tq3, int hkv, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, const int32_t* __restrict__ n_dev, TableUpdate upd) {
  constexpr int G = D / 32;
  constexpr int NTRI = 4 * D;                        // triples of a head block: 2D of K, 2D of V
  __shared__ __align__(16) uint32_t tw[NTRI];        // one word per triple (24 bits used)
  __shared__ __align__(16) uint16_t sc[D];           // the 2D scale bytes, in block order
  const int layer = blockIdx.x / (n * hkv);
  const int rest = blockIdx.x - layer * n * hkv;
  const int page = rest / hkv;
  const int h = rest - page * hkv;
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
  const uint8_t* __restrict__ fp8_slab = lt.fp8[layer];
  uint8_t* __restrict__ tq3_slab = lt.tq3[layer];
  const float k_scale = lt.k_scale[layer], v_scale = lt.v_scale[layer];
  const uint8_t* in = fp8_slab + (size_t)s_id * fp8_page_bytes(hkv, D) + (size_t)h * 2 * kPage * D;
  uint8_t* out = tq3_slab + (size_t)(d_id - n_fp8) * tq3_page_bytes(hkv, D) + (size_t)h * tq3_head_bytes(D);

  for (int e = threadIdx.x; e < NTRI / 4; e += blockDim.x) reinterpret_cast<uint4*>(tw)[e] = make_uint4(0, 0, 0, 0);
  __syncthreads();

  for (int grp = threadIdx.x; grp < 2 * kPage * G; grp += blockDim.x) {
    const int kv = grp / (kPage * G);
    const int t = (grp / G) % kPage;
    const int g = grp % G;
    const float scl = kv ? v_scale : k_scale;
    const uint4* row = reinterpret_cast<const uint4*>(in + (kv * kPage + t) * D + g * 32);
    const uint4 r0 = row[0], r1 = row[1];
    const uint32_t words[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    float x[32];
    float a = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(words[w], 1.0f, false);   // bytes 0, 1
      const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(words[w], 1.0f, true);    // bytes 2, 3
      x[4 * w] = lo[0];
      x[4 * w + 1] = lo[1];
      x[4 * w + 2] = hi[0];
      x[4 * w + 3] = hi[1];
    }
    if (scl != 1.0f) {                               // uniform; x * 1 is x exactly
#pragma unroll
      for (int c = 0; c < 32; ++c) x[c] = __fmul_rn(x[c], scl);
    }
    const int8_t* const sg = ROT ? lt.signs[layer] : nullptr;
    if (ROT && sg) {                                   // rotated TQ3 (uniform per launch item)
      // y = c H (signs . x) over the row's d channels, in the stage order of
      // the format: channel bits 0..4 within the thread's group, then the
      // group bits across the threads of the row (lanes differing in g)
      const uint4 s0 = *reinterpret_cast<const uint4*>(sg + 32 * g), s1 = *reinterpret_cast<const uint4*>(sg + 32 * g + 16);
      const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if ((int8_t)((sw[c >> 2] >> (8 * (c & 3))) & 0xffu) < 0) x[c] = -x[c];
#pragma unroll
      for (int hs = 1; hs < 32; hs <<= 1) {
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          if (c & hs) continue;
          const float a = x[c], b2 = x[c + hs];
          x[c] = a + b2;
          x[c + hs] = a - b2;
        }
      }
      // group bits: the partner thread is lane ^ gb (the row's G threads are
      // consecutive lanes, G = 4 or 8)
      auto cross = [&](auto gbc) {
        constexpr int gb = decltype(gbc)::value;
        const bool hi = (g & gb) != 0;
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          const float p = lane_xor<gb>(x[c]);
          x[c] = hi ? p - x[c] : x[c] + p;             // (a + b, a - b) with a from the lower channel
        }
      };
      cross(std::integral_constant<int, 1>{});
      cross(std::integral_constant<int, 2>{});
      if constexpr (G == 8) cross(std::integral_constant<int, 4>{});
      static_assert(G == 4 || G == 8, "row of 4 or 8 groups");
      const float cs = D == 256 ? 0.0625f : 0.125f;    // c = 2^-floor(log2(d) / 2), exact
#pragma unroll
      for (int c = 0; c < 32; ++c) x[c] *= cs;
    }
#pragma unroll
    for (int c = 0; c < 32; ++c) a = fmaxf(a, fabsf(x[c]));
    const uint16_t sb = tq3_scale_bits(a);
    const float s = half_bits_to_float(sb);
    sc[(tq3_scale_off(D, kv, t, g) - 12 * D) / 2] = sb;
    // |q| counts the exact fp32 thresholds 0.5 s, 1.5 s (inclusive: ties to
    // even) and 2.5 s below |x|; s == 0 gives q = 0 through infinite thresholds
    const bool zero = s == 0.0f;
    const float t1 = zero ? INFINITY : 0.5f * s, t2 = zero ? INFINITY : 1.5f * s, t3 = zero ? INFINITY : 2.5f * s;
    uint32_t u[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const float ax = fabsf(x[c]);
      const uint32_t m = (uint32_t)(ax > t1) + (uint32_t)(ax >= t2) + (uint32_t)(ax > t3);
      u[c] = (__float_as_uint(x[c]) >> 31) ? 4u - m : 4u + m;
    }
    if (kv == 0) {
      // K: channel 8j + e of the group sits in row t, quarter j, triple
      // 4 (g / 4) + 2 (gg % 2) + e / 4 at slot 2 (e % 4) + gg / 2 (gg = g % 4);
      // groups gg and gg ^ 2 share those triples (even and odd slots), so OR them in
      const int gg = g & 3, sh = 3 * (gg >> 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w = 0;
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) w |= u[8 * j + 4 * hh + e4] << (6 * e4 + sh);
          atomicOr(&tw[t * (D / 8) + j * G + 4 * (g >> 2) + 2 * (gg & 1) + hh], w);
        }
      }
    } else {
      // V: channels (a, a + 1) of token t sit in triple (t / 4, n, p) at slots
      // of (channel in pair, t % 4); four tokens share a triple, so OR them in
      const int r = t & 3;
      const int s0 = 3 * tq3_v_slot(0, r), s1 = 3 * tq3_v_slot(1, r);
#pragma unroll
      for (int pc = 0; pc < 16; ++pc) {
        const int c = g * 32 + 2 * pc;               // channel a of the pair
        const int n = c / (D / 16), p = (c % (D / 16)) / 2;
        atomicOr(&tw[2 * D + ((t >> 2) * 16 + n) * G + p], (u[2 * pc] << s0) | (u[2 * pc + 1] << s1));
      }
    }
  }
  __syncthreads();

  // four triples = 12 bytes per thread, one 12-byte store each
  for (int tau = threadIdx.x; tau < NTRI / 4; tau += blockDim.x) {
    const uint4 q = reinterpret_cast<const uint4*>(tw)[tau];
    const u3v w = {q.x | (q.y << 24), (q.y >> 8) | (q.z << 16), (q.z >> 16) | (q.w << 8)};
    *reinterpret_cast<u3v*>(out + 12 * tau) = w;
  }
  for (int e = threadIdx.x; e < 2 * D / 16; e += blockDim.x)
    reinterpret_cast<uint4*>(out + 12 * D)[e] = reinterpret_cast<const uint4*>(sc)[e];
}

hipError_t launch_demote_listed(const Geometry& g, const LayerTable& lt, int n_layers, const int32_t* src,
                                const int32_t* dst, int n, const int32_t* n_dev, const TableUpdate* upd,
                                hipStream_t stream) {
  if (n == 0 || n_layers == 0) return hipSuccess;
  dim3 grid(n_layers * n * g.hkv);
  const TableUpdate u = upd ? *upd : TableUpdate{nullptr, nullptr, nullptr, nullptr, nullptr};
  // layers with rotated TQ3 pages take the instance with the rotation
  if (g.d == 256) {
    if (lt.any_signs)
      hipLaunchKernelGGL((demote_kernel<256, true>), grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src, dst,
                         n_dev, u);
    else
      hipLaunchKernelGGL((demote_kernel<256, false>), grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src,
                         dst, n_dev, u);
  } else {
    if (lt.any_signs)
      hipLaunchKernelGGL((demote_kernel<128, true>), grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src, dst,
                         n_dev, u);
    else
      hipLaunchKernelGGL((demote_kernel<128, false>), grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src,
                         dst, n_dev, u);
  }
  return hipGetLastError();
}

hipError_t launch_demote(const Geometry& g, const LayerTable& lt, int n_layers,
                         const int32_t* src, const int32_t* dst, int n, hipStream_t stream) {
  return launch_demote_listed(g, lt, n_layers, src, dst, n, nullptr, nullptr, stream);
}

}  // namespace mkv
