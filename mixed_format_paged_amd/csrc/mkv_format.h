// mkv_format.h -- device-side page formats for the mixed FP8 / TQ3 cache.
//
// Minima-KV (arXiv 2608.23834, page 1, Abstract) stores Recent and Anchor
// pages as FP8 and stale pages as packed 3-bit TQ3.  The pages fix neither
// the FP8 variant nor any TQ3 detail; this file implements the readings this
// library documents in include/mkv.h:
//
//  FP8: OCP E4M3FN, round-to-nearest-even, saturating to +-448.
//  FP8 page: [kv head][K, V][16 tokens][head_dim] bytes.
//  TQ3: per token, per KV head, per 32 channels: fp16 scale
//       s = fp16_RNE(fl32(absmax / 3)), codes u = q + 4 with q the nearest
//       integer to x / s (ties to even) clamped to [-3, 3]; 8 codes per
//       3 bytes, slot k at bits [3k, 3k+3) of the little-endian 24-bit word.
//  TQ3 head block (14 * d bytes, G = d / 32, a multiple of 4):
//       [0, 6d)    K codes: token row t at t * 3d/8; in it, quarter j
//                  (channels 8j .. 8j + 7 of every group) at 3 j G, in blocks
//                  of 4 triples (12 bytes), block b for groups 4b .. 4b + 3.
//                  Read as 16 six-bit fields, field f of a block holds
//                  channel 8j + f % 8 of group 4b + f / 8 in its low 3 bits
//                  and of group 4b + 2 + f / 8 in its high 3 bits: channel
//                  32 g + 8 j + e, gg = g % 4, is triple 4 (g / 4) + 2 (gg % 2)
//                  + e / 4 of the quarter, slot 2 (e % 4) + gg / 2.
//       [6d, 12d)  V codes: triple at 3 * ((j * 16 + n) * G + p) holds tokens
//                  4j..4j+3 of channels a = n * d/16 + 2p and b = a + 1, slot
//                  2r = (a, 4j + r), slot 2r + 1 = (b, 4j + r).
//       [12d, 13d) K scales, [13d, 14d) V scales: fp16 of (t = 4j + r, g) at
//                  element (j * G + g) * 4 + r.
//  Why: one GPU lane's triples are adjacent (one aligned vector load), and a
//  block of 4 triples read as 6-bit fields decodes in two FP6 conversions
//  (low codes, then high codes) into operands the matrix cores take as they
//  are: 8 channels of one K group per 4 registers, and V codes of one channel
//  for 2 consecutive tokens per register (see mkv_partial_mfma.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace mkv {

constexpr int kPage = 16;
constexpr int kGroup = 32;
constexpr int kTierRecent = 0, kTierAnchor = 1, kTierStale = 2, kTierFree = 0xFF;

__host__ __device__ inline int fp8_page_bytes(int hkv, int d) { return hkv * 2 * kPage * d; }
__host__ __device__ inline int tq3_head_bytes(int d) { return 14 * d; }
__host__ __device__ inline int tq3_page_bytes(int hkv, int d) { return hkv * 14 * d; }

// ---- E4M3FN ---------------------------------------------------------------

// Encode an fp32 value (already divided by the layer scale).  Integer-exact
// round-to-nearest-even; |y| > 448 saturates; NaN -> 0x7F with sign.
__device__ inline uint32_t e4m3_encode(float y) {
  uint32_t b = __float_as_uint(y);
  uint32_t sign = (b >> 24) & 0x80u;
  uint32_t ab = b & 0x7fffffffu;
  if (ab > 0x7f800000u) return 0x7fu | sign;          // NaN
  if (ab > 0x43e00000u) return 0x7eu | sign;          // > 448 (incl. inf): saturate
  int e = (int)(ab >> 23) - 127;
  if (e >= -6) {                                      // normal E4M3 range
    uint32_t m = ab & 0x7fffffu;
    uint32_t q = m >> 20;
    uint32_t rem = m & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q++;
    return (((uint32_t)(e + 7) << 3) + q) | sign;     // q == 8 carries into the exponent
  }
  // subnormal E4M3 range: value = m * 2^-9; scaling by 2^9 is exact, rint is RNE
  float t = __uint_as_float(ab) * 512.0f;
  return (uint32_t)__builtin_rintf(t) | sign;          // 8 -> 0x08, the smallest normal
}

// Decode one code to fp32 (exact).  Codes 0x7F/0xFF are never produced.
__device__ inline float e4m3_decode(uint32_t c) {
  uint32_t s = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 0xfu;
  uint32_t m = c & 7u;
  float v = (e == 0) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(v) | s);
}

// ---- TQ3 ------------------------------------------------------------------

// fl32(a / 3) for finite a: the product with fl32(1/3), corrected by its
// exact remainder (one fma) and a second fma.  Checked against IEEE fp32
// division for every finite non-negative fp32 a; a = inf gives NaN.
__device__ inline float div3_rn(float a) {
  constexpr float c = 0x1.555556p-2f;                  // fl32(1/3)
  const float q = a * c;
  return fmaf(fmaf(-3.0f, q, a), c, q);
}

// s = fp16_RNE(fl32(a / 3)), saturating at 65504.  Returned as fp16 bits.
__device__ inline uint16_t tq3_scale_bits(float absmax) {
  float r = div3_rn(absmax);
  __half h = __float2half_rn(r);
  uint16_t bits = __half_as_ushort(h);
  if ((bits & 0x7c00u) == 0x7c00u) bits = 0x7bffu;     // inf (and the NaN of a = inf) -> 65504
  return bits;
}

// Signed code in [-3, 3] via exact fp32 thresholds (0.5 s, 1.5 s, 2.5 s are
// exact because s has at most 11 significant bits).
__device__ inline int tq3_code(float x, float s) {
  if (s == 0.0f) return 0;
  float ax = fabsf(x);
  int m = (ax > 0.5f * s) + (ax >= 1.5f * s) + (ax > 2.5f * s);
  return (__float_as_uint(x) & 0x80000000u) ? -m : m;
}

__device__ inline float half_bits_to_float(uint16_t b) { return __half2float(__ushort_as_half(b)); }

// Byte offset of the triple holding K (t, c) inside a head block, and its slot.
__host__ __device__ inline int tq3_k_triple(int d, int t, int c, int* slot) {
  int G = d >> 5;
  int g = c >> 5, j = (c >> 3) & 3, e = c & 7, gg = g & 3;
  *slot = 2 * (e & 3) + (gg >> 1);
  return t * (3 * d / 8) + 3 * (j * G + 4 * (g >> 2) + 2 * (gg & 1) + (e >> 2));
}

// V slot of (channel-in-pair ci, token-in-quarter r).
__host__ __device__ inline int tq3_v_slot(int ci, int r) { return 2 * r + ci; }

__host__ __device__ inline int tq3_v_triple(int d, int t, int c, int* slot) {
  int G = d >> 5;
  int per = d >> 4;                                    // channels per slice n
  int j = t >> 2, r = t & 3;
  int n = c / per, w = c - n * per;
  int p = w >> 1, ci = w & 1;
  *slot = tq3_v_slot(ci, r);
  return 6 * d + 3 * ((j * 16 + n) * G + p);
}

__host__ __device__ inline int tq3_scale_off(int d, int kv, int t, int g) {
  int G = d >> 5;
  return 12 * d + kv * d + 2 * (((t >> 2) * G + g) * 4 + (t & 3));
}

}  // namespace mkv
