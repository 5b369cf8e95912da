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

template <int GB>
__device__ inline uint32_t lane_xor(uint32_t x) {
  return __builtin_bit_cast(uint32_t, lane_xor<GB>(__builtin_bit_cast(float, x)));
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

// ---- plain pages: the code rule -------------------------------------------
//
// The code of x against its group's scale s: B = [|x| >= 3s/2],
// D = [|x| > (B ? 5s/2 : s/2)] and N = [x < -s/2].  The magnitude
// m = [|x| > s/2] + [|x| >= 3s/2] + [|x| > 5s/2] is 2 B + D, and the code
// u = 4 + m (x >= 0) or 4 - m (x < 0; N is then m > 0) has
//   u0 = D (4 + m and 4 - m are odd together),
//   u1 = B ^ (N & D) (4 - m is 3 or 2 for m = 1, 2; 4 + m is 6 or 7 for m >= 2),
//   u2 = !N.
// A thread builds whole triples: a K thread takes one token row of the
// groups g and g + 2 that share K triples, a V thread the four tokens of one
// token quarter in half of a group (its partner lane holds the other half).

struct Thresholds {
  float t1, t2, t3;   // s/2, 3s/2, 5s/2 (exact); +inf for s = 0
};

__device__ inline Thresholds thresholds(float s) {
  const float z = s == 0.0f ? INFINITY : s;
  return {0.5f * z, 1.5f * z, 2.5f * z};
}

// Largest |decode| of 16 FP8 bytes.  With the layer scale: the largest
// fl32(|d| scl) is fl32(max |d| scl), fp32 rounding being monotone.
__device__ inline float absmax_fp8x16(const uint4 q) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[i], 1.0f, true);
    a = fmaxf(fmaxf(a, fabsf(lo[0])), fabsf(lo[1]));
    a = fmaxf(fmaxf(a, fabsf(hi[0])), fabsf(hi[1]));
  }
  return a;
}

__device__ inline uint32_t word_of(const uint4& q, int i) { return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w; }

// ---- codes from the FP8 bytes, four at a time -------------------------------
//
// With the layer scale 1, x is decode(e) exactly, and |x| grows with the
// byte's magnitude field e & 0x7f (with a scale too: see below).  Each compare of the code rule is then a
// compare of that field against a code-space threshold of the group:
// C1 = [|x| > s/2], C2 = B = [|x| >= 3s/2] and C3 = [|x| > 5s/2] hold iff
// the field exceeds T1, T2 and T3, the largest codes whose values are at
// most s/2, below 3s/2 and at most 5s/2.  The byte sum field + (0x7f - T)
// has bit 7 set iff the field exceeds T, and no byte carries into the next.
// Since C3 => C2 => C1: D = C1 ^ C2 ^ C3 and N = sign & C1, so u0 = D,
// u1 = C2 ^ (N & D) and u2 = !N, each as bit 7 of its byte.  (NaN codes are
// outside the input contract; their field, 0x7f, exceeds every threshold.)

// Largest E4M3 magnitude code whose value is at most t (t >= 0, inf
// allowed): exponent and top three mantissa bits of t in the normal range,
// floor(512 t) below 2^-6, 0x7e from 448 up.
__device__ inline uint32_t e4m3_floor_code(float t) {
  const uint32_t n = (__float_as_uint(t) >> 20) - 960u;
  const uint32_t c = t < 0x1p-6f ? (uint32_t)(t * 512.0f) : n;
  return c < 126u ? c : 126u;
}

// 0x7f - T1, 0x7f - T2, 0x7f - T3 of a group (T2 from the float just below
// 3s/2: a code's value is below 3s/2 iff it is at most that float)
struct Keys {
  uint32_t k1, k2, k3;
};

__device__ inline Keys code_keys(const Thresholds& th) {
  return {127u - e4m3_floor_code(th.t1), 127u - e4m3_floor_code(__uint_as_float(__float_as_uint(th.t2) - 1u)),
          127u - e4m3_floor_code(th.t3)};
}

// With a layer scale, x = fl32(decode(e) scl) is still monotone in the
// magnitude field, and T is the largest code c whose product fl32(value(c)
// scl) is at most t (below t for T2).  The floor code of t / scl, from an
// approximate reciprocal, is within one code of T: codes are at least 1/16
// apart relatively, the quotient and the products near a nonzero threshold
// (normal fp32 numbers) within 2^-22.  The exact products of that code and
// the next decide (code 127 decodes to NaN, which is never at most t).
template <bool STRICT>
__device__ inline uint32_t scaled_floor_code(float t, float scl, float rscl) {
  const uint32_t c = e4m3_floor_code(t * rscl);
  const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c | (c + 1u) << 8, 1.0f, false);
  const float p0 = __fmul_rn(v[0], scl), p1 = __fmul_rn(v[1], scl);
  const bool ok0 = STRICT ? p0 < t : p0 <= t, ok1 = STRICT ? p1 < t : p1 <= t;
  return ok1 ? c + 1u : ok0 ? c : c - 1u;                 // c = 0 is always ok (t > 0)
}

template <bool SCALED>
__device__ inline Keys group_keys(const Thresholds& th, float scl, float rscl) {
  if constexpr (!SCALED) return code_keys(th);
  return {127u - scaled_floor_code<false>(th.t1, scl, rscl), 127u - scaled_floor_code<true>(th.t2, scl, rscl),
          127u - scaled_floor_code<false>(th.t3, scl, rscl)};
}

// Three-input bitwise functions as one v_bitop3 each: the truth table's bit
// (a b c) (a the most significant) is the result for those input bits, so a
// is 0xf0, b is 0xcc and c is 0xaa.
template <uint32_t kTable>
__device__ inline uint32_t bitop3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, kTable);
}
constexpr uint32_t kXor3 = (0xf0 ^ 0xcc ^ 0xaa) & 0xff;                     // a ^ b ^ c
constexpr uint32_t kXorAnd = (0xf0 ^ (0xcc & 0xaa)) & 0xff;                 // a ^ (b & c)
constexpr uint32_t kSelA = ((0xf0 & 0xaa) | (0xcc & ~0xaa)) & 0xff;         // c ? a : b, bit by bit
constexpr uint32_t kSelNotA = ((~0xf0 & 0xaa) | (0xcc & ~0xaa)) & 0xff;     // c ? ~a : b
constexpr uint32_t kSelBNotA = ((0xcc & 0xaa) | (~0xf0 & ~0xaa)) & 0xff;    // c ? b : ~a

// Byte 0 of k in all four bytes (v_perm: selector 0 picks byte 0 of the
// second operand)
__device__ inline uint32_t bytes4(uint32_t k) { return __builtin_amdgcn_perm(0u, k, 0u); }

// Bit 7 of each byte: u0, u1 and N of that byte's code (the other bits are
// not used); k1..k3 hold each byte's keys
struct Planes {
  uint32_t u0, u1, n;
};

__device__ inline Planes code_planes(uint32_t x, uint32_t k1, uint32_t k2, uint32_t k3) {
  const uint32_t a = x & 0x7f7f7f7fu;
  const uint32_t s1 = a + k1, s2 = a + k2, s3 = a + k3;
  const uint32_t d = bitop3<kXor3>(s1, s2, s3);
  const uint32_t n = x & s1;
  return {d, bitop3<kXorAnd>(s2, n, d), n};
}

// Bits 2..7 of byte i: the code of byte i of l (bits 2..4) and of h (5..7)
__device__ inline uint32_t pair_fields(const Planes& l, const Planes& h) {
  uint32_t f = bitop3<kSelNotA>(h.n, h.u1 >> 1, 0x80808080u);   // !N of h at bit 7, u1 at 6
  f = bitop3<kSelA>(f, h.u0 >> 2, 0xc0c0c0c0u);                  // u0 of h at 5
  f = bitop3<kSelBNotA>(l.n >> 3, f, 0xe0e0e0e0u);               // !N of l at 4
  f = bitop3<kSelA>(f, l.u1 >> 4, 0xf0f0f0f0u);                  // u1 of l at 3
  return bitop3<kSelA>(f, l.u0 >> 5, 0xf8f8f8f8u);               // u0 of l at 2
}

// The four 6-bit fields at bits 8 i + 2 .. 8 i + 7 -> bits 6 i .. 6 i + 5
// (a triple word: slot 2 i the code of byte i of l, slot 2 i + 1 of h)
__device__ inline uint32_t compact_fields(uint32_t f) {
  const uint32_t y = bitop3<kSelA>(f >> 2, f >> 4, 0x003f003fu);
  return bitop3<kSelA>(y, y >> 4, 0x00000fffu);
}

// Workgroup of 128 threads: wave 0 builds the K triples, wave 1 the V
// triples, of PH (layer, page, KV head) items (8 G threads each per wave).
// SCALED: some layer of the launch has a k_scale or v_scale other than 1
// (every value is then multiplied by its layer's scale; by 1 it is exact).
// A thread codes 64 FP8 bytes: K, token row t of groups g (gg = g mod 4 in
// {0, 1}) and g + 2; V, tokens 4 j .. 4 j + 3 of channels 32 g + 16 hh .. + 15.
// It keeps them as bytes, which keeps the registers few and the waves per
// SIMD many: each value is converted once for the group's maximum, and the
// codes come from the bytes, four at a time, in code space.
template <int D, bool SCALED>
__global__ void __launch_bounds__(128) demote_plain_kernel(
    LayerTable lt, int n, int n_fp8, int n_tq3, int hkv, const int32_t* __restrict__ src,
    const int32_t* __restrict__ dst, const int32_t* __restrict__ n_dev, TableUpdate upd, int n_items) {
  constexpr int G = D / 32;
  constexpr int PH = 64 / (8 * G);                   // items per workgroup: 1 at d = 256, 2 at d = 128
  constexpr int NTRI = 4 * D;
  __shared__ __align__(16) uint32_t tw[PH][NTRI];    // one word per triple (24 bits used)
  __shared__ __align__(16) uint16_t sc[PH][D];       // the 2D scale bytes, in block order
  __shared__ uint8_t* outp[PH];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ph = lane / (8 * G), r8 = lane % (8 * G);

  const int item = blockIdx.x * PH + ph;
  bool valid = item < n_items;
  int layer = 0, page = 0, h = 0, s_id = -1, d_id = -1;
  if (valid) {
    layer = item / (n * hkv);
    const int rest = item - layer * n * hkv;
    page = rest / hkv;
    h = rest - page * hkv;
    if (n_dev && page >= *n_dev) valid = false;
  }
  if (valid) {
    s_id = src[page];
    d_id = dst[page];
    valid = !(s_id < 0 || s_id >= n_fp8 || d_id < n_fp8 || d_id >= n_fp8 + n_tq3);
  }
  uint8_t* out = nullptr;
  const uint8_t* in = nullptr;
  if (valid) {
    in = lt.fp8[layer] + (size_t)s_id * fp8_page_bytes(hkv, D) + (size_t)h * 2 * kPage * D;
    out = lt.tq3[layer] + (size_t)(d_id - n_fp8) * tq3_page_bytes(hkv, D) + (size_t)h * tq3_head_bytes(D);
  }
  if (wave == 0 && r8 == 0) {
    outp[ph] = out;
    if (valid && upd.bt_pages && layer == 0 && h == 0) {
      upd.bt_pages[upd.entry[page]] = d_id;
      upd.tier[d_id] = kTierStale;
      upd.tier[s_id] = kTierFree;
      upd.fp8_free[*upd.push_base + page] = s_id;
    }
  }

  if (valid && wave == 0) {
    const int t = r8 / (G / 2), pr = r8 % (G / 2);
    const int g = 4 * (pr >> 1) + (pr & 1);
    const float scl = lt.k_scale[layer];
    const uint4* row = reinterpret_cast<const uint4*>(in + t * D);
    const uint4 q[4] = {row[2 * g], row[2 * g + 1], row[2 * g + 4], row[2 * g + 5]};   // groups g, g + 2
    const float al = fmaxf(absmax_fp8x16(q[0]), absmax_fp8x16(q[1]));
    const float ah = fmaxf(absmax_fp8x16(q[2]), absmax_fp8x16(q[3]));
    const uint16_t sbl = tq3_scale_bits(SCALED ? __fmul_rn(al, scl) : al);
    const uint16_t sbh = tq3_scale_bits(SCALED ? __fmul_rn(ah, scl) : ah);
    sc[ph][(tq3_scale_off(D, 0, t, g) - 12 * D) / 2] = sbl;
    sc[ph][(tq3_scale_off(D, 0, t, g + 2) - 12 * D) / 2] = sbh;
    const Thresholds thl = thresholds(half_bits_to_float(sbl)), thh = thresholds(half_bits_to_float(sbh));
    // channel 8 j + e of the pair sits in triple j G + 4 (g / 4) + 2 gg + e / 4
    // of the row, slot 2 (e % 4) (group g) or 2 (e % 4) + 1 (group g + 2);
    // channels 8 j + 4 e4 .. + 3 of a group are its dword 2 j + e4
    const float rscl = __builtin_amdgcn_rcpf(scl);
    const Keys kl = group_keys<SCALED>(thl, scl, rscl), kh = group_keys<SCALED>(thh, scl, rscl);
    const uint32_t l1 = bytes4(kl.k1), l2 = bytes4(kl.k2), l3 = bytes4(kl.k3);
    const uint32_t h1 = bytes4(kh.k1), h2 = bytes4(kh.k2), h3 = bytes4(kh.k3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t w2[2];
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const int k = 2 * j + e4;
        const uint32_t wl = word_of(q[k >> 2], k & 3), wh = word_of(q[2 + (k >> 2)], k & 3);
        w2[e4] = compact_fields(pair_fields(code_planes(wl, l1, l2, l3), code_planes(wh, h1, h2, h3)));
      }
      *reinterpret_cast<uint2*>(&tw[ph][t * (D / 8) + j * G + 4 * (g >> 2) + 2 * (g & 3)]) = make_uint2(w2[0], w2[1]);
    }
  } else if (valid) {
    const int j = r8 / (2 * G), g = (r8 >> 1) % G, hh = r8 & 1;
    const float scl = lt.v_scale[layer];
    uint4 q[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) q[r] = *reinterpret_cast<const uint4*>(in + (kPage + 4 * j + r) * D + 32 * g + 16 * hh);
    // channel pair (a, a + 1), a = 32 g + 16 hh + 2 pc, is triple
    // (16 j + n) G + p of the V codes; the 8 pairs are consecutive triples;
    // slot 2 r + ci holds (channel a + ci, token 4 j + r)
    const int tb = 2 * D + (j * 16 + (32 * g + 16 * hh) / (D / 16)) * G;
    uint32_t w8[8];
    // The two lanes of a group each hold half of the four tokens' rows:
    // lane hh forms the scales and keys of tokens 2 hh and 2 hh + 1 from
    // both halves' maxima, and the lanes swap keys.  Byte r of a key is
    // token 4 j + r's.
    float a[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = absmax_fp8x16(q[r]);
    const float am0 = fmaxf(hh ? a[2] : a[0], lane_xor<1>(hh ? a[0] : a[2]));
    const float am1 = fmaxf(hh ? a[3] : a[1], lane_xor<1>(hh ? a[1] : a[3]));
    const uint16_t sb0 = tq3_scale_bits(SCALED ? __fmul_rn(am0, scl) : am0);
    const uint16_t sb1 = tq3_scale_bits(SCALED ? __fmul_rn(am1, scl) : am1);
    sc[ph][(tq3_scale_off(D, 1, 4 * j + 2 * hh, g) - 12 * D) / 2] = sb0;
    sc[ph][(tq3_scale_off(D, 1, 4 * j + 2 * hh + 1, g) - 12 * D) / 2] = sb1;
    const float rscl = __builtin_amdgcn_rcpf(scl);
    const Keys c0 = group_keys<SCALED>(thresholds(half_bits_to_float(sb0)), scl, rscl);
    const Keys c1 = group_keys<SCALED>(thresholds(half_bits_to_float(sb1)), scl, rscl);
    const int sh = 16 * hh;
    uint32_t k1 = (c0.k1 | c1.k1 << 8) << sh, k2 = (c0.k2 | c1.k2 << 8) << sh, k3 = (c0.k3 | c1.k3 << 8) << sh;
    k1 |= lane_xor<1>(k1);
    k2 |= lane_xor<1>(k2);
    k3 |= lane_xor<1>(k3);
    // the bytes of dword kq of the four token rows, regrouped so that byte
    // r is token r's: bytes 0 and 1 of each row make word 2 kq, bytes 2
    // and 3 word 2 kq + 1
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      const uint32_t x0 = word_of(q[0], kq), x1 = word_of(q[1], kq), x2 = word_of(q[2], kq), x3 = word_of(q[3], kq);
      const uint32_t e01 = __builtin_amdgcn_perm(x1, x0, 0x05010400u), e23 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);
      const uint32_t f01 = __builtin_amdgcn_perm(x1, x0, 0x07030602u), f23 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);
      w8[2 * kq] = compact_fields(pair_fields(code_planes(__builtin_amdgcn_perm(e23, e01, 0x05040100u), k1, k2, k3),
                                              code_planes(__builtin_amdgcn_perm(e23, e01, 0x07060302u), k1, k2, k3)));
      w8[2 * kq + 1] = compact_fields(pair_fields(code_planes(__builtin_amdgcn_perm(f23, f01, 0x05040100u), k1, k2, k3),
                                                  code_planes(__builtin_amdgcn_perm(f23, f01, 0x07060302u), k1, k2, k3)));
    }
    uint4* dstw = reinterpret_cast<uint4*>(&tw[ph][tb]);
    dstw[0] = make_uint4(w8[0], w8[1], w8[2], w8[3]);
    dstw[1] = make_uint4(w8[4], w8[5], w8[6], w8[7]);
  }
  __syncthreads();

  // four triples = 12 bytes per store; then the scales as 16-byte chunks
  for (int e = threadIdx.x; e < PH * (NTRI / 4); e += 128) {
    const int p = e / (NTRI / 4), tau = e - p * (NTRI / 4);
    uint8_t* o = outp[p];
    if (!o) continue;
    const uint4 w = reinterpret_cast<const uint4*>(tw[p])[tau];
    const u3v b3 = {w.x | (w.y << 24), (w.y >> 8) | (w.z << 16), (w.z >> 16) | (w.w << 8)};
    *reinterpret_cast<u3v*>(o + 12 * tau) = b3;
  }
  for (int e = threadIdx.x; e < PH * (2 * D / 16); e += 128) {
    const int p = e / (2 * D / 16), c = e - p * (2 * D / 16);
    uint8_t* o = outp[p];
    if (!o) continue;
    reinterpret_cast<uint4*>(o + 12 * D)[c] = reinterpret_cast<const uint4*>(sc[p])[c];
  }
}

hipError_t launch_demote_listed(const Geometry& g, const LayerTable& lt, int n_layers, const int32_t* src,
                                const int32_t* dst, int n, const int32_t* n_dev, const TableUpdate* upd,
                                hipStream_t stream) {
  if (n == 0 || n_layers == 0) return hipSuccess;
  dim3 grid(n_layers * n * g.hkv);
  const TableUpdate u = upd ? *upd : TableUpdate{nullptr, nullptr, nullptr, nullptr, nullptr};
  // layers with rotated TQ3 pages take the instance with the rotation; plain
  // pools the mask-based one
  const int items = n_layers * n * g.hkv;
  if (!lt.any_signs) {
    bool scaled = false;
    for (int l = 0; l < n_layers; ++l) scaled = scaled || lt.k_scale[l] != 1.0f || lt.v_scale[l] != 1.0f;
    const int wgs = g.d == 256 ? items : (items + 1) / 2;
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(wgs), dim3(128), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src, dst, n_dev, u,
                         items);
    };
    if (g.d == 256)
      scaled ? go(demote_plain_kernel<256, true>) : go(demote_plain_kernel<256, false>);
    else
      scaled ? go(demote_plain_kernel<128, true>) : go(demote_plain_kernel<128, false>);
  } else if (g.d == 256) {
    hipLaunchKernelGGL((demote_kernel<256, true>), grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src, dst,
                       n_dev, u);
  } else {
    hipLaunchKernelGGL((demote_kernel<128, true>), grid, dim3(256), 0, stream, lt, n, g.n_fp8, g.n_tq3, g.hkv, src, dst,
                       n_dev, u);
  }
  return hipGetLastError();
}

hipError_t launch_demote(const Geometry& g, const LayerTable& lt, int n_layers,
                         const int32_t* src, const int32_t* dst, int n, hipStream_t stream) {
  return launch_demote_listed(g, lt, n_layers, src, dst, n, nullptr, nullptr, stream);
}

}  // namespace mkv
