// mkv_partial_mfma.hip -- matrix-core partial-attention kernels for gfx950.
//
// Minima-KV's format-specific kernels compute partial attention states over
// the pages of one format, read in place without a dense shadow (arXiv
// 2608.23834, page 1, Abstract).  Here both formats run on the CDNA4 matrix
// cores with fp32 accumulation:
//
//  * Work item = (layer, chunk of pages, KV head); a workgroup of 4 waves
//    takes one item, wave w the pages w, w+4, ...; each KV page is read once
//    for the whole GQA group.  The 4 wave states are merged in LDS and one
//    partial (m, l, acc) per item is written.
//  * Scores S^T = K Q^T with v_mfma_f32_16x16x32_f16: A = 16 tokens x 32
//    channels of K, B = 32 channels x 16 query rows.  Query rows 0..G-1 hold
//    fp16(q) and rows 8..8+G-1 the fp16 remainder q - fp16(q), so one DPP
//    row-rotate by 8 adds the two halves (q carried to ~22 bits).  For TQ3
//    each MFMA covers exactly one 32-channel scale group and the fp32 group
//    scale multiplies its result; codes enter the MFMA as exact fp16 (u - 4).
//  * Online softmax in log2 units with a lazy rescale: the running max moves
//    only when a page's max exceeds it by more than 8 (p <= 2^8, safe in fp16).
//  * P V with v_mfma_f32_16x16x16_f16: A = P (rows 0..G-1 fp16(p), rows
//    8..8+G-1 the remainder), B = 16 tokens x 16 channels of V.  TQ3 V is
//    (u - 4) * s split into an exact fp16 pair hi + lo (two MFMAs); FP8 V is
//    exact in fp16 (one MFMA).
//  Lane maps follow the byte layout in mkv_format.h: a TQ3 lane's triples
//  arrive in one aligned chunk, and each triple becomes four fp16 pairs with
//  one mask-and-or and one packed fma per pair.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr float kRescale = 8.0f;        // log2 units

__device__ inline h2 u2h(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ inline uint32_t h2u(h2 h) { return __builtin_bit_cast(uint32_t, h); }
__device__ inline h2 mkh2(float a, float b) { return h2{(_Float16)a, (_Float16)b}; }

__device__ inline float dpp_ror8(float x) {             // lane l <- lane (l ^ 8) within each 16-lane row
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
}

// Byte `o` of a little-endian array of dwords, as the start of a triple: the
// three dwords X = [b0 b1 b2 .], Y = [b1 b2 b0 b1], W = [b1 b2 b1 b2].
template <int NW>
__device__ inline void triple_words(const uint32_t (&c)[NW], int o, uint32_t& X, uint32_t& Y, uint32_t& W) {
  const int i = o >> 2, s = o & 3;
  const uint32_t lo = c[i];
  const uint32_t hi = (s + 2 >= 4) ? c[i + 1] : lo;
  const uint32_t b0 = s, b1 = s + 1, b2 = s + 2;
  X = __builtin_amdgcn_perm(hi, lo, b0 | (b1 << 8) | (b2 << 16) | (b2 << 24));
  Y = __builtin_amdgcn_perm(hi, lo, b1 | (b2 << 8) | (b0 << 16) | (b1 << 24));
  W = __builtin_amdgcn_perm(hi, lo, b1 | (b2 << 8) | (b1 << 16) | (b2 << 24));
}

// One triple -> four fp16 pairs of (u - 4):
//   r[0] = (slot0, slot6)  r[1] = (slot1, slot7)  r[2] = (slot3, slot2)  r[3] = (slot4, slot5)
// Each code is dropped into the mantissa of fp16 1024.0 at bit offset j
// (value 1024 + u 2^j) and one packed fma maps it exactly to u - 4.
__device__ inline void decode_triple(uint32_t X, uint32_t Y, uint32_t W, h2 (&r)[4]) {
  const uint32_t one024 = 0x64006400u;
  r[0] = __builtin_elementwise_fma(u2h((X & 0x001C0007u) | one024), mkh2(1.0f, 0.25f), mkh2(-1028.0f, -260.0f));
  r[1] = __builtin_elementwise_fma(u2h((X & 0x00E00038u) | one024), mkh2(0.125f, 0.03125f), mkh2(-132.0f, -36.0f));
  r[2] = __builtin_elementwise_fma(u2h((Y & 0x01C0000Eu) | one024), mkh2(0.5f, 0.015625f), mkh2(-516.0f, -20.0f));
  r[3] = __builtin_elementwise_fma(u2h((W & 0x03800070u) | one024), mkh2(0.0625f, 0.0078125f), mkh2(-68.0f, -12.0f));
}

// Per-lane page data.
template <bool TQ3, int D>
struct PageData;

template <int D>
struct PageData<true, D> {
  static constexpr int G = D / 32;
  static constexpr int NW = 3 * G / 4;     // dwords of a lane's code chunk
  uint32_t kc[NW], vc[NW];                 // K / V code chunks
  uint32_t ks[2 * G];                      // K scales of tokens 4j..4j+3, all groups
  uint32_t vs[2];                          // V scales of tokens 4j..4j+3, the lane's group

  __device__ inline void load(const uint8_t* __restrict__ blk, int lane) {
    const int t = lane & 15, j = lane >> 4;
    const uint8_t* kp = blk + (4 * t + j) * (3 * G);
    const uint8_t* vp = blk + 6 * D + lane * (3 * G);
    if constexpr (D == 256) {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const uint2 a = *reinterpret_cast<const uint2*>(kp + 8 * i);
        const uint2 b = *reinterpret_cast<const uint2*>(vp + 8 * i);
        kc[2 * i] = a.x; kc[2 * i + 1] = a.y;
        vc[2 * i] = b.x; vc[2 * i + 1] = b.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        kc[i] = reinterpret_cast<const uint32_t*>(kp)[i];
        vc[i] = reinterpret_cast<const uint32_t*>(vp)[i];
      }
    }
    const uint4* ksp = reinterpret_cast<const uint4*>(blk + 12 * D + j * 8 * G);
#pragma unroll
    for (int i = 0; i < G / 2; ++i) {
      const uint4 a = ksp[i];
      ks[4 * i] = a.x; ks[4 * i + 1] = a.y; ks[4 * i + 2] = a.z; ks[4 * i + 3] = a.w;
    }
    const int gn = (lane & 15) * D / 512;    // the lane's V channel group
    const uint2 v = *reinterpret_cast<const uint2*>(blk + 13 * D + 8 * (j * G + gn));
    vs[0] = v.x; vs[1] = v.y;
  }
};

template <int D>
struct PageData<false, D> {
  static constexpr int KW = D / 16;        // dwords of K per lane (D/4 bytes)
  static constexpr int VW = D / 64;        // dwords of V per lane per token (D/16 bytes)
  uint32_t k[KW];
  uint32_t v[4][VW];

  __device__ inline void load(const uint8_t* __restrict__ pg, int lane) {
    const int t = lane & 15, j = lane >> 4, n = lane & 15;
    const uint4* kp = reinterpret_cast<const uint4*>(pg + t * D + j * (D / 4));
#pragma unroll
    for (int i = 0; i < KW / 4; ++i) {
      const uint4 a = kp[i];
      k[4 * i] = a.x; k[4 * i + 1] = a.y; k[4 * i + 2] = a.z; k[4 * i + 3] = a.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint8_t* vp = pg + kPage * D + (4 * j + r) * D + n * (D / 16);
      if constexpr (VW == 4) {
        const uint4 a = *reinterpret_cast<const uint4*>(vp);
        v[r][0] = a.x; v[r][1] = a.y; v[r][2] = a.z; v[r][3] = a.w;
      } else {
        const uint2 a = *reinterpret_cast<const uint2*>(vp);
        v[r][0] = a.x; v[r][1] = a.y;
      }
    }
  }
};

// fp32 -> (fp16 hi, fp16 lo) with hi + lo = x to ~22 bits.
__device__ inline void split_hi_lo(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

}  // namespace

template <bool TQ3, int D>
__global__ void __launch_bounds__(256) partial_mfma_kernel(
    LayerTable lt, int n_layers, int hkv, int G, const float* __restrict__ q, size_t q_ls,
    float qscale, Plan plan) {
  constexpr int NG = D / 32;               // 32-channel MFMA k-chunks (TQ3: scale groups)
  constexpr int NT = D / 16;               // 16-channel output tiles of P V
  __shared__ float so[kWaves][kMaxG][D];
  __shared__ float sm[kWaves][kMaxG], sl[kWaves][kMaxG];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15, j = lane >> 4;   // C/B column (query row or channel slice), row group
  const int n_chunks = plan.totals[TQ3 ? T_NCT : T_NCF];
  const int4* __restrict__ chunks = TQ3 ? plan.chunks_t : plan.chunks_f;
  const int32_t* __restrict__ list = TQ3 ? plan.list_t : plan.list_f;
  const int hq = hkv * G;
  const long items = (long)n_layers * hkv * n_chunks;

  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int h = (int)(item % hkv);
    const int chunk = (int)((item / hkv) % n_chunks);
    const int layer = (int)(item / ((long)hkv * n_chunks));
    const int4 cd = chunks[chunk];
    const int b = cd.x, start = cd.y, count = cd.z & 0xffff, last_tok = cd.z >> 16, pidx = cd.w;
    if (pidx >= plan.np_cap) {               // plan made for more layers than this call
      if (threadIdx.x == 0) atomicOr(plan.status, kDevBadSeqLen);
      continue;
    }
    const float ks_layer = TQ3 ? 1.0f : lt.k_scale[layer];
    const uint8_t* __restrict__ slab = TQ3 ? lt.tq3[layer] : lt.fp8[layer];
    const size_t page_bytes = TQ3 ? (size_t)tq3_page_bytes(hkv, D) : (size_t)fp8_page_bytes(hkv, D);
    const size_t head_off = TQ3 ? (size_t)h * tq3_head_bytes(D) : (size_t)h * 2 * kPage * D;

    // ---- B operand of the score MFMAs: hi rows 0..G-1, lo rows 8..8+G-1 ----
    h8 qf[NG];
    {
      const int row = n < 8 ? n : n - 8;
      const bool use = row < G;
      const float* qrow = q + layer * q_ls + ((size_t)b * hq + (size_t)h * G + (use ? row : 0)) * D;
      const float sc = qscale * ks_layer;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int c0 = TQ3 ? 32 * g + 8 * j : j * (D / 4) + 8 * g;
        const float4 a = *reinterpret_cast<const float4*>(qrow + c0);
        const float4 c = *reinterpret_cast<const float4*>(qrow + c0 + 4);
        float v[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
        // TQ3 slot order of the k-slots: (0,6) (1,7) (3,2) (4,5)
        const int perm[8] = {0, 6, 1, 7, 3, 2, 4, 5};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (TQ3 ? v[perm[e]] : v[e]) * sc;
          _Float16 hi, lo;
          split_hi_lo(x, hi, lo);
          qf[g][e] = !use ? (_Float16)0.0f : (n < 8 ? hi : lo);
        }
      }
    }

    // ---- per-wave online softmax over pages wave, wave+4, ... ----
    f4 O[NT];
#pragma unroll
    for (int T = 0; T < NT; ++T) O[T] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY;
    float l_run = 0.0f;
    const int my_pages = count > wave ? (count - wave + kWaves - 1) / kWaves : 0;
    int ids = 0;                              // page ids of this wave's pages, one per lane (batches of 64)

    PageData<TQ3, D> cur, nxt;
    if (my_pages > 0) {
      ids = lane < my_pages ? list[start + wave + kWaves * lane] : 0;
      const int pid = __builtin_amdgcn_readfirstlane(ids);
      cur.load(slab + (size_t)pid * page_bytes + head_off, lane);
    }
    for (int k = 0; k < my_pages; ++k) {
      if (k + 1 < my_pages) {
        if (((k + 1) & 63) == 0)
          ids = (k + 1 + lane < my_pages) ? list[start + wave + kWaves * (k + 1 + lane)] : 0;
        const int pid = __builtin_amdgcn_readlane(ids, (k + 1) & 63);
        nxt.load(slab + (size_t)pid * page_bytes + head_off, lane);
      }
      const int e = wave + kWaves * k;
      const int ntok = (e == count - 1) ? last_tok : kPage;

      // scores for tokens 4j..4j+3 (rows) of query row n (column)
      f4 s = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        h8 a;
        if constexpr (TQ3) {
          uint32_t X, Y, W;
          triple_words(cur.kc, 3 * g, X, Y, W);
          h2 r[4];
          decode_triple(X, Y, W, r);
          a = h8{r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
          const f4 sg = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[g], f4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          const h2 s01 = u2h(cur.ks[2 * g]), s23 = u2h(cur.ks[2 * g + 1]);
          s[0] = fmaf(sg[0], (float)s01[0], s[0]);
          s[1] = fmaf(sg[1], (float)s01[1], s[1]);
          s[2] = fmaf(sg[2], (float)s23[0], s[2]);
          s[3] = fmaf(sg[3], (float)s23[1], s[3]);
        } else {
          const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.k[2 * g], 1.0f, false);
          const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.k[2 * g], 1.0f, true);
          const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.k[2 * g + 1], 1.0f, false);
          const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(cur.k[2 * g + 1], 1.0f, true);
          a = h8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
          s = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qf[g], s, 0, 0, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[r] += dpp_ror8(s[r]);               // hi + lo query rows
        if (4 * j + r >= ntok) s[r] = -INFINITY;
      }
      float pm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      pm = fmaxf(pm, __shfl_xor(pm, 16));
      pm = fmaxf(pm, __shfl_xor(pm, 32));
      const bool need = pm > m_run + kRescale;
      if (__any(need)) {
        const float m_new = need ? pm : m_run;
        const float alpha = exp2f(m_run - m_new);   // 0 on the first page (m_run = -inf)
        l_run *= alpha;
        m_run = m_new;
        // O rows 4j + r belong to query-row columns 4j + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * j + r);
#pragma unroll
          for (int T = 0; T < NT; ++T) O[T][r] *= ar;
        }
      }
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = exp2f(s[r] - m_run);
        l_run += p[r];
      }
      // A operand of P V: rows 0..7 fp16(p), rows 8..15 the remainder
      h4 pa;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        _Float16 hi, lo;
        split_hi_lo(p[r], hi, lo);
        pa[r] = n < 8 ? hi : lo;
      }

      if constexpr (TQ3) {
        const h2 sv01 = u2h(cur.vs[0]), sv23 = u2h(cur.vs[1]);
#pragma unroll
        for (int pp = 0; pp < NG; ++pp) {
          uint32_t X, Y, W;
          triple_words(cur.vc, 3 * pp, X, Y, W);
          h2 r[4];
          decode_triple(X, Y, W, r);
          const h2 hi0 = r[0] * sv01, hi1 = r[1] * sv23, hi2 = r[2] * sv01, hi3 = r[3] * sv23;
          const h2 lo0 = __builtin_elementwise_fma(r[0], sv01, -hi0);
          const h2 lo1 = __builtin_elementwise_fma(r[1], sv23, -hi1);
          const h2 lo2 = __builtin_elementwise_fma(r[2], sv01, -hi2);
          const h2 lo3 = __builtin_elementwise_fma(r[3], sv23, -hi3);
          O[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, h4{hi0[0], hi0[1], hi1[0], hi1[1]}, O[2 * pp], 0, 0, 0);
          O[2 * pp] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, h4{lo0[0], lo0[1], lo1[0], lo1[1]}, O[2 * pp], 0, 0, 0);
          O[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, h4{hi2[0], hi2[1], hi3[0], hi3[1]}, O[2 * pp + 1], 0, 0, 0);
          O[2 * pp + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, h4{lo2[0], lo2[1], lo3[0], lo3[1]}, O[2 * pp + 1], 0, 0, 0);
        }
      } else {
        constexpr int VW = D / 64;
#pragma unroll
        for (int T = 0; T < NT; T += 2) {
          const int wi = T >> 2, bo = T & 3;           // dword and byte of channel T in a token row
          const uint32_t sel = bo | ((4 + bo) << 8) | ((bo + 1) << 16) | ((5 + bo) << 24);
          const uint32_t w01 = __builtin_amdgcn_perm(cur.v[1][wi], cur.v[0][wi], sel);
          const uint32_t w23 = __builtin_amdgcn_perm(cur.v[3][wi], cur.v[2][wi], sel);
          const h2 a01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w01, 1.0f, false);   // channel T, tokens 0,1
          const h2 b01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w01, 1.0f, true);    // channel T+1
          const h2 a23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w23, 1.0f, false);
          const h2 b23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w23, 1.0f, true);
          O[T] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, h4{a01[0], a01[1], a23[0], a23[1]}, O[T], 0, 0, 0);
          O[T + 1] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, h4{b01[0], b01[1], b23[0], b23[1]}, O[T + 1], 0, 0, 0);
          (void)VW;
        }
      }
      if (k + 1 < my_pages) cur = nxt;
    }

    // ---- wave state -> LDS: O rows i (hi) + i + 8 (lo) live in lanes l and l ^ 32 ----
    const float vscale = TQ3 ? 1.0f : lt.v_scale[layer];
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);             // sum over the four token rows of column n
#pragma unroll
    for (int T = 0; T < NT; ++T) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float tot = O[T][r] + __shfl_xor(O[T][r], 32);
        const int row = 4 * j + r;
        if (j < 2 && row < G) so[wave][row][n * (D / 16) + T] = tot * vscale;
      }
    }
    if (j == 0 && n < G) {
      sm[wave][n] = m_run;
      sl[wave][n] = l_run;
    }
    __syncthreads();

    // ---- merge the 4 wave states and write the item's partial ----
    const size_t slot = ((size_t)layer * plan.np_cap + pidx) * hkv + h;
    float* __restrict__ ml = plan.part_ml + slot * G * 2;
    float* __restrict__ pa_out = plan.part_acc + slot * G * D;
    for (int idx = threadIdx.x; idx < G * D; idx += 256) {
      const int i = idx / D, c = idx - (idx / D) * D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w][i]);
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float wgt = (sm[w][i] == -INFINITY) ? 0.0f : exp2f(sm[w][i] - M);
        acc = fmaf(wgt, so[w][i][c], acc);
      }
      pa_out[idx] = acc;
      if (c == 0) {
        float L = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
          L += (sm[w][i] == -INFINITY) ? 0.0f : sl[w][i] * exp2f(sm[w][i] - M);
        ml[2 * i] = M;
        ml[2 * i + 1] = L;
      }
    }
    __syncthreads();
  }
}

hipError_t launch_partial_mfma(bool tq3, const Geometry& g, const LayerTable& lt, int n_layers,
                               const float* q, size_t q_layer_stride, float qscale,
                               const Plan& plan, hipStream_t stream) {
  long cap = (long)n_layers * g.hkv * (plan.np_cap / 2);
  const dim3 grid((unsigned)(cap < 2048 ? (cap > 0 ? cap : 1) : 2048)), block(256);
  if (tq3) {
    if (g.d == 256)
      hipLaunchKernelGGL((partial_mfma_kernel<true, 256>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
    else
      hipLaunchKernelGGL((partial_mfma_kernel<true, 128>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
  } else {
    if (g.d == 256)
      hipLaunchKernelGGL((partial_mfma_kernel<false, 256>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
    else
      hipLaunchKernelGGL((partial_mfma_kernel<false, 128>), grid, block, 0, stream, lt, n_layers, g.hkv, g.G, q, q_layer_stride, qscale, plan);
  }
  return hipGetLastError();
}

}  // namespace mkv
