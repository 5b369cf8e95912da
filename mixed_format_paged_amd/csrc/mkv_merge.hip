// mkv_merge.hip -- globally normalised log-sum-exp merge of partial states.
//
// Minima-KV combines the format-specific partial attention states through a
// globally normalised online-softmax merge (arXiv 2608.23834, page 1,
// Abstract): with partials (m_p, l_p, acc_p) in log2 units,
//   M = max_p m_p,  w_p = 2^(m_p - M),  L = sum_p l_p w_p,
//   o = sum_p acc_p w_p / L,  lse = (M + log2 L) * ln 2.
// One launch merges any number of partials per request.  A workgroup takes
// (layer, request, KV head, group of up to 8 query rows, slice of 32
// channels), 512 threads (a KV head has R = T G rows: T query tokens per
// request times G heads; row r = t G + g goes to out[b][t][h G + g]):
//   1. each thread requests its share of the partial states (registers) and
//      the workgroup the (m, l) pairs of the request (LDS), in one go;
//   2. M per query head, then the weights w_p into LDS (one exp2 per partial
//      and head, shared by every channel of the slice) and L: one wave per
//      head, lanes strided over partials, DPP / permlane reductions;
//   3. each (head, channel) pair of the slice is summed by several threads
//      over interleaved partials, and their sums are added in a fixed order.
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

namespace {

__device__ inline const int* req_row(const Plan& p, int field) { return p.req + (size_t)field * (p.batch + 1); }

typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kSliceC = 32;                      // channels per workgroup
constexpr int kQuads = kSliceC / 4;              // float4 columns of a slice
constexpr int kSubs = kThreads / (kMaxG * kQuads);   // threads sharing one (head, float4 column)
constexpr int kTileP = 512;                      // partials whose weights sit in LDS at once
constexpr int kReg = 16;                         // partial states (float4) a thread prefetches

// Reductions over a wave without LDS: DPP row rotates inside each 16-lane
// row, then the gfx950 permlane swaps across rows; every lane gets the result.
template <int K>
__device__ inline float ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x120 + K, 0xf, 0xf, false));
}
__device__ inline float wave_max(float x) {
  x = fmaxf(x, ror<1>(x));
  x = fmaxf(x, ror<2>(x));
  x = fmaxf(x, ror<4>(x));
  x = fmaxf(x, ror<8>(x));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wave_sum(float x) {
  x += ror<1>(x);
  x += ror<2>(x);
  x += ror<4>(x);
  x += ror<8>(x);
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace

// Thread t takes float4 column q = t % kQuads of the slice, query row
// i = (t / kQuads) % kMaxG of the row group (idle past its rows) and every kSubs-th partial from
// sub = t / (kQuads kMaxG): its loads are 16-byte vectors, and the kQuads
// threads of one (partial, head) read one contiguous 128-byte line.
template <int D>
__global__ void __launch_bounds__(kThreads) merge_kernel(int n_layers, int hkv, int Gh, Plan plan,
                                                         float* __restrict__ out, float* __restrict__ lse,
                                                         size_t out_ls, size_t lse_ls) {
  constexpr int NS = D / kSliceC;
  const int T = plan.n_query;
  const int R = T * Gh;                                     // rows per KV head
  const int NRG = (R + kMaxG - 1) / kMaxG;                  // row groups
  __shared__ float sw[kTileP * kMaxG];          // weights of the current tile, [p][i]
  __shared__ float sml[kTileP * kMaxG * 2];     // (m, l) of the current tile, [p][i][2]
  __shared__ f4v sred[kThreads];                // per-thread sums, [sub][i][q]
  __shared__ float sM[kMaxG], sL[kMaxG];
  const int B = plan.batch;
  const int* poff = req_row(plan, R_POFF);
  const int* inval = req_row(plan, R_INVALID);
  const int hq = hkv * Gh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qc = tid % kQuads, pi = (tid / kQuads) % kMaxG, sub = tid / (kQuads * kMaxG);
  const long items = (long)n_layers * B * hkv * NRG * NS;
  // output element of row r of request b, KV head h
  auto out_at = [&](int layer, int b, int h, int r) {
    const int t = r / Gh;
    return ((size_t)(b * T + t) * hq + (size_t)h * Gh + (r - t * Gh));
  };
  for (long item = blockIdx.x; item < items; item += gridDim.x) {
    const int cs = (int)(item % NS);
    const int rg = (int)((item / NS) % NRG);
    const int h = (int)((item / ((long)NS * NRG)) % hkv);
    const int b = (int)((item / ((long)NS * NRG * hkv)) % B);
    const int layer = (int)(item / ((long)NS * NRG * hkv * B));
    const int r0 = rg * kMaxG;
    const int G = R - r0 < kMaxG ? R - r0 : kMaxG;          // rows of this group
    const bool live = pi < G;
    const int p0 = poff[b], np = poff[b + 1] - poff[b];
    float* out_row = out + layer * out_ls + out_at(layer, b, h, r0 + (live ? pi : 0)) * D + cs * kSliceC;
    float* lse_l = lse ? lse + layer * lse_ls : nullptr;
    if (inval[b] || np == 0 || p0 + np > plan.np_cap) {   // uniform per workgroup
      const bool nan = inval[b] != 0 || np != 0;
      if (sub == 0 && live)
        *reinterpret_cast<f4v*>(out_row + 4 * qc) = nan ? f4v{NAN, NAN, NAN, NAN} : f4v{0.0f, 0.0f, 0.0f, 0.0f};
      if (cs == 0 && lse_l && tid < G) lse_l[out_at(layer, b, h, r0 + tid)] = nan ? __int_as_float(0x7fc00000) : -INFINITY;
      continue;
    }
    const size_t sstride = (size_t)hkv * R;                 // states between consecutive partials
    const size_t st0 = ((size_t)layer * plan.np_cap * hkv + (size_t)p0 * hkv + h) * R + r0;
    const float* ml = plan.part_ml + st0 * 2;
    const float* acc = plan.part_acc + st0 * D + cs * kSliceC + (size_t)(live ? pi : 0) * D + 4 * qc;
    f4v a = f4v{0.0f, 0.0f, 0.0f, 0.0f};
    for (int t0 = 0; t0 < np; t0 += kTileP) {
      const int nt = np - t0 < kTileP ? np - t0 : kTileP;
      const float* ap = acc + (size_t)t0 * sstride * D;
      const int cnt = live ? (nt - sub + kSubs - 1) / kSubs : 0;   // this thread's partials
      const bool in_regs = nt <= kSubs * kReg;                   // uniform
      // 1. this thread's partial states to registers, the tile's (m, l) to LDS
      f4v av[kReg];
      if (in_regs) {
#pragma unroll
        for (int k = 0; k < kReg; ++k)
          av[k] = k < cnt ? *reinterpret_cast<const f4v*>(ap + (size_t)(sub + k * kSubs) * sstride * D)
                          : f4v{0.0f, 0.0f, 0.0f, 0.0f};
      }
      for (int idx = tid; idx < nt * 2 * G; idx += kThreads) {      // (m, l) rows of 2G floats
        const int p = idx / (2 * G), k = idx - p * (2 * G);
        sml[idx] = ml[(t0 + p) * sstride * 2 + k];
      }
      __syncthreads();
      // 2. M per query head (first tile), then the tile's weights and L
      if (t0 == 0) {
        for (int i = wave; i < G; i += kThreads / 64) {
          float M = -INFINITY;
          for (int p = lane; p < nt; p += 64) M = fmaxf(M, sml[p * 2 * G + 2 * i]);
          M = wave_max(M);
          if (lane == 0) { sM[i] = M; sL[i] = 0.0f; }
        }
        if (nt < np) {                                              // the other tiles' maxima
          __syncthreads();
          for (int i = wave; i < G; i += kThreads / 64) {
            float M = sM[i];
            for (int p = nt + lane; p < np; p += 64) M = fmaxf(M, ml[(p * sstride + i) * 2]);
            M = wave_max(M);
            if (lane == 0) sM[i] = M;
          }
        }
        __syncthreads();
      }
      for (int i = wave; i < G; i += kThreads / 64) {
        const float M = sM[i];
        float l = 0.0f;
        for (int p = lane; p < nt; p += 64) {
          const float m = sml[p * 2 * G + 2 * i];
          const float w = (m == -INFINITY) ? 0.0f : exp2f(m - M);
          sw[p * G + i] = w;
          l += sml[p * 2 * G + 2 * i + 1] * w;
        }
        l = wave_sum(l);
        if (lane == 0) sL[i] += l;
      }
      __syncthreads();
      // 3. this thread's interleaved partials, in index order
      if (in_regs) {
#pragma unroll
        for (int k = 0; k < kReg; ++k)
          if (k < cnt) a += sw[(sub + k * kSubs) * G + pi] * av[k];
      } else {
        for (int k = 0; k < cnt; ++k)
          a += sw[(sub + k * kSubs) * G + pi] * *reinterpret_cast<const f4v*>(ap + (size_t)(sub + k * kSubs) * sstride * D);
      }
      __syncthreads();
    }
    sred[tid] = a;
    __syncthreads();
    if (sub == 0 && live) {
      f4v o = a;
      for (int s = 1; s < kSubs; ++s) o += sred[s * kQuads * kMaxG + tid];
      const float L = sL[pi];
      const f4v r = L > 0.0f ? o / L : f4v{0.0f, 0.0f, 0.0f, 0.0f};
      *reinterpret_cast<f4v*>(out_row + 4 * qc) = r;
    }
    if (cs == 0 && lse_l && tid < G)
      lse_l[out_at(layer, b, h, r0 + tid)] = sL[tid] > 0.0f ? (sM[tid] + log2f(sL[tid])) * 0.69314718055994531f : -INFINITY;
    __syncthreads();
  }
}

hipError_t launch_merge(const Geometry& g, int n_layers, const Plan& plan, float* out, float* lse,
                        size_t out_ls, size_t lse_ls, hipStream_t stream) {
  const int R = plan.n_query * g.G;
  const long cap = (long)n_layers * plan.batch * g.hkv * ((R + kMaxG - 1) / kMaxG) * (g.d / kSliceC);
  const dim3 grid((unsigned)(cap < 4096 ? (cap > 0 ? cap : 1) : 4096));
  if (g.d == 256)
    hipLaunchKernelGGL(merge_kernel<256>, grid, dim3(kThreads), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
  else
    hipLaunchKernelGGL(merge_kernel<128>, grid, dim3(kThreads), 0, stream, n_layers, g.hkv, g.G, plan, out, lse, out_ls, lse_ls);
  return hipGetLastError();
}

}  // namespace mkv
