// mkv_gather.hip -- page-table gather of raw page bytes (test support).
//
// Every live-request page stays addressable through the block table
// (arXiv 2608.23834, page 1, Abstract).  One workgroup per logical page copies
// the page's bytes, in logical order, into a record of FP8-page size.
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

__global__ void __launch_bounds__(256) gather_kernel(
    const uint8_t* __restrict__ fp8_slab, const uint8_t* __restrict__ tq3_slab, int n_fp8,
    int n_tq3, int hkv, int d, const int32_t* __restrict__ bt_offsets,
    const int32_t* __restrict__ bt_pages, int b, uint8_t* __restrict__ out) {
  const int lp = blockIdx.x;
  const int rec = fp8_page_bytes(hkv, d);
  const int tqb = tq3_page_bytes(hkv, d);
  const int id = bt_pages[bt_offsets[b] + lp];
  uint4* o = reinterpret_cast<uint4*>(out + (size_t)lp * rec);
  const int n16 = rec / 16;
  const uint4 ff = make_uint4(~0u, ~0u, ~0u, ~0u), zero = make_uint4(0u, 0u, 0u, 0u);
  if (id >= 0 && id < n_fp8) {
    const uint4* in = reinterpret_cast<const uint4*>(fp8_slab + (size_t)id * rec);
    for (int e = threadIdx.x; e < n16; e += blockDim.x) o[e] = in[e];
  } else if (id >= n_fp8 && id < n_fp8 + n_tq3) {
    const uint4* in = reinterpret_cast<const uint4*>(tq3_slab + (size_t)(id - n_fp8) * tqb);
    for (int e = threadIdx.x; e < n16; e += blockDim.x) o[e] = (e < tqb / 16) ? in[e] : zero;
  } else {
    for (int e = threadIdx.x; e < n16; e += blockDim.x) o[e] = ff;
  }
}

hipError_t launch_gather(const Geometry& g, const uint8_t* fp8_slab, const uint8_t* tq3_slab,
                         const int32_t* bt_offsets, const int32_t* bt_pages, int b, int n_pages,
                         uint8_t* out, hipStream_t stream) {
  if (n_pages == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(n_pages), dim3(256), 0, stream, fp8_slab, tq3_slab,
                     g.n_fp8, g.n_tq3, g.hkv, g.d, bt_offsets, bt_pages, b, out);
  return hipGetLastError();
}

}  // namespace mkv
