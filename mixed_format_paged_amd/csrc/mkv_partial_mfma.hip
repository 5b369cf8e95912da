// mkv_partial_mfma.hip -- matrix-core partial-attention kernels (placeholder).
#include "mkv_format.h"
#include "mkv_internal.h"

namespace mkv {

hipError_t launch_partial_mfma(bool, const Geometry&, const LayerTable&, int, const float*, size_t,
                               float, const Plan&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace mkv
