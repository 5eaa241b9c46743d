// Segmented path (SGMV) for long slot segments.
#include "common.h"

namespace lora {

hipError_t launch_sgmv_shrink(lora_dtype dt, const ShrinkParams& p, hipStream_t stream) {
  return launch_bgmv_shrink(dt, p, /*tiles=*/true, stream);
}

hipError_t launch_sgmv_expand(lora_dtype dt, const ExpandParams& p, hipStream_t stream) {
  return launch_bgmv_expand(dt, p, /*tiles=*/true, stream);
}

}  // namespace lora
