// Instantiates the FP8 attention kernels with one scale per 64 positions, head dimensions
// (192, 128), every probability mode.
#include "attn_fwd_impl.hpp"

namespace miattn {

hipError_t launch_attn_fp8_block64_d192(const AttnParams& p, dim3 grid, hipStream_t stream) {
  return launch_attn_fp8_modes<192, true>(p, grid, stream);
}

}  // namespace miattn
