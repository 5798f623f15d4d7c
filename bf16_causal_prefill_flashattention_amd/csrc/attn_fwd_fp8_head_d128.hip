// Instantiates the FP8 attention kernels with one scale per (batch, head), head dimensions
// (128, 128), every probability mode.
#include "attn_fwd_impl.hpp"

namespace miattn {

hipError_t launch_attn_fp8_head_d128(const AttnParams& p, dim3 grid, hipStream_t stream) {
  return launch_attn_fp8_modes<128, false>(p, grid, stream);
}

}  // namespace miattn
