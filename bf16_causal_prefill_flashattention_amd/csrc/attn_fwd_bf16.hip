// Instantiates the BF16 variants of the attention kernel.
#include "attn_fwd_impl.hpp"

namespace miattn {

hipError_t launch_attn_bf16(const AttnParams& p, int d_qk, dim3 grid, hipStream_t stream) {
  if (d_qk == 128) return launch_attn_variant<128, false, false, false, false>(p, grid, stream);
  if (d_qk == 192) return launch_attn_variant<192, false, false, false, false>(p, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace miattn
