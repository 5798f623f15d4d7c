// attn_fwd_noalloc: attn_fwd_ws with the library's own static scratch in place
// of a workspace argument, for callers that cannot allocate device memory.
//
// The scratch is a file-scope device array, one copy per GPU the library runs
// on, held until the process ends.  In host code its name only stands for the
// symbol; the device address of the current GPU's copy comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept, and only that address is handed to the kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "kernels.h"
#include "miattn.h"

namespace {

// The most any key-split plan needs on a device with 256 compute units: a plan
// runs at most one workgroup per compute unit, each with one 256-query range
// of fp32 rows (d_v = 128) and their log2 sums of exp.
constexpr size_t kScratchBytes = MIATTN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes == (size_t)256 * miattn::kQueryTile * (128 + 1) * sizeof(float),
              "the scratch covers every plan on 256 compute units");

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up

// Device address of the current device's scratch (looked up on first use).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MIATTN_ERR_HIP;
  void* ptr = scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MIATTN_ERR_HIP;
    scratch_ptr[dev].store(ptr, std::memory_order_release);  // concurrent callers store the same address
  }
  *out = ptr;
  return MIATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                                int Hkv, int Nq, int Nk, int d_qk, int d_v, int dtype, const float* q_scale,
                                const float* k_scale, const float* v_scale, float softmax_scale, int scales,
                                int p_mode, void* stream) {
  size_t need = 0;
  const int st = attn_fwd_ws_size(B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, scales, p_mode, &need);
  if (st != MIATTN_OK) return st;
  if (need > kScratchBytes) return MIATTN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int a = scratch_address(&ws);
    if (a != MIATTN_OK) return a;
  }
  // every other check, and the launch, are attn_fwd_ws's
  return attn_fwd_ws(q, k, v, out, lse, B, Hq, Hkv, Nq, Nk, d_qk, d_v, dtype, q_scale, k_scale, v_scale,
                     softmax_scale, scales, p_mode, ws, need > 0 ? kScratchBytes : 0, stream);
}
