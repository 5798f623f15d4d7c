// LDS access patterns with a known bank behaviour, for reading the hardware's
// LDS bank-conflict counter against them (bench.py --lds-probe, under
// rocprofv3 --pmc).  A measurement aid built into its own library
// (libmiattn_probe.so); the attention path does not use it.
//
// Each probe kernel has every wave read LDS `iters` times with one
// instruction form, lane l of a wave at byte offset l * STRIDE plus a shift by
// a multiple of 4 KB (which keeps every lane's bank) taken from the value the
// lane read last, so no read can be folded away or hoisted.
// With the LDS's 4-byte banks:
//   ds_read_b32,  STRIDE 4   : consecutive words, no two lanes share a bank
//   ds_read_b32,  STRIDE 8   : lanes l and l + 32 (64 banks) or l + 16 (32
//                              banks) share a bank: a 2-way conflict
//   ds_read_b32,  STRIDE 256 : every lane reads bank 0
//   ds_read_b128, STRIDE 16  : consecutive 16-byte chunks (conflict-free)
//   ds_read_b128, STRIDE 256 : every lane's chunk starts at bank 0
//   ds_read_b64_tr_b8 (the transposing read of the attention kernel's V
//   operand), STRIDE 8 : consecutive 8-byte pieces; STRIDE 256: bank 0 for all.
// The values read are summed into one word per thread and stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kLdsBytes = 64 * 1024;
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

enum Kind { kB32 = 0, kB128 = 1, kTr8 = 2 };

template <int KIND, int STRIDE>
__global__ __launch_bounds__(kThreads) void lds_probe_kernel(int* out, int iters) {
  __shared__ __attribute__((aligned(16))) int lds[kLdsBytes / 4];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < kLdsBytes / 4; i += kThreads) lds[i] = i * 2654435761u;
  __syncthreads();
  int acc = lane;
  for (int it = 0; it < iters; ++it) {
    // (offsets stay below 64 KB and aligned to the access size)
    const uint32_t a = ((uint32_t)lane * STRIDE + ((uint32_t)acc & 3u) * 4096u) & (kLdsBytes - 1);
    if constexpr (KIND == kB32) {
      acc += lds[a / 4];
    } else if constexpr (KIND == kB128) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(reinterpret_cast<const char*>(lds) + a);
      acc += v[0] ^ v[1] ^ v[2] ^ v[3];
    } else {
      const uint32_t base = (uint32_t)(size_t)(__attribute__((address_space(3))) int*)lds;
      const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(size_t)(base + a));
      acc += v[0] ^ v[1];
    }
  }
  out[blockIdx.x * kThreads + tid] = acc;
}

template <int KIND, int STRIDE>
int run(int* out, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL((lds_probe_kernel<KIND, STRIDE>), dim3(blocks), dim3(kThreads), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace

extern "C" {

// Threads per probe workgroup (out holds blocks * this many ints).
int lds_probe_threads(void) { return kThreads; }

// Run probe (kind, stride): kind 0 = ds_read_b32 (stride 4, 8 or 256 bytes),
// 1 = ds_read_b128 (16 or 256), 2 = ds_read_b64_tr_b8 (8 or 256); `blocks`
// workgroups of lds_probe_threads() threads, `iters` reads each, one int per
// thread written to out (device memory).  Returns 0, -1 for an unknown
// probe or non-positive sizes, -5 when the launch failed.
int lds_probe_run(int kind, int stride, int blocks, int iters, int* out, void* stream) {
  if (blocks < 1 || iters < 1 || out == nullptr) return -1;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == kB32 && stride == 4) return run<kB32, 4>(out, blocks, iters, s);
  if (kind == kB32 && stride == 8) return run<kB32, 8>(out, blocks, iters, s);
  if (kind == kB32 && stride == 256) return run<kB32, 256>(out, blocks, iters, s);
  if (kind == kB128 && stride == 16) return run<kB128, 16>(out, blocks, iters, s);
  if (kind == kB128 && stride == 256) return run<kB128, 256>(out, blocks, iters, s);
  if (kind == kTr8 && stride == 8) return run<kTr8, 8>(out, blocks, iters, s);
  if (kind == kTr8 && stride == 256) return run<kTr8, 256>(out, blocks, iters, s);
  return -1;
}

}  // extern "C"
