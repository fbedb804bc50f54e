// mk_static.hip — the fixed device scratch of mk_decode_step_noalloc.
//
// Callers that cannot allocate device memory while they decode (code under
// HIP graph capture, tight serving loops) run the decode step with its
// scratch (tagged activations, counters, argmax slots, status word) in one
// file-scope device array of MK_NOALLOC_SCRATCH_BYTES bytes instead of the
// context's arena.  Every GPU the library runs on holds its own copy of the
// array until the process ends.  Host code never uses the array's name as a
// device address: mk_scratch_init looks the address up once per device
// (with that device current) and every later use goes through that pointer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mk.h"

namespace {
static __device__ __align__(256) unsigned char scratch[MK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_ptr[kMaxDevices] = {};
std::mutex g_mu;

// Fill [p, p + n16 * 16) with zeros: a kernel, so that the fill is an
// ordinary kernel node if a caller captures the step in a graph.
__global__ void __launch_bounds__(256) mk_fill_zero(uint4* p, uint64_t n16) {
  for (uint64_t i = blockIdx.x * 256ull + threadIdx.x; i < n16; i += uint64_t(gridDim.x) * 256ull)
    p[i] = uint4{0u, 0u, 0u, 0u};
}
}  // namespace

// Device address of this device's scratch array (device = the current one).
// Looked up on the first call per device and kept.
extern "C" hipError_t mk_scratch_init(int device, void** out) {
  if (device < 0 || device >= kMaxDevices || !out) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidSymbol;
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return hipSuccess;
}

// Zero `bytes` (a multiple of 16) at p on `stream`.
extern "C" hipError_t mk_launch_fill_zero(void* p, uint64_t bytes, hipStream_t stream) {
  const uint64_t n16 = bytes / 16;
  if (!n16) return hipSuccess;
  uint64_t blocks = (n16 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(mk_fill_zero, dim3(uint32_t(blocks)), dim3(256), 0, stream, static_cast<uint4*>(p), n16);
  return hipGetLastError();
}
