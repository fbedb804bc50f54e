// mk_diag.hip — calibration kernel: a plain streaming read of device memory.
//
// The achievable HBM read rate of the box, measured with the same 16-byte
// non-temporal loads the decode path streams its weights with, spread over
// every CU; the decode step's achieved bandwidth is reported against it as
// well as against the published peak.  Each block reads a contiguous span in
// 16 KiB strides with eight loads in flight per thread, folds what it read
// into one word (so that the loads cannot be dropped) and stores it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk.h"

namespace {
typedef uint32_t u4v __attribute__((ext_vector_type(4)));
__global__ void __launch_bounds__(256) mk_stream_read_kernel(const u4v* __restrict__ src, uint64_t n16,
                                                             uint32_t* sink) {
  const uint64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const uint64_t lo = per * blockIdx.x, hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  constexpr int U = 8;
  uint64_t i = lo + threadIdx.x;
  for (; i + (U - 1) * 256 < hi; i += U * 256) {
    u4v v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const u4v v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per block: the xor of every thread's fold
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; t++) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}
}  // namespace

extern "C" mk_status mk_stream_read(const void* d_src, size_t bytes, uint32_t* d_sink, int32_t blocks,
                                    void* stream) {
  if (!d_src || !d_sink || blocks <= 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(d_src) & 15))
    return MK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mk_stream_read_kernel, dim3(uint32_t(blocks)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u4v*>(d_src),
                     uint64_t(bytes / 16), d_sink);
  return hipGetLastError() == hipSuccess ? MK_OK : MK_ERR_HIP;
}
