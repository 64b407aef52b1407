// Streaming read of a device buffer: the HBM read rate this device reaches on
// a plain linear stream, measured beside the decode kernel so its KV-read
// bandwidth can be stated against the device's own ceiling as well as the
// published peak.
//
// Every thread walks the buffer with a grid-wide stride, four 16-byte loads in
// flight, and folds the words into an XOR.  Nothing is stored unless the fold
// equals a fixed pattern, so the loads stay live without a write stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pa.h"
#include "pa_runtime.h"

namespace {

constexpr uint32_t kPattern = 0x5a17c0deu;
constexpr int kThreads = 512;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ u32x4 load16(const u32x4* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n_vec,
                                                               uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    const u32x4 a = load16<NT>(src + i), b = load16<NT>(src + i + stride);
    const u32x4 c = load16<NT>(src + i + 2 * stride), d = load16<NT>(src + i + 3 * stride);
    acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
  }
  for (; i < n_vec; i += stride) acc ^= fold(load16<NT>(src + i));
  if (acc == kPattern) *sink = acc;
}

}  // namespace

extern "C" int pa_stream_read(const void* src, size_t bytes, void* sink, int nontemporal, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0 || (uintptr_t)sink % 4 != 0)
    return PA_ERR_INVALID_ARG;
  const int64_t n_vec = (int64_t)(bytes / 16);
  // 16384 workgroups of 512 threads measured fastest for a linear stream;
  // small buffers get one thread per four vectors
  const int64_t want = (n_vec + 4 * kThreads - 1) / (4 * kThreads);
  const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(want, 16384));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (nontemporal)
    return pa::launch_kernel(stream_read_kernel<true>, dim3(grid), dim3(kThreads), st, (const u32x4*)src, n_vec,
                             (uint32_t*)sink);
  return pa::launch_kernel(stream_read_kernel<false>, dim3(grid), dim3(kThreads), st, (const u32x4*)src, n_vec,
                           (uint32_t*)sink);
}
