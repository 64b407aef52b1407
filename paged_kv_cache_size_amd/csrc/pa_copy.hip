// Whole-block copies inside the K and V pools, for copy-on-write: a sequence
// about to write into a partly filled block it shares with a fork first gets
// a private copy of that block ("KV cache: capacity derivation, paging and
// reclamation", section on shared prefixes and reference counts; the block
// pool's pa_seq_append reports each such (source, destination) pair).
//
// One workgroup per (pair, pool, slice of the block), vector loads and stores
// of the widest width the block size and the pool addresses allow (16, 4 or 2
// bytes).  A pair with an id outside the pool is skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pa.h"
#include "pa_host.h"
#include "pa_runtime.h"

namespace {

template <typename V>
__global__ __launch_bounds__(256) void copy_blocks_kernel(V* __restrict__ k_pool, V* __restrict__ v_pool,
                                                          const int64_t* __restrict__ src,
                                                          const int64_t* __restrict__ dst, int64_t block_vecs,
                                                          int64_t num_blocks) {
  const int64_t s = src[blockIdx.x], d = dst[blockIdx.x];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  V* pool = blockIdx.y == 0 ? k_pool : v_pool;
  const V* from = pool + s * block_vecs;
  V* to = pool + d * block_vecs;
  for (int64_t i = (int64_t)blockIdx.z * blockDim.x + threadIdx.x; i < block_vecs; i += (int64_t)gridDim.z * blockDim.x)
    to[i] = from[i];
}

// Slices of 1024 vectors per workgroup (four per thread).  Measured on the
// 8192-copy Llama-layer batch: this plain loop beat variants that batch four
// loads ahead of the stores or mark the stream non-temporal (185 us vs
// 210-222 us).
template <typename V>
void launch(void* k_pool, void* v_pool, const int64_t* src, const int64_t* dst, int64_t pairs, int64_t block_bytes,
            int64_t num_blocks, hipStream_t st) {
  const int64_t vecs = block_bytes / (int64_t)sizeof(V);
  const int64_t per_wg = 256 * 4;
  const unsigned slices = (unsigned)std::min<int64_t>((vecs + per_wg - 1) / per_wg, 65535);
  hipLaunchKernelGGL(copy_blocks_kernel<V>, dim3((unsigned)pairs, 2, slices), dim3(256), 0, st, (V*)k_pool,
                     (V*)v_pool, src, dst, vecs, num_blocks);
}

}  // namespace

extern "C" int pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* src_blocks, const int64_t* dst_blocks,
                              int64_t num_pairs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, pa_dtype dtype, void* stream) {
  const int rc = pa::check_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, num_pairs, block_size, num_kv_heads,
                                       head_dim, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  if (num_pairs == 0) return PA_OK;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * pa::elem_bytes(dtype);
  const uintptr_t align = (uintptr_t)k_pool | (uintptr_t)v_pool;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (block_bytes % 16 == 0 && align % 16 == 0)
    launch<uint4>(k_pool, v_pool, src_blocks, dst_blocks, num_pairs, block_bytes, num_blocks, st);
  else if (block_bytes % 4 == 0 && align % 4 == 0)
    launch<uint32_t>(k_pool, v_pool, src_blocks, dst_blocks, num_pairs, block_bytes, num_blocks, st);
  else
    launch<uint16_t>(k_pool, v_pool, src_blocks, dst_blocks, num_pairs, block_bytes, num_blocks, st);
  return pa::launch_status();
}
