// Whole-block copies of K and V:
//  * inside one pair of pools, for copy-on-write: a sequence about to write
//    into a partly filled block it shares with a fork first gets a private
//    copy of that block ("KV cache: capacity derivation, paging and
//    reclamation", section on shared prefixes and reference counts; the block
//    pool's pa_seq_append reports each such (source, destination) pair);
//  * between two pairs of pools, one of them in pinned host memory, to swap
//    the blocks of a preempted sequence out of HBM and back (handbook "分页 KV
//    Cache", section on scheduling when memory runs short).
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
__global__ __launch_bounds__(256) void copy_blocks_kernel(const V* k_src, const V* v_src, V* k_dst, V* v_dst,
                                                          const int64_t* __restrict__ src,
                                                          const int64_t* __restrict__ dst, int64_t block_vecs,
                                                          int64_t src_blocks, int64_t dst_blocks) {
  const int64_t s = src[blockIdx.x], d = dst[blockIdx.x];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const V* from = (blockIdx.y == 0 ? k_src : v_src) + s * block_vecs;
  V* to = (blockIdx.y == 0 ? k_dst : v_dst) + d * block_vecs;
  for (int64_t i = (int64_t)blockIdx.z * blockDim.x + threadIdx.x; i < block_vecs; i += (int64_t)gridDim.z * blockDim.x)
    to[i] = from[i];
}

// Slices of 1024 vectors per workgroup (four per thread).  Measured on the
// 8192-copy Llama-layer batch: this plain loop beat variants that batch four
// loads ahead of the stores or mark the stream non-temporal (185 us vs
// 210-222 us).
template <typename V>
void launch(const void* k_src, const void* v_src, void* k_dst, void* v_dst, const int64_t* src, const int64_t* dst,
            int64_t pairs, int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks, hipStream_t st) {
  const int64_t vecs = block_bytes / (int64_t)sizeof(V);
  const int64_t per_wg = 256 * 4;
  const unsigned slices = (unsigned)std::min<int64_t>((vecs + per_wg - 1) / per_wg, 65535);
  hipLaunchKernelGGL(copy_blocks_kernel<V>, dim3((unsigned)pairs, 2, slices), dim3(256), 0, st, (const V*)k_src,
                     (const V*)v_src, (V*)k_dst, (V*)v_dst, src, dst, vecs, src_blocks, dst_blocks);
}

int copy_between(const void* k_src, const void* v_src, int64_t src_blocks, void* k_dst, void* v_dst,
                 int64_t dst_blocks, const int64_t* src, const int64_t* dst, int64_t pairs, int64_t block_bytes,
                 void* stream) {
  if (pairs == 0) return PA_OK;
  const uintptr_t align = (uintptr_t)k_src | (uintptr_t)v_src | (uintptr_t)k_dst | (uintptr_t)v_dst;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (block_bytes % 16 == 0 && align % 16 == 0)
    launch<uint4>(k_src, v_src, k_dst, v_dst, src, dst, pairs, block_bytes, src_blocks, dst_blocks, st);
  else if (block_bytes % 4 == 0 && align % 4 == 0)
    launch<uint32_t>(k_src, v_src, k_dst, v_dst, src, dst, pairs, block_bytes, src_blocks, dst_blocks, st);
  else
    launch<uint16_t>(k_src, v_src, k_dst, v_dst, src, dst, pairs, block_bytes, src_blocks, dst_blocks, st);
  return pa::launch_status();
}

}  // namespace

extern "C" int pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* src_blocks, const int64_t* dst_blocks,
                              int64_t num_pairs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, pa_dtype dtype, void* stream) {
  const int rc = pa::check_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, num_pairs, block_size, num_kv_heads,
                                       head_dim, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * pa::elem_bytes(dtype);
  return copy_between(k_pool, v_pool, num_blocks, k_pool, v_pool, num_blocks, src_blocks, dst_blocks, num_pairs,
                      block_bytes, stream);
}

extern "C" int pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, int64_t dst_num_blocks, const void* src_k_pool,
                              const void* src_v_pool, int64_t src_num_blocks, const int64_t* src_blocks,
                              const int64_t* dst_blocks, int64_t num_pairs, int32_t block_size, int32_t num_kv_heads,
                              int32_t head_dim, pa_dtype dtype, void* stream) {
  int rc = pa::check_copy_blocks(dst_k_pool, dst_v_pool, src_blocks, dst_blocks, num_pairs, block_size, num_kv_heads,
                                 head_dim, dst_num_blocks, dtype);
  if (rc != PA_OK) return rc;
  if (!src_k_pool || !src_v_pool || src_num_blocks <= 0) return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * pa::elem_bytes(dtype);
  return copy_between(src_k_pool, src_v_pool, src_num_blocks, dst_k_pool, dst_v_pool, dst_num_blocks, src_blocks,
                      dst_blocks, num_pairs, block_bytes, stream);
}
