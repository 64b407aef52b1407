// Whole-block copies of K and V:
//  * inside one pair of pools, for copy-on-write: a sequence about to write
//    into a partly filled block it shares with a fork first gets a private
//    copy of that block ("KV cache: capacity derivation, paging and
//    reclamation", section on shared prefixes and reference counts; the block
//    pool's pa_seq_append reports each such (source, destination) pair);
//  * between two pairs of pools, one of them in pinned host memory, to swap
//    the blocks of a preempted sequence out of HBM and back (handbook "分页 KV
//    Cache", section on scheduling when memory runs short);
//  * between pools of different layouts (split K and V pools, or one pool
//    with K and V joined on the last axis): the handbook's source notes say
//    attention backends differ in layout, so moving KV between them needs a
//    layout conversion (same page, section "源码对照").
//
// Same layout: one workgroup per (pair, pool, slice of the block), vector
// loads and stores of the widest width the block size and the pool addresses
// allow (16, 4 or 2 bytes).  Different layouts: the same grid over head rows,
// each row moved from its source to its destination address.  A pair with an
// id outside its pool is skipped.
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
// `planes` = 2: a K and a V pool; 1: one pool (the fused layout; the v
// pointers are not used).
template <typename V>
int launch(const void* k_src, const void* v_src, void* k_dst, void* v_dst, const int64_t* src, const int64_t* dst,
            int64_t pairs, int planes, int64_t block_bytes, int64_t src_blocks, int64_t dst_blocks, hipStream_t st) {
  const int64_t vecs = block_bytes / (int64_t)sizeof(V);
  const int64_t per_wg = 256 * 4;
  const unsigned slices = (unsigned)std::min<int64_t>((vecs + per_wg - 1) / per_wg, 65535);
  return pa::launch_kernel(copy_blocks_kernel<V>, dim3((unsigned)pairs, (unsigned)planes, slices), dim3(256), st,
                           (const V*)k_src, (const V*)v_src, (V*)k_dst, (V*)v_dst, src, dst, vecs, src_blocks,
                           dst_blocks);
}

int copy_between(const void* k_src, const void* v_src, int64_t src_blocks, void* k_dst, void* v_dst,
                 int64_t dst_blocks, const int64_t* src, const int64_t* dst, int64_t pairs, int planes,
                 int64_t block_bytes, void* stream) {
  if (pairs == 0) return PA_OK;
  uintptr_t align = (uintptr_t)k_src | (uintptr_t)k_dst;
  if (planes == 2) align |= (uintptr_t)v_src | (uintptr_t)v_dst;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (block_bytes % 16 == 0 && align % 16 == 0)
    return launch<uint4>(k_src, v_src, k_dst, v_dst, src, dst, pairs, planes, block_bytes, src_blocks, dst_blocks,
                         st);
  if (block_bytes % 4 == 0 && align % 4 == 0)
    return launch<uint32_t>(k_src, v_src, k_dst, v_dst, src, dst, pairs, planes, block_bytes, src_blocks,
                            dst_blocks, st);
  return launch<uint16_t>(k_src, v_src, k_dst, v_dst, src, dst, pairs, planes, block_bytes, src_blocks, dst_blocks,
                          st);
}

// Pool geometry in vectors of the copy width.
struct RowGeom {
  int64_t block, row, head;
};

// Different layouts: workgroup (pair, K or V, slice) moves head rows of the
// block; vector i of the block is row i / head_vecs (token t, head h in
// token-major order) at position i % head_vecs.
template <typename V>
__global__ __launch_bounds__(256) void convert_blocks_kernel(const V* k_src, const V* v_src, V* k_dst, V* v_dst,
                                                             RowGeom gs, RowGeom gd, const int64_t* __restrict__ src,
                                                             const int64_t* __restrict__ dst, int64_t src_blocks,
                                                             int64_t dst_blocks, int num_kv_heads, int head_vecs,
                                                             int64_t block_vecs) {
  const int64_t s = src[blockIdx.x], d = dst[blockIdx.x];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;
  const V* from = (blockIdx.y == 0 ? k_src : v_src) + s * gs.block;
  V* to = (blockIdx.y == 0 ? k_dst : v_dst) + d * gd.block;
  for (int64_t i = (int64_t)blockIdx.z * blockDim.x + threadIdx.x; i < block_vecs;
       i += (int64_t)gridDim.z * blockDim.x) {
    const int64_t row = i / head_vecs, e = i - row * head_vecs;
    const int64_t t = row / num_kv_heads, h = row - t * num_kv_heads;
    to[t * gd.row + h * gd.head + e] = from[t * gs.row + h * gs.head + e];
  }
}

template <typename V>
int launch_convert(const pa::PoolView& s, const pa::PoolView& d, const int64_t* src, const int64_t* dst,
                    int64_t pairs, int64_t src_blocks, int64_t dst_blocks, int block_size, int num_kv_heads,
                    int head_bytes, hipStream_t st) {
  constexpr int64_t W = sizeof(V);
  const RowGeom gs{s.block_stride / W, s.row_stride / W, s.head_stride / W};
  const RowGeom gd{d.block_stride / W, d.row_stride / W, d.head_stride / W};
  const int64_t vecs = (int64_t)block_size * num_kv_heads * head_bytes / W;  // per plane
  const int64_t per_wg = 256 * 4;
  const unsigned slices = (unsigned)std::min<int64_t>((vecs + per_wg - 1) / per_wg, 65535);
  return pa::launch_kernel(convert_blocks_kernel<V>, dim3((unsigned)pairs, 2, slices), dim3(256), st, (const V*)s.k,
                           (const V*)s.v, (V*)const_cast<uint8_t*>(d.k), (V*)const_cast<uint8_t*>(d.v), gs, gd, src,
                           dst, src_blocks, dst_blocks, num_kv_heads, (int)(head_bytes / W), vecs);
}

}  // namespace

extern "C" int pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* src_blocks, const int64_t* dst_blocks,
                              int64_t num_pairs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                              int64_t num_blocks, pa_dtype dtype, void* stream) {
  const int rc = pa::check_copy_blocks(k_pool, v_pool, src_blocks, dst_blocks, num_pairs, block_size, num_kv_heads,
                                       head_dim, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  const int64_t block_bytes = (int64_t)block_size * num_kv_heads * head_dim * pa::elem_bytes(dtype);
  return copy_between(k_pool, v_pool, num_blocks, k_pool, v_pool, num_blocks, src_blocks, dst_blocks, num_pairs, 2,
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
                      dst_blocks, num_pairs, 2, block_bytes, stream);
}

extern "C" int pa_convert_blocks(void* dst_k_pool, void* dst_v_pool, pa_kv_layout dst_layout, int64_t dst_num_blocks,
                                 const void* src_k_pool, const void* src_v_pool, pa_kv_layout src_layout,
                                 int64_t src_num_blocks, const int64_t* src_blocks, const int64_t* dst_blocks,
                                 int64_t num_pairs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                 pa_dtype dtype, void* stream) {
  int rc = pa::check_convert_blocks(dst_k_pool, dst_v_pool, (int)dst_layout, dst_num_blocks, src_k_pool, src_v_pool,
                                    (int)src_layout, src_num_blocks, src_blocks, dst_blocks, num_pairs, block_size,
                                    num_kv_heads, head_dim, (int)dtype);
  if (rc != PA_OK) return rc;
  if (num_pairs == 0) return PA_OK;
  pa::PoolView s, d;
  pa::pool_view(src_k_pool, src_v_pool, (int)src_layout, block_size, num_kv_heads, head_dim, (int)dtype, &s);
  pa::pool_view(dst_k_pool, dst_v_pool, (int)dst_layout, block_size, num_kv_heads, head_dim, (int)dtype, &d);
  const int head_bytes = head_dim * pa::elem_bytes(dtype);
  if (src_layout == dst_layout) {  // whole blocks: one pool (fused) or two
    const bool fused = src_layout == PA_KV_FUSED;
    return copy_between(s.k, s.v, src_num_blocks, const_cast<uint8_t*>(d.k), const_cast<uint8_t*>(d.v),
                        dst_num_blocks, src_blocks, dst_blocks, num_pairs, fused ? 1 : 2,
                        fused ? s.block_stride : (int64_t)block_size * num_kv_heads * head_bytes, stream);
  }
  const uintptr_t align = (uintptr_t)s.k | (uintptr_t)s.v | (uintptr_t)d.k | (uintptr_t)d.v | (uintptr_t)head_bytes;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (align % 16 == 0)
    return launch_convert<uint4>(s, d, src_blocks, dst_blocks, num_pairs, src_num_blocks, dst_num_blocks, block_size,
                                 num_kv_heads, head_bytes, st);
  if (align % 4 == 0)
    return launch_convert<uint32_t>(s, d, src_blocks, dst_blocks, num_pairs, src_num_blocks, dst_num_blocks,
                                    block_size, num_kv_heads, head_bytes, st);
  return launch_convert<uint16_t>(s, d, src_blocks, dst_blocks, num_pairs, src_num_blocks, dst_num_blocks,
                                  block_size, num_kv_heads, head_bytes, st);
}
