// One decode step in fewer launches: the slot of each sequence's new token
// and the write of its K/V rows in one kernel (slot mapping and the pool
// writer fused), then paged attention as pa_decode_attention_layout runs it.
//
// Source pages: the handbook's slot mapping (section on block tables and
// slot mapping: slot = block_tables[seq][p / block_size] * block_size +
// p % block_size) and its cache write (section "实现", PagedKVCache.write);
// the new token of a decode step is the last position of its context
// (section on paged attention).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_host.h"
#include "pa_runtime.h"

namespace {

// One workgroup per sequence: the new token sits at position
// context_lens[b] - 1.  Its slot goes to slot_out (when given); its K and V
// rows of every KV head are copied into the slot, unless the slot is outside
// the pool (a context of 0 tokens, a table entry past the pool), which, as
// in the separate pool writer, writes nothing.  Strides in units of V.
template <typename V>
__global__ void write_new_tokens_kernel(const V* __restrict__ key, const V* __restrict__ value, V* __restrict__ k_pool,
                                        V* __restrict__ v_pool, const int32_t* __restrict__ block_tables,
                                        const int32_t* __restrict__ context_lens, int64_t* __restrict__ slot_out,
                                        int max_blocks, int block_size, int head_vecs, int num_kv_heads,
                                        int64_t block_stride, int64_t row_stride, int64_t head_stride,
                                        int64_t num_slots) {
  const int64_t b = blockIdx.x;
  const int pos = context_lens[b] - 1;
  int64_t slot = -1;
  if (pos >= 0 && pos / block_size < max_blocks)
    slot = (int64_t)block_tables[b * max_blocks + pos / block_size] * block_size + pos % block_size;
  if (slot_out && threadIdx.x == 0) slot_out[b] = slot;
  if (slot < 0 || slot >= num_slots) return;
  const int row_vecs = head_vecs * num_kv_heads;
  const V* ks = key + b * row_vecs;
  const V* vs = value + b * row_vecs;
  const int64_t base = (slot / block_size) * block_stride + (slot % block_size) * row_stride;
  V* kd = k_pool + base;
  V* vd = v_pool + base;
  for (int t = threadIdx.x; t < row_vecs; t += blockDim.x) {
    const int h = t / head_vecs;
    const int64_t o = h * head_stride + (t - h * head_vecs);
    kd[o] = ks[t];
    vd[o] = vs[t];
  }
}

template <typename V>
int launch_write(const void* key, const void* value, const pa::PoolView& pv, const int32_t* block_tables,
                 const int32_t* context_lens, int64_t* slot_out, int num_seqs, int max_blocks, int block_size,
                 int num_kv_heads, int head_bytes, int64_t num_slots, int threads, hipStream_t st) {
  constexpr int64_t W = sizeof(V);
  return pa::launch_kernel(write_new_tokens_kernel<V>, dim3((unsigned)num_seqs), dim3(threads), st, (const V*)key,
                           (const V*)value, (V*)const_cast<uint8_t*>(pv.k), (V*)const_cast<uint8_t*>(pv.v),
                           block_tables, context_lens, slot_out, max_blocks, block_size, (int)(head_bytes / W),
                           num_kv_heads, pv.block_stride / W, pv.row_stride / W, pv.head_stride / W, num_slots);
}

}  // namespace

extern "C" int pa_write_new_tokens(const void* key, const void* value, void* k_pool, void* v_pool,
                                   const int32_t* block_tables, const int32_t* context_lens, int64_t* slot_mapping,
                                   int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int64_t num_blocks, pa_dtype dtype,
                                   pa_kv_layout layout, void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || !key || !value || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (layout != PA_KV_SPLIT && layout != PA_KV_FUSED) return PA_ERR_INVALID_ARG;
  if (pa::elem_bytes((int)dtype) == 0) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_kv_heads * head_dim > (int64_t)1 << 28) return PA_ERR_INVALID_ARG;
  pa::PoolView pv;
  int rc = pa::pool_view(k_pool, v_pool, (int)layout, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
  const int head_bytes = head_dim * pa::elem_bytes((int)dtype);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_bytes;
  const int64_t num_slots = num_blocks * block_size;
  const uintptr_t align = (uintptr_t)key | (uintptr_t)value | (uintptr_t)pv.k | (uintptr_t)pv.v;
  int vec = 16;
  while (vec > 1 && ((head_bytes % vec) != 0 || (align % vec) != 0)) vec >>= 1;
  const int64_t row_vecs = row_bytes / vec;
  const int threads = row_vecs >= 256 ? 256 : (row_vecs > 64 ? 128 : 64);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const auto run = [&](auto vec_type) {
    using V = decltype(vec_type);
    return launch_write<V>(key, value, pv, block_tables, context_lens, slot_mapping, num_seqs, max_blocks_per_seq,
                           block_size, num_kv_heads, head_bytes, num_slots, threads, st);
  };
  switch (vec) {
    case 16: return run(uint4{});
    case 8: return run(uint2{});
    case 4: return run(uint32_t{});
    case 2: return run(uint16_t{});
    default: return run(uint8_t{});
  }
}

extern "C" int pa_decode_step(void* out, const void* query, const void* key, const void* value, void* k_pool,
                              void* v_pool, const int32_t* block_tables, const int32_t* context_lens,
                              int64_t* slot_mapping, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                              int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                              size_t workspace_bytes, int32_t partition_size, pa_kv_layout layout, void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch
  // Everything the attention call checks, before anything is enqueued: a
  // rejected step writes nothing.
  const pa::DecodeShape shp{num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            max_context_len, (int)dtype};
  int rc = pa::check_decode(out, query, k_pool, layout == PA_KV_FUSED ? k_pool : v_pool, block_tables, context_lens,
                            shp, scale);
  if (rc != PA_OK) return rc;
  if (!key || !value || num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (layout != PA_KV_SPLIT && layout != PA_KV_FUSED) return PA_ERR_INVALID_ARG;
  if (partition_size != 0 && pa::validate_partition(partition_size, block_size) < 0) return PA_ERR_INVALID_ARG;
  // the documented sizing (the bound over the library's own choices when
  // partition_size is 0), so that the attention call cannot refuse it
  const size_t need = pa_decode_workspace_bytes_ex(num_seqs, num_heads, head_dim, max_context_len, block_size,
                                                   partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  rc = pa_write_new_tokens(key, value, k_pool, v_pool, block_tables, context_lens, slot_mapping, num_seqs,
                           num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype, layout, stream);
  if (rc != PA_OK) return rc;
  return pa_decode_attention_layout(out, query, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                                    num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len, scale,
                                    dtype, workspace, workspace_bytes, partition_size, layout, stream);
}
