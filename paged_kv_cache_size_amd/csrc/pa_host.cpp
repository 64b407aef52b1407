// Host-side argument checks and partition policy of libpa (no HIP calls).
#include "pa_host.h"

#include <cmath>

namespace pa {

int elem_bytes(int dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

int rep_per_wave(int rep, int cap) {
  for (int c = cap; c >= 1; --c)
    if (rep % c == 0) return c;
  return 1;
}

int max_rep_per_wave(int dtype) { return dtype == PA_F32 ? kMaxRepPerWaveValu : kMaxRepPerWaveMfma; }

int check_decode(const void* out, const void* query, const void* k_pool, const void* v_pool,
                 const int32_t* block_tables, const int32_t* context_lens, const DecodeShape& s,
                 float scale) {
  if (!out || !query || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (s.num_seqs <= 0 || s.num_heads <= 0 || s.num_kv_heads <= 0 || s.head_dim <= 0 ||
      s.block_size <= 0 || s.max_blocks_per_seq <= 0 || s.max_context_len <= 0)
    return PA_ERR_INVALID_ARG;
  if (s.num_heads % s.num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)s.max_context_len > (int64_t)s.max_blocks_per_seq * s.block_size) return PA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
  if (elem_bytes(s.dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (s.head_dim != 64 && s.head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (s.block_size != kBlockSize) return PA_ERR_UNSUPPORTED;
  // grid: num_seqs * partitions * head groups workgroups must fit a 32-bit grid
  if ((int64_t)s.num_seqs * s.num_heads > (int64_t)1 << 30) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int num_partitions(int max_context_len, int partition) {
  return (max_context_len + partition - 1) / partition;
}

DecodeGrid decode_grid(const DecodeShape& s) {
  DecodeGrid g;
  g.rep = s.num_heads / s.num_kv_heads;
  g.repc = rep_per_wave(g.rep, max_rep_per_wave(s.dtype));
  g.chunks = g.rep / g.repc;
  g.units = s.num_kv_heads * g.chunks;
  g.wpw = g.units % 4 == 0 ? 4 : (g.units % 2 == 0 ? 2 : 1);
  g.groups = g.units / g.wpw;
  return g;
}

int partition_size(const DecodeShape& s, int requested, int num_cus, int wg_per_cu) {
  const int bs = s.block_size;
  const int max_ps = kMaxPartitionBlocks * bs;
  if (requested != 0) {
    if (requested < bs || requested > max_ps || requested % bs != 0) return -PA_ERR_INVALID_ARG;
    return requested;
  }
  // Cost model in "block steps" (every resident workgroup processing one
  // 16-token block): the batch is assumed to be at max_context_len.
  const DecodeGrid g = decode_grid(s);
  const int64_t slots = (int64_t)(num_cus > 0 ? num_cus : 256) * (wg_per_cu > 0 ? wg_per_cu : 1);
  const int64_t nb = (s.max_context_len + bs - 1) / bs;
  const int64_t bound = auto_partition_bound(s.max_context_len, bs);
  const double wg_block_bytes = (double)g.wpw * 2.0 * bs * s.head_dim * elem_bytes(s.dtype);
  const double setup = 1.0, merge_launch = 1.5;
  int best_pb = 0;
  double best = 0.0;
  for (int64_t parts = 1; parts <= bound; ++parts) {
    const int64_t pb = (nb + parts - 1) / parts;  // blocks per partition
    if (pb > kMaxPartitionBlocks) continue;
    const int64_t p = (nb + pb - 1) / pb;
    const int64_t wgs = (int64_t)s.num_seqs * p * g.groups;
    const int64_t rounds = (wgs + slots - 1) / slots;
    double cost = (double)rounds * ((double)pb + setup);
    if (p > 1)
      cost += merge_launch + 2.0 * (double)s.num_seqs * s.num_heads * p * (s.head_dim + 2) * 4.0 /
                                 ((double)slots * wg_block_bytes);
    if (best_pb == 0 || cost < best - 1e-9) {
      best = cost;
      best_pb = (int)pb;
    }
  }
  if (best_pb == 0) best_pb = kMaxPartitionBlocks;
  return best_pb * bs;
}

int auto_partition_bound(int max_context_len, int block_size) {
  (void)block_size;
  int b = (max_context_len + kMinPartition - 1) / kMinPartition;
  return b < 1 ? 1 : b;
}

size_t workspace_bytes(int num_seqs, int num_heads, int head_dim, int parts) {
  if (parts <= 1) return 0;
  return (size_t)num_seqs * num_heads * parts * ((size_t)head_dim + 2) * sizeof(float);
}

int check_combine(const void* out, const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                  int max_context_len, int partition_size, int dtype) {
  if (!out || !context_lens) return PA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || num_heads <= 0 || max_context_len <= 0) return PA_ERR_INVALID_ARG;
  if (partition_size < kBlockSize || partition_size % kBlockSize != 0 ||
      partition_size > kMaxPartitionBlocks * kBlockSize)
    return PA_ERR_INVALID_ARG;
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int check_reshape(const void* key, const void* value, const void* k_pool, const void* v_pool,
                  const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads, int head_dim,
                  int block_size, int64_t num_blocks, int dtype) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!key || !value || !slot_mapping)) return PA_ERR_INVALID_ARG;
  if (!k_pool || !v_pool) return PA_ERR_INVALID_ARG;
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (num_tokens > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  if ((int64_t)num_kv_heads * head_dim > (int64_t)1 << 28) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int check_slot_mapping(const int64_t* slot_mapping, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start_loc, int num_seqs,
                       int max_blocks_per_seq, int block_size, int64_t num_tokens) {
  if (!slot_mapping || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (num_seqs <= 0 || max_blocks_per_seq <= 0 || block_size <= 0 || num_tokens <= 0)
    return PA_ERR_INVALID_ARG;
  if (!query_start_loc && num_tokens != num_seqs) return PA_ERR_INVALID_ARG;
  if (num_tokens > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: invalid argument";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: dtype, head_dim or block_size not compiled in";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime or launch error";
    default: return "unknown pa_status";
  }
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                            int32_t max_context_len, int32_t block_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || block_size <= 0)
    return 0;
  return pa::workspace_bytes(num_seqs, num_heads, head_dim,
                             pa::auto_partition_bound(max_context_len, block_size));
}

extern "C" size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t block_size,
                                               int32_t partition_size) {
  if (partition_size == 0)
    return pa_decode_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, block_size);
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || block_size <= 0 ||
      partition_size < block_size || partition_size % block_size != 0)
    return 0;
  return pa::workspace_bytes(num_seqs, num_heads, head_dim,
                             pa::num_partitions(max_context_len, partition_size));
}
