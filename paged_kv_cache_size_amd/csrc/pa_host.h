// Host-side checks and launch-shape policy of libpa.  Pure C++: nothing here
// calls HIP, so every argument check runs (and is tested) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kBlockSize = 16;           // compiled block size (tokens per block)
constexpr int kMaxRepPerWave = 8;        // query heads one wave serves from one K/V read
constexpr int kMinPartition = 128;       // smallest partition the library picks itself
constexpr int kMaxPartitionBlocks = 64;  // a partition's table slice fits one wave (one entry per lane)

int elem_bytes(int dtype);  // 0 for an unknown dtype

// Query heads served per wave (largest divisor of rep that is <= kMaxRepPerWave)
// and the number of such chunks per KV head.
int rep_per_wave(int rep);

struct DecodeShape {
  int num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len;
  int dtype;
};

// Argument checks of pa_decode_attention that do not depend on the device.
int check_decode(const void* out, const void* query, const void* k_pool, const void* v_pool,
                 const int32_t* block_tables, const int32_t* context_lens, const DecodeShape& s,
                 float scale);

// Partition size in tokens for the decode kernels.  `requested` = 0 picks one
// from the shape and the compute-unit count; otherwise it is validated.
// Returns the size (> 0) or a negated pa_status.
int partition_size(const DecodeShape& s, int requested, int num_cus);

int num_partitions(int max_context_len, int partition);

// Workspace bytes for `parts` partitions (0 when parts <= 1).
size_t workspace_bytes(int num_seqs, int num_heads, int head_dim, int parts);

// Upper bound of partition counts the automatic policy can pick.
int auto_partition_bound(int max_context_len, int block_size);

int check_combine(const void* out, const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                  int max_context_len, int partition_size, int dtype);

int check_reshape(const void* key, const void* value, const void* k_pool, const void* v_pool,
                  const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads, int head_dim,
                  int block_size, int64_t num_blocks, int dtype);

int check_slot_mapping(const int64_t* slot_mapping, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start_loc, int num_seqs,
                       int max_blocks_per_seq, int block_size, int64_t num_tokens);

}  // namespace pa
