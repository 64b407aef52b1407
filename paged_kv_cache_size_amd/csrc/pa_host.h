// Host-side checks and launch-shape policy of libpa.  Pure C++: nothing here
// calls HIP, so every argument check runs (and is tested) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kBlockSize = 16;           // compiled block size (tokens per block)
constexpr int kMaxRepPerWaveValu = 8;    // query heads a VALU (fp32) wave serves from one K/V read
constexpr int kMaxRepPerWaveMfma = 16;   // query heads an MFMA (16-bit) wave serves: the 16 MFMA columns
constexpr int kMinPartition = 128;       // smallest partition the library picks itself
constexpr int kMaxPartitionBlocks = 256;  // a partition's table slice: 4 VGPRs of a wave, one entry per lane
constexpr int kMaxSmallBlockPartition = 1024;  // blocks under 16 tokens: the table in LDS (4 KiB)
constexpr int kMaxAutoPartitionBlocks = 64;  // automatic choice without the context lengths: short
                                             // enough partitions to balance a ragged batch

int elem_bytes(int dtype);  // 0 for an unknown dtype

// Pool block sizes every path runs (powers of two, 1..256): the tiles take
// 16-token steps, so a larger block holds several steps and a smaller one
// contributes a few rows to a step.
constexpr int kMinDecodeBlock = 1;
constexpr int kMaxDecodeBlock = 256;
bool decode_block_size_ok(int block_size, int dtype);
int partition_granule(int block_size);  // partitions are multiples of max(16, block_size) tokens
// log2 of block_size / 16 (blocks of 16 or more tokens) or 16 / block_size.
int block_shift(int block_size);
// Largest partition in tokens: kMaxPartitionBlocks pool blocks, or
// kMaxSmallBlockPartition for blocks under 16 tokens (their table is staged in
// LDS instead of VGPR lanes); the same for the decode and prefill tiles.
int max_partition_tokens(int block_size);
int max_prefill_partition_tokens(int block_size);
int validate_partition(int requested, int block_size);  // decode: requested, or a negated pa_status
int validate_prefill_partition(int requested, int block_size);

// Query heads served per wave: the largest divisor of rep that is <= cap.
int rep_per_wave(int rep, int cap);
// The cap for a dtype's decode kernel (fp32: VALU kernel; fp16/bf16: MFMA kernel).
int max_rep_per_wave(int dtype);

struct DecodeShape {
  int num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len;
  int dtype;
};

// Byte geometry of a K/V pool pair in one of the pa_kv_layout layouts: the K
// row of (block p, token t, KV head h) starts at k + p*block_stride +
// t*row_stride + h*head_stride, its V row at the same offset from v.
//  * PA_KV_SPLIT: two pools [NB, BS, H_kv, D];
//  * PA_KV_FUSED: one pool [NB, H_kv, BS, 2D], K in the first D elements of
//    each row and V in the second (v = k + D elements).
struct PoolView {
  const uint8_t* k = nullptr;
  const uint8_t* v = nullptr;
  int64_t block_stride = 0;
  int64_t row_stride = 0;
  int64_t head_stride = 0;
  // bytes from a block's first byte (at head 0) to the end of the last row of
  // the last head of its first 16 tokens: what one 16-token step may touch
  int64_t step_span(int head_dim_bytes, int num_kv_heads) const {
    return (int64_t)(num_kv_heads - 1) * head_stride + 15 * row_stride + head_dim_bytes;
  }
};

// Kernels address inside one block with 32-bit offsets.
constexpr int64_t kMaxBlockBytes = (int64_t)1 << 31;

// INVALID_ARG for a block larger than kMaxBlockBytes, a null k_pool, an unknown layout, a null v_pool with the
// split layout or a non-null one with the fused layout; UNSUPPORTED for an
// unknown dtype.  Sizes must already be positive.
int pool_view(const void* k_pool, const void* v_pool, int layout, int block_size, int num_kv_heads, int head_dim,
              int dtype, PoolView* pv);

// Argument checks of pa_decode_attention that do not depend on the device.
int check_decode(const void* out, const void* query, const void* k_pool, const void* v_pool,
                 const int32_t* block_tables, const int32_t* context_lens, const DecodeShape& s,
                 float scale);

#ifndef PA_DECODE_MAX_WPW
#define PA_DECODE_MAX_WPW 4
#endif
// Most waves per workgroup of the 16-bit decode kernel (4, or 8 when the
// build sets PA_DECODE_MAX_WPW=8).
constexpr int kDecodeMaxWpw = PA_DECODE_MAX_WPW;

// Launch geometry of the decode partition kernel: one wave per (sequence,
// partition, KV head, chunk of `repc` query heads); `wpw` waves per workgroup
// share (sequence, partition); `groups` workgroups per (sequence, partition).
struct DecodeGrid {
  int rep, repc, chunks, units, wpw, groups;
};
DecodeGrid decode_grid(const DecodeShape& s);

// Predicted duration, in block steps (one 16-token block per resident
// workgroup with every workgroup busy), of the partition and merge launches
// for partitions of `pb` blocks.  `lens`: the num_seqs context lengths in host
// memory, or NULL to take every sequence at max_context_len.
double decode_cost(const DecodeShape& s, int64_t pb, const int32_t* lens, int num_cus, int wg_per_cu);

// Partition size in tokens for the decode kernels.  `requested` = 0 picks the
// candidate of least decode_cost (partitions of at most kMaxAutoPartitionBlocks
// blocks without `lens`, kMaxPartitionBlocks with them); otherwise `requested`
// is validated.  Returns the size (> 0) or a negated pa_status.
int partition_size(const DecodeShape& s, int requested, int num_cus, int wg_per_cu,
                   const int32_t* lens = nullptr);

int num_partitions(int max_context_len, int partition);

// check_decode for a partition-size query (sizes only, no pointers).
int check_partition_query(const DecodeShape& s);

// Workspace bytes for `parts` partitions (0 when parts <= 1).
size_t workspace_bytes(int num_seqs, int num_heads, int head_dim, int parts);

// Upper bound of partition counts the automatic policy can pick.
int auto_partition_bound(int max_context_len, int block_size);

// ----------------------------------------------------------------- prefill
//
// Several new tokens per sequence (varlen prefill, chunked prefill, mixed
// batches): the query rows of sequence b are query_start_loc[b] .. [b+1].
struct PrefillShape {
  DecodeShape d;      // num_seqs, heads, head_dim, block_size, table width, max_context_len, dtype
  int num_tokens;     // rows of query / out
  int max_query_len;  // bound of query_start_loc[b+1] - query_start_loc[b]
};

constexpr size_t kPrefillWorkspaceCap = size_t(256) << 20;  // automatic split: partials kept under 256 MiB

// Argument checks of pa_prefill_attention that do not depend on the device.
int check_prefill(const void* out, const void* query, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                  const PrefillShape& s, float scale);

// Column tiles (16 MFMA columns of (token, query head) pairs) per (sequence, wave unit).
int prefill_tiles(const PrefillShape& s, const DecodeGrid& g);

// Launch geometry of the prefill kernels.  Up to 16 columns per (sequence,
// KV head unit) run the per-wave tile: `items` workgroups of `waves` waves per
// partition, one unit per wave.  More run the cooperative tile, whose waves
// share one unit's K/V blocks: 2 waves of one 16-column tile (32 columns),
// 2 waves of two tiles (64 columns), or kPrefillWgWaves waves of
// kPrefillWaveTiles tiles (128 columns) - the smallest shape that covers the
// columns, so no wave streams K/V for columns it does not have.
constexpr int kPrefillWideCols = 17;
#ifndef PA_PREFILL_WG_WAVES
#define PA_PREFILL_WG_WAVES 4
#endif
constexpr int kPrefillWgWaves = PA_PREFILL_WG_WAVES;  // waves of the cooperative tile
#ifndef PA_PREFILL_WAVE_TILES
#define PA_PREFILL_WAVE_TILES 2
#endif
constexpr int kPrefillWaveTiles = PA_PREFILL_WAVE_TILES;  // 16-column MFMA tiles per wave of the cooperative tile
struct PrefillGrid {
  bool wide;
  int tiles;       // column tiles (16 columns) or column groups (wg_cols columns) per sequence
  int groups;      // workgroups per (sequence, tile, partition): unit groups or units
  int waves;       // waves per workgroup
  int wave_tiles;  // cooperative tile: 16-column tiles per wave
  int64_t items;   // workgroups per partition
};
PrefillGrid prefill_grid(const PrefillShape& s);

// Column mode of the fp32 tiles (fp32 prefill): the columns of a (sequence,
// KV head) are its (new token, query head) pairs, `cols` per wave, the waves
// of a workgroup on consecutive columns so they read each K/V block at the
// same time; ctiles workgroups per (sequence, KV head, partition).  The
// matrix-core tile (fp32 MFMA, the default) takes 16 columns per wave; the
// VALU tile (a build with PA_F32_COLUMNS_MFMA=0) eight at head_dim 64 and
// four at 128 (eight would need more than 256 registers: one wave per SIMD,
// not two).
#ifndef PA_F32_COLUMNS_MFMA
#define PA_F32_COLUMNS_MFMA 1
#endif
constexpr bool kColumnsMfma = PA_F32_COLUMNS_MFMA != 0;
int cols_per_wave(int head_dim);
struct ColumnGrid {
  int cols;       // columns per wave
  int wpw;        // waves per workgroup
  int ctiles;     // workgroups per (sequence, KV head, partition)
  int64_t items;  // workgroups per partition
};
ColumnGrid column_grid(const PrefillShape& s);

// Partitions the automatic prefill split may use: at least enough for the
// 256-block table slice, at most one per 128 tokens, and partials within
// kPrefillWorkspaceCap.
int prefill_partition_bounds(const PrefillShape& s, int* min_parts, int* max_parts);

// Partition size (tokens) for the prefill kernels: `requested` validated, or 0
// to pick the candidate of least cost (every item taken at max_context_len,
// whole waves of `slots` workgroups, plus the merge).  Negated pa_status on error.
int prefill_partition_size(const PrefillShape& s, int requested, int num_cus, int wg_per_cu);
// The same choice for a launch of `items` workgroups of `waves` waves per partition.
int prefill_partition_size_for(const PrefillShape& s, int64_t items, int waves, int requested, int num_cus,
                               int wg_per_cu);

// Shared-prefix decode in one launch: a workgroup per (group, KV head, chunk
// of query heads, set of members), the set's members x query heads filling
// the 16 columns of the matrix-core tile; `waves` waves split the set's key
// steps (its shared blocks, then each member's own) and merge in LDS.
// waves == 0: the batch does not fit this form (block size other than 16,
// fp32, or more than 4 x 256 steps per set) and takes the three-launch
// cascade.
struct SharedPrefixGrid {
  int members_per_set, sets, waves;
  int64_t items;  // workgroups
};
SharedPrefixGrid shared_prefix_grid(const DecodeShape& s, int num_groups, int max_group_size, int num_cus);

// Shared-prefix (cascade) decode: partitions of both passes, and the partial
// slots per (row, head): the prefix's partitions, then the suffix's.
constexpr int kSharedPrefixPartition = 1024;
int shared_prefix_slots(int max_context_len, int max_prefix_len);
int check_shared_prefix(const void* out, const void* query, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_start,
                        const int32_t* prefix_lens, const int32_t* seq_prefix_lens, const PrefillShape& s,
                        int num_groups, int max_group_size, int max_prefix_len, float scale);

int check_combine(const void* out, const int32_t* context_lens, int num_seqs, int num_heads, int head_dim,
                  int max_context_len, int partition_size, int dtype);

int check_reshape(const void* key, const void* value, const void* k_pool, const void* v_pool,
                  const int64_t* slot_mapping, int64_t num_tokens, int num_kv_heads, int head_dim,
                  int block_size, int64_t num_blocks, int dtype);

// pa_convert_blocks: both views built, ids present when pairs > 0.
int check_convert_blocks(const void* dst_k, const void* dst_v, int dst_layout, int64_t dst_num_blocks,
                         const void* src_k, const void* src_v, int src_layout, int64_t src_num_blocks,
                         const int64_t* src, const int64_t* dst, int64_t num_pairs, int block_size,
                         int num_kv_heads, int head_dim, int dtype);

int check_copy_blocks(const void* k_pool, const void* v_pool, const int64_t* src, const int64_t* dst,
                      int64_t num_pairs, int block_size, int num_kv_heads, int head_dim, int64_t num_blocks,
                      int dtype);

int check_slot_mapping(const int64_t* slot_mapping, const int32_t* block_tables,
                       const int32_t* context_lens, const int32_t* query_start_loc, int num_seqs,
                       int max_blocks_per_seq, int block_size, int64_t num_tokens);

}  // namespace pa
