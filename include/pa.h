/*
 * pa.h - C ABI of libpa: the paged KV-cache write and paged decode attention
 * for AMD MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   HB - inference-systems handbook, chapter "分页 KV Cache" (Paged KV Cache)
 *   MV - mini-vllm tutorial step 12, "PagedAttention：分页内存管理"
 *   KC - "KV cache：容量推导、分页与回收" (capacity, paging and reclamation)
 *   AQ - aiqz.cc article "paged-attention"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument except `stream` is a DEVICE pointer on the current
 *    HIP device, allocated and owned by the caller.  The library allocates
 *    nothing, keeps no state beyond per-device caches of the compute-unit
 *    count and of how many workgroups of each decode kernel fit one compute
 *    unit (both filled on first use, guarded for concurrent callers) and the
 *    static partial buffer of pa_decode_attention_noalloc (one per GPU, the
 *    only call that uses it), and may be called from several threads.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; nothing synchronises the device.  Two
 *    calls on one stream run in call order, which is how a pool write is
 *    ordered before the attention that reads it.
 *  - The return value is a pa_status.  Arguments are checked on the host
 *    before any HIP call: a failed check returns PA_ERR_INVALID_ARG /
 *    PA_ERR_UNSUPPORTED / PA_ERR_WORKSPACE and enqueues nothing.  A launch
 *    failure returns PA_ERR_HIP.  Device-side CONTENTS (block ids, context
 *    lengths, slots) are not checked by the host; what each kernel does with
 *    out-of-range contents is stated per entry point.
 *  - Layouts are dense, row-major, with no padding:
 *      KV pool   [num_blocks, block_size, num_kv_heads, head_dim]  (HB, "实现":
 *                one K tensor and one V tensor of this shape per layer; the
 *                token at slot s = block * block_size + offset is row s of the
 *                pool viewed as [num_blocks*block_size, num_kv_heads, head_dim])
 *      key/value [num_tokens, num_kv_heads, head_dim]
 *      query/out [num_seqs, num_heads, head_dim]
 *      block_tables [num_seqs, max_blocks_per_seq] int32, entry j = physical
 *                block of logical block j (HB, "块表与 slot mapping"; AQ,
 *                "块表管理机制"); entries past a sequence's last block are
 *                never read
 *      context_lens [num_seqs] int32 = tokens of the context AFTER this step,
 *                the new token included (HB, "分页注意力", the seq_lens input)
 *  - Element types: query, key, value, pools and out share one pa_dtype.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enums below are int-sized in C and in C++ (where they get int as a
 * fixed underlying type), so a caller may pass any int: a value outside the
 * listed ones is rejected with an error status, never read as undefined. */
#ifdef __cplusplus
#define PA_ENUM_BASE : int
#else
#define PA_ENUM_BASE
#endif

typedef enum pa_status PA_ENUM_BASE {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, inconsistent shape */
  PA_ERR_UNSUPPORTED = 2, /* dtype / head_dim / block_size outside the compiled set */
  PA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  PA_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  PA_ERR_NO_BLOCKS = 5    /* the block pool has too few free blocks; nothing changed */
} pa_status;

typedef enum pa_dtype PA_ENUM_BASE {
  PA_F32 = 0,  /* IEEE binary32 */
  PA_F16 = 1,  /* IEEE binary16 */
  PA_BF16 = 2  /* bfloat16 (upper 16 bits of a binary32) */
} pa_dtype;

/*
 * Physical arrangement of a layer's K/V pool (the _layout entry points).
 *   PA_KV_SPLIT  one K pool and one V pool, each [num_blocks, block_size,
 *                num_kv_heads, head_dim] (HB, "实现") - what every entry point
 *                without a layout argument takes;
 *   PA_KV_FUSED  one pool [num_blocks, num_kv_heads, block_size, 2*head_dim]
 *                with a token's K row in the first head_dim elements of its
 *                row and the V row in the second (HB, "源码对照": the tensor
 *                shape of vLLM's FlashAttention backend, K and V joined on the
 *                last axis).  A head's rows of one block are contiguous.
 * Both hold the same logical K[slot][h][:], V[slot][h][:]; only addresses
 * differ, so every result is the same in both layouts.
 */
typedef enum pa_kv_layout PA_ENUM_BASE {
  PA_KV_SPLIT = 0,
  PA_KV_FUSED = 1
} pa_kv_layout;

/*
 * pa_slot_mapping - physical slot of every new token of one step.
 *
 * Position p of a sequence lives in logical block p / block_size at offset
 * p % block_size; its slot is block_tables[seq][p / block_size] * block_size
 * + p % block_size (HB, "块表与 slot mapping"; MV, "block_table：逻辑位置到物理
 * 槽位的翻译").  Sequence b's new tokens are the LAST n_b positions of its
 * context, context_lens[b] - n_b .. context_lens[b] - 1 (HB, "分页注意力").
 *
 *   slot_mapping     out, int64 [num_tokens]; tokens of sequence b occupy
 *                    query_start_loc[b] .. query_start_loc[b+1]-1
 *   block_tables     int32 [num_seqs, max_blocks_per_seq]
 *   context_lens     int32 [num_seqs]
 *   query_start_loc  int32 [num_seqs+1] prefix sums of n_b, or NULL for a
 *                    decode step (n_b = 1, token b of sequence b)
 *   num_tokens       = query_start_loc[num_seqs] (num_seqs when NULL)
 *
 * Device contents: a token whose position is negative or whose logical block
 * is >= max_blocks_per_seq gets slot -1 (pa_reshape_and_cache skips it).
 * Errors: INVALID_ARG for null pointers, num_seqs/num_tokens/block_size/
 * max_blocks_per_seq <= 0, or num_tokens != num_seqs when query_start_loc is
 * NULL.  An empty batch (num_seqs == num_tokens == 0) is allowed and enqueues
 * nothing; its pointers may be NULL.
 */
int pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                    const int32_t* context_lens, const int32_t* query_start_loc,
                    int32_t num_seqs, int32_t max_blocks_per_seq, int32_t block_size,
                    int64_t num_tokens, void* stream);

/*
 * pa_reshape_and_cache - write each new token's K and V rows into its slot.
 *
 * k_pool viewed as [num_blocks*block_size, num_kv_heads, head_dim] gets
 * row slot_mapping[i] = key[i], and v_pool likewise gets value[i]; a raw bit
 * copy (HB, "实现", PagedKVCache.write).  Slots must be distinct.
 *
 *   key, value        [num_tokens, num_kv_heads, head_dim], dtype
 *   k_pool, v_pool    [num_blocks, block_size, num_kv_heads, head_dim], dtype
 *   slot_mapping      int64 [num_tokens]
 *
 * Device contents: a slot outside [0, num_blocks*block_size) - e.g. -1 for
 * padding - is skipped and nothing is written for that token.  Duplicate
 * slots race (which row lands is unspecified).
 * Errors: INVALID_ARG for null pointers or non-positive sizes; UNSUPPORTED
 * for an unknown dtype.  num_tokens == 0 is allowed and enqueues nothing.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                         const int64_t* slot_mapping, int64_t num_tokens,
                         int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                         int64_t num_blocks, pa_dtype dtype, void* stream);

/*
 * Workspace for pa_decode_attention: float32 partial results of the split
 * (partitioned) context, bytes >= what any partition size the library
 * chooses needs for these sizes.  0 if the sizes are invalid.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t block_size);

/* Workspace bytes for an explicit partition_size (see _ex below). */
size_t pa_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t block_size,
                                    int32_t partition_size);

/*
 * pa_decode_attention - one decode step of paged attention.
 *
 * For every sequence b and query head h, with g = h / (num_heads /
 * num_kv_heads) the KV head serving h (grouped-query attention, HB "实现"
 * paged_attention), and t over the context_lens[b] positions read through
 * block_tables[b]:
 *     out[b,h,:] = sum_t softmax_t(scale * <query[b,h,:], K[t,g,:]>) V[t,g,:]
 * (HB, "分页注意力"; AQ, "工程实现要点": blocks are processed one by one and
 * merged with the online-softmax rescaling).  Scores, softmax and the value
 * sum are accumulated in float32; out is rounded to dtype (nearest-even).
 * The context may be split into partitions whose partial results are merged
 * by a second kernel through the workspace.
 *
 *   out            [num_seqs, num_heads, head_dim], dtype
 *   query          [num_seqs, num_heads, head_dim], dtype
 *   k_pool, v_pool [*, block_size, num_kv_heads, head_dim], dtype
 *   block_tables   int32 [num_seqs, max_blocks_per_seq]
 *   context_lens   int32 [num_seqs], each in [1, max_context_len]
 *   scale          softmax scale, usually head_dim^-1/2 (HB, "分页注意力"); any finite value,
 *                  negative and zero included (zero: the plain mean of the visible V rows)
 *   workspace      device buffer of workspace_bytes >=
 *                  pa_decode_workspace_bytes(...), or NULL/0 when
 *                  max_context_len needs a single partition
 *
 * Supported: dtype F32/F16/BF16, head_dim 64 or 128, num_heads a multiple
 * of num_kv_heads; block_size a power of two from 1 to 256 (the handbook's
 * block-size trade-off, section "块大小怎么选").
 * Device contents: block ids must address blocks of the pools and
 * context_lens must lie in [0, max_context_len]; anything else is undefined
 * (reads outside the pools).  A context length of 0 yields zeros.
 * Errors: INVALID_ARG for null pointers, non-positive sizes,
 * num_heads % num_kv_heads != 0, max_context_len > max_blocks_per_seq *
 * block_size, or a non-finite scale; UNSUPPORTED for other dtype /
 * head_dim / block_size; WORKSPACE if the workspace is too small.
 * num_seqs == 0 (an empty batch) is allowed and enqueues nothing; the
 * pointers other than v_pool may then be NULL.  The same holds for
 * pa_decode_partitions, pa_decode_combine and
 * pa_decode_attention_shared_prefix.
 */
int pa_decode_attention(void* out, const void* query, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens,
                        int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                        int32_t max_context_len, float scale, pa_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * As pa_decode_attention with an explicit partition size in tokens: a
 * multiple of max(16, block_size) (whole pool blocks and whole 16-token steps
 * of the matrix-core tile) of at most 256 blocks - 1024 blocks for blocks
 * under 16 tokens - or 0 to let the library choose.  INVALID_ARG for other
 * values.
 */
int pa_decode_attention_ex(void* out, const void* query, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                           int32_t max_context_len, float scale, pa_dtype dtype,
                           void* workspace, size_t workspace_bytes, int32_t partition_size,
                           void* stream);

/*
 * The two stages of pa_decode_attention_ex, for callers that time or
 * schedule them separately.  `partition_size` must be explicit here (a value
 * pa_decode_partition_size returned, or any valid size) and identical in both
 * calls.
 *
 * pa_decode_partitions: attention over every (sequence, partition, KV head)
 * tile.  A sequence whose context fits one partition gets its final output
 * directly; the others leave per-partition (max, denominator, weighted value
 * sum) partials in the workspace.
 *
 * pa_decode_combine: merges the partials of every sequence that spans more
 * than one partition into out (softmax rescaling by exp(m_s - max_s m_s));
 * enqueues nothing when max_context_len fits one partition.
 * Errors: as pa_decode_attention_ex.
 */
int pa_decode_partitions(void* out, const void* query, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t max_context_len, float scale, pa_dtype dtype,
                         void* workspace, size_t workspace_bytes, int32_t partition_size,
                         void* stream);

int pa_decode_combine(void* out, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t head_dim, int32_t max_context_len,
                      int32_t partition_size, pa_dtype dtype, const void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * pa_decode_attention_noalloc - pa_decode_attention_ex for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments without the workspace; the
 * call allocates nothing (no hipMalloc / hipFree, no allocating library
 * routine).  The split-context partials go to a device buffer of
 * PA_DECODE_SCRATCH_BYTES that the library holds, one per GPU, from the first
 * call on that GPU until the process ends.
 *   partition_size  as pa_decode_attention_ex (0: the library's own choice).
 * Errors: as pa_decode_attention_ex, and PA_ERR_WORKSPACE, with nothing
 * enqueued, when the partition size needs more partial bytes than
 * PA_DECODE_SCRATCH_BYTES (pa_decode_workspace_bytes_ex gives the count for
 * an explicit size); PA_ERR_HIP if the buffer's address cannot be obtained.
 * Sharing: every call on one GPU uses that GPU's one buffer, which keeps the
 * last call's partials (each partial a call reads, the same call writes
 * first, so nothing needs clearing).  Calls ordered on one stream are safe;
 * calls whose work may overlap on the device (several streams, or several
 * threads enqueueing at once) race on the buffer and may return wrong results.
 */
#define PA_DECODE_SCRATCH_BYTES ((size_t)64 << 20)
int pa_decode_attention_noalloc(void* out, const void* query, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t max_context_len, float scale, pa_dtype dtype,
                                int32_t partition_size, void* stream);

/*
 * Partition size (tokens) for the decode kernels on the current device, or a
 * negative pa_status (INVALID_ARG / UNSUPPORTED as pa_decode_attention; HIP if
 * the device cannot be queried).
 *
 * host_context_lens: NULL, or the num_seqs context lengths in HOST memory (a
 * serving scheduler holds them there; they are only read during the call).
 * NULL gives the size pa_decode_attention picks by itself: every sequence is
 * taken to be at max_context_len and partitions stay at most 64 blocks long,
 * so that a ragged batch still balances.  With the lengths the library
 * simulates the launch (its workgroups dealt to the XCDs and list-scheduled
 * onto the resident slots, each costing its blocks plus a fixed setup) for
 * every candidate size up to the partition limit (256 blocks, 1024 for
 * blocks under 16 tokens) and returns the fastest, merge
 * included; the host work is O(num_seqs x partitions) per candidate.
 *
 * The choice depends on the compute-unit count and on how many workgroups of
 * the decode kernel fit one compute unit (two HIP queries, cached per device).
 */
int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                 pa_dtype dtype, const int32_t* host_context_lens);

/*
 * The same choice without a device: `num_cus` compute units holding
 * `workgroups_per_cu` decode workgroups each (both > 0, else INVALID_ARG).
 * For planning on a host, and to test the policy.
 */
int32_t pa_decode_plan_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                      pa_dtype dtype, const int32_t* host_context_lens,
                                      int32_t num_cus, int32_t workgroups_per_cu);

/*
 * Paged attention for several new tokens per sequence: varlen prefill,
 * chunked prefill, and batches mixing prefill chunks with decode steps
 * (handbook "分页 KV Cache", section "分页注意力": context lengths after this
 * step, query_start_loc delimiting each sequence's new tokens, causal mask).
 *
 *   query, out       [num_tokens, num_heads, head_dim]  (dtype; rows packed by sequence)
 *   query_start_loc  int32 [num_seqs + 1], device: sequence b owns rows
 *                    query_start_loc[b] .. query_start_loc[b+1]-1
 *                    (non-decreasing, [0] = 0, [num_seqs] <= num_tokens)
 *   context_lens     int32 [num_seqs], device: L_b, the context INCLUDING the
 *                    n_b new tokens, whose K/V must already be in the pools
 *                    (pa_slot_mapping with query_start_loc, then
 *                    pa_reshape_and_cache); new token i sits at position
 *                    L_b - n_b + i and attends to positions 0 .. L_b - n_b + i.
 *   max_query_len    host bound of n_b; 1 <= max_query_len <= num_tokens.
 *   other arguments  as pa_decode_attention (pools, tables, scale, dtype, stream).
 * fp16 and bf16 run matrix-core tiles shared by the rows of a sequence; fp32
 * runs the fp32 matrix-core column tile, whose columns are the (new token,
 * query head) pairs of one sequence and KV head, each with its own causal
 * key limit, so the rows of a sequence share every K/V read.  Block sizes as
 * pa_decode_attention.
 * partition_size: 0 lets the library choose (it may split long contexts into
 * partitions merged by a second kernel, keeping the partials within 256 MiB),
 * or a size pa_decode_attention_ex accepts.  The workspace
 * must hold pa_prefill_workspace_bytes(...) for the same partition_size (0 when
 * the context fits one partition).  Rows past query_start_loc[num_seqs] are
 * not written.  num_tokens == 0 is allowed and enqueues nothing (pointers may
 * then be NULL).  Device contents are the caller's contract (n_b <= L_b <=
 * max_context_len, n_b <= max_query_len, valid block ids).
 */
int pa_prefill_attention(void* out, const void* query, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                         int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                         int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                         size_t workspace_bytes, int32_t partition_size, void* stream);

/* Workspace bytes pa_prefill_attention needs for this partition_size (0: the
 * most the automatic choice can use); 0 for invalid sizes. */
size_t pa_prefill_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t block_size, int32_t partition_size);

/*
 * Whole-block copies inside both pools: for every i < num_pairs, block
 * dst_blocks[i] of k_pool and of v_pool becomes a copy of block src_blocks[i]
 * (block_size * num_kv_heads * head_dim elements each), the copy-on-write step
 * of a forked sequence that writes into a shared, partly filled block
 * ("KV cache: capacity derivation, paging and reclamation", section on shared
 * prefixes and reference counts).
 *   src_blocks, dst_blocks  int64 [num_pairs], device memory.  The dst ids
 *                           must be distinct and none may be a src id (the
 *                           copies run concurrently); ids outside
 *                           [0, num_blocks) skip their pair.
 * num_pairs = 0 enqueues nothing.  Errors: INVALID_ARG (null pools, null id
 * arrays with num_pairs > 0, non-positive sizes), UNSUPPORTED (dtype), HIP.
 */
int pa_copy_blocks(void* k_pool, void* v_pool, const int64_t* src_blocks, const int64_t* dst_blocks,
                   int64_t num_pairs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                   int64_t num_blocks, pa_dtype dtype, void* stream);

/*
 * Whole-block copies between two pairs of pools of the same block shape:
 * block dst_blocks[i] of (dst_k_pool, dst_v_pool) becomes a copy of block
 * src_blocks[i] of (src_k_pool, src_v_pool).  One pair may live in pinned
 * host memory (hipHostMalloc / a pinned torch tensor, which the device
 * addresses directly): swapping a preempted sequence's blocks out of HBM and
 * back in (handbook "分页 KV Cache", section on scheduling when memory runs
 * short).  Id arrays in device memory; ids outside either pool skip their
 * pair; dst ids distinct.  Errors as pa_copy_blocks (INVALID_ARG also for
 * null source pools or src_num_blocks <= 0).
 */
int pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, int64_t dst_num_blocks, const void* src_k_pool,
                   const void* src_v_pool, int64_t src_num_blocks, const int64_t* src_blocks,
                   const int64_t* dst_blocks, int64_t num_pairs, int32_t block_size, int32_t num_kv_heads,
                   int32_t head_dim, pa_dtype dtype, void* stream);

/*
 * Host-side block pool (host memory only; no HIP call, no device memory).
 * A fixed set of num_blocks physical blocks with a FIFO free queue and a
 * reference count per block (handbook "分页 KV Cache", section "块表与 slot
 * mapping": blocks leave from the head of the free queue, an allocation that
 * cannot be met changes nothing, freed blocks rejoin at the tail), and
 * sequences built on it: an ordered block list and a token count.  A pool and
 * its sequences belong to one thread at a time.
 *
 * pa_block_pool_create: free_order NULL hands blocks out as 0, 1, ...;
 *   otherwise a permutation of 0..num_blocks-1 giving the initial queue.
 *   NULL for invalid arguments or when host memory runs out.
 * pa_block_pool_allocate: n blocks (reference count 1 each) into blocks[0..n),
 *   or NO_BLOCKS and nothing changed.
 * pa_block_pool_free: drops one reference per listed block; a block reaching
 *   zero rejoins the free queue, in list order.  INVALID_ARG (nothing
 *   changed) if an id is out of range or listed more often than referenced.
 * pa_block_pool_num_free / _ref_count: -1 for a NULL pool or an id out of range.
 *
 * pa_seq_create: a new, empty sequence handle (handles are reused after release).
 * pa_seq_fork: a child sharing every block of the parent (one more reference
 *   each) and its token count (parallel sampling, beam search).
 * pa_seq_append: num_tokens more tokens: new blocks as the last one fills; if
 *   the last block is partly filled and shared, it is first replaced by a
 *   fresh block and (*cow_src, *cow_dst) report the pair to copy on the device
 *   (pa_copy_blocks) before writing; otherwise both are -1.  NO_BLOCKS if the
 *   pool cannot supply every block the call needs: nothing changed.
 * pa_seq_release: drops the sequence's references (in block order); the handle
 *   becomes invalid.
 * pa_seq_length: tokens, or -1 for an invalid handle.
 * pa_seq_block_table: the block ids into table[0..*num_blocks); WORKSPACE if
 *   *num_blocks > max_blocks (table untouched, *num_blocks still set).
 */
typedef struct pa_block_pool pa_block_pool;
pa_block_pool* pa_block_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pa_block_pool_destroy(pa_block_pool* pool);
int32_t pa_block_pool_num_free(const pa_block_pool* pool);
int32_t pa_block_pool_ref_count(const pa_block_pool* pool, int32_t block);
int pa_block_pool_allocate(pa_block_pool* pool, int32_t n, int32_t* blocks);
int pa_block_pool_free(pa_block_pool* pool, const int32_t* blocks, int32_t n);
int pa_seq_create(pa_block_pool* pool, int32_t* seq);
int pa_seq_fork(pa_block_pool* pool, int32_t parent, int32_t* child);
int pa_seq_append(pa_block_pool* pool, int32_t seq, int64_t num_tokens, int32_t* cow_src, int32_t* cow_dst);
int pa_seq_release(pa_block_pool* pool, int32_t seq);
int64_t pa_seq_length(const pa_block_pool* pool, int32_t seq);
int pa_seq_block_table(const pa_block_pool* pool, int32_t seq, int32_t* table, int32_t max_blocks,
                       int32_t* num_blocks);

/*
 * Decode with shared prompt prefixes read once per group (cascade): the
 * sequences group_start[g] .. group_start[g+1]-1 (consecutive; the groups
 * cover all num_seqs sequences) share their first prefix_lens[g] tokens -
 * whole blocks, the same ids in every member's table (forks of one prompt,
 * parallel sampling: "KV cache: capacity derivation, paging and reclamation",
 * section on shared prefixes; xxqk.cn PagedAttention article, parallel
 * sampling).  seq_prefix_lens[b] repeats its group's prefix length.
 * With 16-token blocks and fp16/bf16 one launch does it all: a workgroup per
 * (group, KV head, set of members whose query heads fill the 16 matrix-core
 * columns) reads the shared blocks once for the set, then each member's own
 * blocks, its waves splitting those steps and merging their softmax states
 * in LDS.  Otherwise (other block sizes, or more steps per set than four
 * waves' table slices hold) a prefix pass reads each group's prefix blocks
 * once and scores them against every member's query, a suffix pass reads
 * each sequence's blocks past the prefix, and a merge combines the two
 * softmax partials per (sequence, head).  Either way the result equals
 * pa_decode_attention's within rounding.
 *   group_start int32 [num_groups + 1], prefix_lens int32 [num_groups],
 *   seq_prefix_lens int32 [num_seqs]: device memory (pa_shared_prefix_groups
 *   computes them on the host from the tables).
 *   max_group_size, max_prefix_len: host bounds (max_prefix_len a multiple of
 *   block_size, <= max_context_len).
 *   workspace: pa_shared_prefix_workspace_bytes(...) bytes, always needed.
 * fp16 / bf16 only; block sizes as pa_decode_attention.  Errors as
 * pa_decode_attention.
 */
int pa_decode_attention_shared_prefix(void* out, const void* query, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens,
                                      const int32_t* group_start, const int32_t* prefix_lens,
                                      const int32_t* seq_prefix_lens, int32_t num_seqs, int32_t num_groups,
                                      int32_t max_group_size, int32_t num_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                      int32_t max_context_len, int32_t max_prefix_len, float scale,
                                      pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

size_t pa_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t max_prefix_len);

/*
 * The groups of shared prefixes in a decode batch, from HOST copies of the
 * block tables and context lengths: maximal runs of consecutive sequences
 * whose tables share at least min_prefix_blocks leading blocks.  A group's
 * prefix is the whole blocks all members share before any member's last token;
 * a run of one sequence is a group with prefix 0.  Outputs (host, caller
 * allocated): group_start [num_seqs + 1], prefix_lens [num_seqs],
 * seq_prefix_lens [num_seqs], and the counts and bounds the cascade call takes.
 */
int pa_shared_prefix_groups(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t min_prefix_blocks,
                            int32_t* group_start, int32_t* prefix_lens, int32_t* seq_prefix_lens,
                            int32_t* num_groups, int32_t* max_group_size, int32_t* max_prefix_len);

/*
 * Entry points over either pool layout (pa_kv_layout), the shared-prefix
 * decode's among them (declared above with the others).  Each behaves exactly
 * as the entry point of the same name without "_layout" - same arguments,
 * device-content rules and errors - with the pool given by `layout`:
 *   PA_KV_SPLIT  k_pool and v_pool as everywhere else;
 *   PA_KV_FUSED  k_pool = the one pool [num_blocks, num_kv_heads, block_size,
 *                2*head_dim] and v_pool = NULL.
 * INVALID_ARG also for an unknown layout, a NULL v_pool with PA_KV_SPLIT or
 * a non-NULL one with PA_KV_FUSED, or a block over 2 GiB.  A result does not
 * depend on the layout: the kernels read the same rows in the same order.
 */
int pa_reshape_and_cache_layout(const void* key, const void* value, void* k_pool, void* v_pool,
                                const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                                pa_kv_layout layout, void* stream);
int pa_decode_attention_shared_prefix_layout(void* out, const void* query, const void* k_pool, const void* v_pool,
                                             const int32_t* block_tables, const int32_t* context_lens,
                                             const int32_t* group_start, const int32_t* prefix_lens,
                                             const int32_t* seq_prefix_lens, int32_t num_seqs, int32_t num_groups,
                                             int32_t max_group_size, int32_t num_heads, int32_t num_kv_heads,
                                             int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                             int32_t max_context_len, int32_t max_prefix_len, float scale,
                                             pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                             pa_kv_layout layout, void* stream);
int pa_decode_attention_layout(void* out, const void* query, const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                               int32_t max_blocks_per_seq, int32_t max_context_len, float scale, pa_dtype dtype,
                               void* workspace, size_t workspace_bytes, int32_t partition_size,
                               pa_kv_layout layout, void* stream);
int pa_prefill_attention_layout(void* out, const void* query, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens,
                                const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                                float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                int32_t partition_size, pa_kv_layout layout, void* stream);

/*
 * Whole-block copies between two pools of any layouts: block dst_blocks[i] of
 * the destination gets the K and V rows of block src_blocks[i] of the source,
 * rearranged when the layouts differ (HB, "源码对照": attention backends
 * differ in KV layout, so moving KV between them converts it).  Pools as in
 * the _layout entry points; either may be pinned host memory (as for
 * pa_swap_blocks); the block shape (block_size, num_kv_heads, head_dim, dtype)
 * is shared.  Same layouts: a plain whole-block copy (copy-on-write or swap of
 * a fused pool).  Id arrays int64 in device memory; a pair with an id outside
 * its pool is skipped; destination ids distinct; source and destination
 * blocks must not overlap.  num_pairs = 0 enqueues nothing.
 * Errors: INVALID_ARG (pool pointers not matching their layouts, unknown
 * layouts, null id arrays with num_pairs > 0, non-positive sizes),
 * UNSUPPORTED (dtype), HIP.
 */
int pa_convert_blocks(void* dst_k_pool, void* dst_v_pool, pa_kv_layout dst_layout, int64_t dst_num_blocks,
                      const void* src_k_pool, const void* src_v_pool, pa_kv_layout src_layout,
                      int64_t src_num_blocks, const int64_t* src_blocks, const int64_t* dst_blocks,
                      int64_t num_pairs, int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                      pa_dtype dtype, void* stream);

/*
 * pa_write_new_tokens - the slot mapping and the pool write of one decode
 * step in one launch.
 *
 * Sequence b's new token is the last position of its context, p =
 * context_lens[b] - 1 (HB, "分页注意力"); its slot is
 * block_tables[b][p / block_size] * block_size + p % block_size (HB, "块表与
 * slot mapping"), and its K and V rows key[b], value[b] are copied bit for bit
 * into that slot of the pools (HB, "实现", PagedKVCache.write): the result of
 * pa_slot_mapping (query_start_loc NULL) followed by pa_reshape_and_cache_layout.
 *
 *   key, value      [num_seqs, num_kv_heads, head_dim], dtype
 *   k_pool, v_pool  pools of `layout` with num_blocks blocks (v_pool NULL
 *                   for PA_KV_FUSED)
 *   block_tables    int32 [num_seqs, max_blocks_per_seq]
 *   context_lens    int32 [num_seqs], each including the new token
 *   slot_mapping    out, int64 [num_seqs], or NULL when the caller does not
 *                   need the slots
 *
 * Device contents: as pa_slot_mapping and pa_reshape_and_cache - a context
 * of 0 tokens or a logical block >= max_blocks_per_seq gives slot -1, and a
 * slot outside the pool writes nothing; each new token's slot must be its
 * sequence's own.  Errors: INVALID_ARG for null pointers or non-positive
 * sizes, UNSUPPORTED for an unknown dtype, HIP.  num_seqs == 0 enqueues
 * nothing.
 */
int pa_write_new_tokens(const void* key, const void* value, void* k_pool, void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, int64_t* slot_mapping,
                        int32_t num_seqs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                        int32_t max_blocks_per_seq, int64_t num_blocks, pa_dtype dtype,
                        pa_kv_layout layout, void* stream);

/*
 * pa_decode_step - a whole decode step: pa_write_new_tokens, then
 * pa_decode_attention_layout over the contexts that now include the new
 * tokens (two launches, three when a context is split into partitions).
 * Arguments as those two calls take them; workspace >=
 * pa_decode_workspace_bytes_ex(..., partition_size) (with partition_size 0,
 * pa_decode_workspace_bytes).  Every argument check of both calls runs
 * before anything is enqueued, so a rejected step writes nothing.
 */
int pa_decode_step(void* out, const void* query, const void* key, const void* value, void* k_pool,
                   void* v_pool, const int32_t* block_tables, const int32_t* context_lens,
                   int64_t* slot_mapping, int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                   int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int64_t num_blocks,
                   int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                   size_t workspace_bytes, int32_t partition_size, pa_kv_layout layout, void* stream);

/*
 * Measurement: a streaming read of `bytes` bytes of device memory at `src`
 * (16-byte aligned, bytes a multiple of 16), each byte loaded once in 16-byte
 * vector loads spread over the whole device, non-temporal if `nontemporal` is
 * non-zero.  The rate a plain linear read reaches on this device: the ceiling
 * the decode kernel's KV-read bandwidth (each context token's K and V rows
 * read once, handbook "分页 KV Cache", section on paged attention) is
 * compared against besides the published HBM peak.  Nothing is written
 * unless the XOR of the words one thread reads equals 0x5a17c0de; then that
 * value goes to `sink` (4 bytes, device, caller owned).  Errors: INVALID_ARG
 * (null pointers, misaligned or zero size), HIP (launch failure).
 */
int pa_stream_read(const void* src, size_t bytes, void* sink, int nontemporal, void* stream);

/* Static, human-readable name of a pa_status value. */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
