// libpa kernels for gfx950 (CDNA4) and the extern "C" entry points of pa.h.
//
//  * slot mapping      - slot of each new token from its block table
//                        (handbook "分页 KV Cache", section "块表与 slot mapping")
//  * reshape_and_cache - bit copy of each new token's K/V row into its slot
//                        (same page, section "实现", PagedKVCache.write)
//  * decode_partition  - paged decode attention over one partition of a
//                        sequence's context for one KV head and its group of
//                        query heads: block-table lookups on chip, 16-byte
//                        coalesced row loads, QK with DPP lane reductions,
//                        online softmax and the P.V accumulation in float32
//                        (same page, section "分页注意力"; aiqz.cc
//                        "paged-attention", section "工程实现要点": per-block
//                        pieces merged by the online-softmax rescaling)
//  * combine           - merge of the partitions' (max, sum, acc) partials
//
// Wave64 throughout.  A token row of one KV head is head_dim * elem bytes
// (256 B for D=128 16-bit); LPR lanes cover it with one 16-byte load each,
// so one load instruction of a wave reads RPI = 64 / LPR whole rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "pa.h"
#include "pa_device.h"
#include "pa_host.h"
#include "pa_runtime.h"

namespace {

// ------------------------------------------------------------------ slot mapping

__device__ __forceinline__ int64_t slot_of(const int32_t* table, int max_blocks, int block_size, int pos) {
  if (pos < 0) return -1;
  const int lb = pos / block_size;
  if (lb >= max_blocks) return -1;
  return (int64_t)table[lb] * block_size + pos % block_size;
}

__global__ void slot_mapping_decode_kernel(int64_t* __restrict__ slots, const int32_t* __restrict__ tables,
                                           const int32_t* __restrict__ lens, int num_seqs, int max_blocks,
                                           int block_size) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= num_seqs) return;
  slots[b] = slot_of(tables + (size_t)b * max_blocks, max_blocks, block_size, lens[b] - 1);
}

__global__ void slot_mapping_varlen_kernel(int64_t* __restrict__ slots, const int32_t* __restrict__ tables,
                                           const int32_t* __restrict__ lens, const int32_t* __restrict__ qsl,
                                           int max_blocks, int block_size, int64_t num_tokens) {
  const int b = blockIdx.x;
  const int s0 = qsl[b], s1 = qsl[b + 1];
  const int n = s1 - s0;
  const int L = lens[b];
  const int32_t* table = tables + (size_t)b * max_blocks;
  for (int t = threadIdx.x; t < n; t += blockDim.x) {
    const int64_t dst = (int64_t)s0 + t;
    if (dst < 0 || dst >= num_tokens) continue;
    slots[dst] = slot_of(table, max_blocks, block_size, L - n + t);
  }
}

// ------------------------------------------------------------------ pool write

// One workgroup per (token, K or V).  Strides in units of V: the head rows
// of a token are head_vecs apart in key/value and head_stride apart in the
// pool (contiguous in the split layout, a block's head planes apart in the
// fused one).
template <typename V>
__global__ void reshape_and_cache_kernel(const V* __restrict__ key, const V* __restrict__ value,
                                         V* __restrict__ k_pool, V* __restrict__ v_pool,
                                         const int64_t* __restrict__ slots, int head_vecs, int num_kv_heads,
                                         int block_size, int64_t block_stride, int64_t row_stride,
                                         int64_t head_stride, int64_t num_slots) {
  const int64_t i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int row_vecs = head_vecs * num_kv_heads;
  const V* src = (blockIdx.y == 0 ? key : value) + i * row_vecs;
  V* dst = (blockIdx.y == 0 ? k_pool : v_pool) + (slot / block_size) * block_stride + (slot % block_size) * row_stride;
  for (int t = threadIdx.x; t < row_vecs; t += blockDim.x) {
    const int h = t / head_vecs;
    dst[h * head_stride + (t - h * head_vecs)] = src[t];
  }
}

// ------------------------------------------------------------------ decode attention

struct DecodeArgs {
  void* out;
  const void* query;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_acc;   // [B, H, P, D]
  float2* ws_ml;   // [B, H, P] (running max in log2 units, softmax denominator)
  int num_heads, num_kv_heads, rep, chunks, max_blocks_per_seq;
  int block_shift;  // pool blocks of 16 << block_shift tokens (the MFMA tile's steps are 16 tokens)
  int part_tokens, num_parts, groups;  // groups = head-group workgroups per (sequence, partition)
  float qscale;    // scale * log2(e): scores come out in log2 units for exp2
  // pool geometry in bytes (layout): K row (block p, token t, head h) at
  // k_pool + p*block_stride + t*row_stride + h*head_stride, V likewise;
  // span = what one 16-token step of a block may touch from its first byte
  int64_t block_stride;
  uint32_t row_stride, head_stride, span;
  // Column mode (VALU kernel only): non-null query_start_loc [num_seqs + 1]
  // makes the columns of a (sequence, KV head) its (new token, query head)
  // pairs - new token i of sequence b at position L_b - n_b + i sees keys
  // [0, L_b - n_b + i] - instead of the query heads of one decode query;
  // ctiles workgroups of wpw waves per (sequence, KV head, partition) cover
  // them, REPC columns per wave.
  const int32_t* query_start_loc;
  int num_seqs, ctiles;
};

template <int DT, int D, int REPC>
struct DecodeTile {
  static constexpr int BS = pa::kBlockSize;
  static constexpr int EB = ElemBytes<DT>::value;
  static constexpr int ROWB = D * EB;    // one KV head's row of one token
  static constexpr int LPR = ROWB / 16;  // lanes per row
  static constexpr int RPI = 64 / LPR;   // rows per load instruction
  static constexpr int NLD = BS / RPI;   // load instructions per block (K or V)
  static constexpr int EPL = 16 / EB;    // elements per lane and row
  static_assert(LPR >= 8 && LPR <= 32 && BS % RPI == 0, "tile shape");
};

// One wave = REPC columns of one (sequence b, partition s, KV head g): in
// decode, a chunk of the query heads g serves; in column mode, consecutive
// (new token, query head) pairs of a varlen batch, each with its own causal
// key limit, so the rows of a sequence share every K/V read of the wave.
// The wave walks the partition in steps of 16 tokens.  Lane l reads, for
// every step, rows i*RPI + l/LPR (i < NLD), bytes (l % LPR)*16 .. +16 of the
// row.  Each lane runs its own online softmax over the tokens it holds (all
// LPR lanes of a row group hold the same tokens and compute identical
// values); the RPI row-group streams merge at the end.
// Pool block sizes (MODE, as in the matrix-core tile below): a 16-token block
// is one step; a larger block is walked in 16-row windows (table entry
// step >> shift); for a smaller one every row's block comes from the
// partition's table staged in LDS (step j, row t: entry (j << shift) +
// t / block_size, row t % block_size of that block).
template <int DT, int D, int REPC, int MODE>
__global__ __launch_bounds__(256) void decode_partition_kernel(const DecodeArgs a) {
  using T = DecodeTile<DT, D, REPC>;
  constexpr int BS = T::BS, ROWB = T::ROWB, LPR = T::LPR, RPI = T::RPI, NLD = T::NLD, EPL = T::EPL;
  constexpr bool SUB = MODE == kBlocksLarge;
  constexpr bool GATHER = MODE == kBlocksSmall;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wpw = blockDim.x >> 6;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int r = lane / LPR, c = lane % LPR;

  // This wave's columns: the output row (query row * H + query head) and the
  // number of context keys each sees; wg_lim bounds the keys of every wave
  // of the workgroup (they share b and s, and so the block-table range).
  int b, g, s, wg_lim;
  size_t qrow[REPC];
  int lim[REPC];
  bool live[REPC];
  if (!a.query_start_loc) {  // decode: the query heads of KV head g, one query row
    const int grp = logical % a.groups;
    const int seq_part = logical / a.groups;
    s = seq_part % a.num_parts;
    b = seq_part / a.num_parts;
    const int unit = grp * wpw + wave;
    g = unit / a.chunks;
    const int h0 = g * a.rep + (unit % a.chunks) * REPC;
    wg_lim = a.context_lens[b];
#pragma unroll
    for (int h = 0; h < REPC; ++h) {
      qrow[h] = (size_t)b * a.num_heads + h0 + h;
      lim[h] = wg_lim;
      live[h] = true;
    }
  } else {  // column mode: (new token, query head) pairs, ctile fastest so they share K/V in L2
    const int ct = logical % a.ctiles;
    int rest = logical / a.ctiles;
    s = rest % a.num_parts;
    rest /= a.num_parts;
    g = rest % a.num_kv_heads;
    b = rest / a.num_kv_heads;
    const int q0 = a.query_start_loc[b], n = a.query_start_loc[b + 1] - q0;
    const int L = a.context_lens[b];
    const int cols = n * a.rep;
    if (ct * wpw * REPC >= cols) return;  // workgroup-uniform: no column of this sequence here
    const int c0 = (ct * wpw + wave) * REPC;
    wg_lim = L - n + (min(cols, (ct + 1) * wpw * REPC) - 1) / a.rep + 1;
#pragma unroll
    for (int h = 0; h < REPC; ++h) {
      const int cc = c0 + h, ti = cc / a.rep;
      live[h] = cc < cols;
      qrow[h] = (size_t)(q0 + (live[h] ? ti : 0)) * a.num_heads + g * a.rep + cc % a.rep;
      lim[h] = live[h] ? L - n + ti + 1 : 0;
    }
  }
  int wlim = 0, lim_min = 1 << 30;  // this wave's key range, and where its masks start
#pragma unroll
  for (int h = 0; h < REPC; ++h)
    if (live[h]) {
      wlim = max(wlim, lim[h]);
      lim_min = min(lim_min, lim[h]);
    }

  const int start = s * a.part_tokens;
  const int wg_end = min(wg_lim, start + a.part_tokens);
  if (start >= wg_end) {  // workgroup-uniform
    if (!a.query_start_loc && s == 0 && r == 0) {  // decode, empty context: zeros
      float z[EPL] = {};
      for (int h = 0; h < REPC; ++h) store_row<DT, EPL>((uint8_t*)a.out + qrow[h] * ROWB + c * 16, z);
    }
    return;
  }
  const int pshift = MODE != kBlocks16 ? a.block_shift : 0;
  const int pool_bs = SUB ? BS << pshift : GATHER ? BS >> pshift : BS;  // tokens per pool block
  const int blk0 = start / pool_bs;  // partitions start on a pool block
  const int nent = (wg_end - start + pool_bs - 1) / pool_bs;  // table entries the workgroup reads

  // This partition's block-table slice: in VGPR lanes, fetched per step by
  // readlane (blocks of 16 tokens or more, <= kMaxPartitionBlocks entries),
  // or staged in LDS for the workgroup and read per row (smaller blocks,
  // <= kMaxSmallBlockPartition entries; every wave of the workgroup serves
  // the same sequence and partition).
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk0;
  TableSlice tab;
  __shared__ int32_t stab[GATHER ? pa::kMaxSmallBlockPartition : 1];
  if constexpr (GATHER)
    stage_table(stab, bt, nent);
  else
    tab.load(bt, nent, lane);

  const int end = min(wlim, start + a.part_tokens);  // this wave's keys
  if (start >= end) return;  // no key of this wave's columns here (no barrier follows)
  const int nblk = (end - start + BS - 1) / BS;  // 16-token steps

  // Query rows of the REPC columns, scaled into log2 units.
  float q[REPC][EPL];
#pragma unroll
  for (int h = 0; h < REPC; ++h) {
    unpack16<DT>(*reinterpret_cast<const uint4*>((const uint8_t*)a.query + qrow[h] * ROWB + c * 16), q[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) q[h][e] *= a.qscale;
  }

  const size_t row_stride = a.row_stride;
  const size_t block_stride = (size_t)a.block_stride;
  const size_t lane_off = (size_t)r * row_stride + (size_t)g * a.head_stride + (size_t)c * 16;
  const uint8_t* kbase = a.k_pool + lane_off;
  const uint8_t* vbase = a.v_pool + lane_off;
  // Small blocks: row i*RPI + r of a step lies in the step's block blk[i],
  // at byte offset in[i] of that block.
  int sblk[GATHER ? NLD : 1];
  size_t sin[GATHER ? NLD : 1];
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int t = i * RPI + r;
      sblk[i] = t / pool_bs;
      sin[i] = (size_t)(t % pool_bs) * row_stride + (size_t)g * a.head_stride + (size_t)c * 16;
    }
  }

  float m[REPC], l[REPC], acc[REPC][EPL];
#pragma unroll
  for (int h = 0; h < REPC; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  // K streams non-temporal in decode, as in the matrix-core tile (fp32
  // 256 x 4096: 1425 -> 1298 us): each K row is read by one wave.  In column
  // mode the waves of a workgroup read the same rows together, so K keeps the
  // default policy and the later waves find it in the caches.
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const bool k_once = a.query_start_loc == nullptr;
  auto load_k = [&](const uint8_t* p) -> uint4 {
    if (k_once) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
    return *reinterpret_cast<const uint4*>(p);
  };
  auto load_block = [&](int j, uint4* kr, uint4* vr) {
    if constexpr (GATHER) {  // per-row blocks; rows past the partition re-read its last block (masked)
      size_t base[NLD];
      step_block_bases<NLD>(stab, j, pshift, nent, block_stride, sblk, base);
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        kr[i] = load_k(a.k_pool + base[i] + sin[i]);
        vr[i] = *reinterpret_cast<const uint4*>(a.v_pool + base[i] + sin[i]);
      }
      return;
    }
    const size_t off = SUB ? (size_t)(uint32_t)tab.get(j >> pshift) * block_stride +
                                 (size_t)(j & ((1 << pshift) - 1)) * BS * row_stride
                           : (size_t)(uint32_t)tab.get(j) * block_stride;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kr[i] = load_k(kbase + off + (size_t)i * RPI * row_stride);
      vr[i] = *reinterpret_cast<const uint4*>(vbase + off + (size_t)i * RPI * row_stride);
    }
  };

  // One step whose first key is tok0: keys at or past a column's limit get
  // score -inf and weight 0 (rows past the wave's last key, stale or NaN,
  // are zeroed before they reach the sums); steps below every limit skip the
  // masks.
  auto process = [&](const uint4* kr, const uint4* vr, int tok0) {
    float sc[NLD][REPC];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      float kf[EPL];
      unpack16<DT>(kr[i], kf);
#pragma unroll
      for (int h = 0; h < REPC; ++h) {
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) part = fmaf(q[h][e], kf[e], part);
        sc[i][h] = group_sum<LPR>(part);
      }
    }
    const bool partial = tok0 + BS > lim_min;
    if (partial) {
#pragma unroll
      for (int i = 0; i < NLD; ++i)
#pragma unroll
        for (int h = 0; h < REPC; ++h)
          if (tok0 + i * RPI + r >= lim[h]) sc[i][h] = -INFINITY;
    }
#pragma unroll
    for (int h = 0; h < REPC; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int i = 1; i < NLD; ++i) bm = fmaxf(bm, sc[i][h]);
      const float mn = fmaxf(m[h], bm);
      if (mn > m[h]) {
        const float alpha = fast_exp2(m[h] - mn);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int key = tok0 + i * RPI + r;
      float vf[EPL];
      unpack16<DT>(vr[i], vf);
      if (partial && key >= end) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;
      }
#pragma unroll
      for (int h = 0; h < REPC; ++h) {
        const bool ok = !partial || key < lim[h];
        const float p = ok ? fast_exp2(sc[i][h] - m[h]) : 0.f;
        l[h] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  };

  // Two register buffers: the next block's loads are in flight while the
  // current block is computed.
  uint4 ka[NLD], va[NLD], kb[NLD], vb[NLD];
  load_block(0, ka, va);
  for (int j = 0; j < nblk; j += 2) {
    if (j + 1 < nblk) load_block(j + 1, kb, vb);
    process(ka, va, start + j * BS);
    if (j + 1 >= nblk) break;
    if (j + 2 < nblk) load_block(j + 2, ka, va);
    process(kb, vb, start + (j + 1) * BS);
  }

  // Merge the RPI row-group streams.
#pragma unroll
  for (int h = 0; h < REPC; ++h) {
    const float M = across_groups_max<LPR>(m[h]);
    const float f = (m[h] == -INFINITY) ? 0.f : fast_exp2(m[h] - M);
    l[h] = across_groups_sum<LPR>(l[h] * f);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = across_groups_sum<LPR>(acc[h][e] * f);
    m[h] = M;
  }
  if (r != 0) return;

  // A column whose keys fit one partition writes its output row; the others
  // leave partials for the merge (none in a partition past their keys).
#pragma unroll
  for (int h = 0; h < REPC; ++h) {
    const int col_parts = (lim[h] + a.part_tokens - 1) / a.part_tokens;
    if (!live[h] || s >= col_parts) continue;
    if (col_parts == 1) {
      const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = acc[h][e] * inv;
      store_row<DT, EPL>((uint8_t*)a.out + qrow[h] * ROWB + c * 16, o);
    } else {
      const size_t idx = qrow[h] * a.num_parts + s;
      float* dst = a.ws_acc + idx * D + c * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4)
        *reinterpret_cast<float4*>(dst + e) = make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
      if (c == 0) a.ws_ml[idx] = make_float2(m[h], l[h]);
    }
  }
}

// ------------------------------------------------------------------ fp32 matrix-core column tile
//
// Column mode in fp32 on the matrix cores (mfma_f32_16x16x4_f32): a wave
// takes 16 columns - (new token, query head) pairs of one (sequence, KV head),
// each with its own causal key limit - so that each fp32 K/V element it loads
// serves 16 columns through the matrix core instead of the VALU.  Per 16-token
// step, lane l = 16 gq + c (c = l % 16):
//  * QK: S[key][column] over D/4 MFMAs.  Lane l holds K row c and the query
//    of column c at dims 16i + 4gq .. +4 (load i), so MFMA 4i + j contracts
//    dim 16i + 4gq + j: a permutation of the dims, the same on both sides.
//    The scores come back as lane l = (gq, c): keys 4gq + r (r = 0..3) of
//    column c.
//  * P.V: O^T[dim][column] over 4 x D/16 MFMAs.  MFMA (r, t) contracts keys
//    4k + r (k = 0..3, the lane group), so the lane's own weight r is its B
//    operand; lane l holds V rows 4gq + r at dims (D/16) c .. +D/16 as the A
//    operand of tiles t = 0..D/16-1.  Tile t, register i of lane (gq, c) is
//    dim (D/16)(4gq + i) + t of column c: a lane owns D/4 consecutive dims.
// Softmax as the 16-bit decode tile: the running max uniform over the four
// lane groups of a column, partial denominators summed at the end.
template <int D, int MODE>
__global__ __launch_bounds__(256) void columns_f32_mfma_kernel(const DecodeArgs a) {
  constexpr int BS = pa::kBlockSize;
  constexpr int ROWB = D * 4;
  constexpr int NKL = D / 16;  // K loads (float4) per lane and step; QK MFMAs = 4 NKL
  constexpr int DV = D / 16;   // dims per lane of one V row (V floats), P.V tiles
  constexpr int NVL = DV / 4;  // float4 loads per V row
  constexpr int DPL = D / 4;   // output dims per lane
  constexpr bool SUB = MODE == kBlocksLarge;
  constexpr bool GATHER = MODE == kBlocksSmall;
  using f4 = f32x4;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wpw = blockDim.x >> 6;
  const int gq = lane >> 4, c = lane & 15;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int ct = logical % a.ctiles;
  int rest = logical / a.ctiles;
  const int s = rest % a.num_parts;
  rest /= a.num_parts;
  const int g = rest % a.num_kv_heads;
  const int b = rest / a.num_kv_heads;
  const int q0 = a.query_start_loc[b], n = a.query_start_loc[b + 1] - q0;
  const int L = a.context_lens[b];
  const int cols = n * a.rep;
  if (ct * wpw * 16 >= cols) return;  // workgroup-uniform: no column of this sequence here
  const int wg_lim = L - n + (min(cols, (ct + 1) * wpw * 16) - 1) / a.rep + 1;
  const int c0 = (ct * wpw + wave) * 16;
  // this lane's column (c) and the wave's last live column
  const int cc = c0 + c, ti = cc / a.rep;
  const bool live = cc < cols;
  const size_t qrow = (size_t)(q0 + (live ? ti : 0)) * a.num_heads + g * a.rep + cc % a.rep;
  const int lim = live ? L - n + ti + 1 : 0;
  const int last_col = min(cols, c0 + 16) - 1;
  const int wlim = c0 < cols ? L - n + last_col / a.rep + 1 : 0;  // limits grow with the column
  const int lim_min = c0 < cols ? L - n + c0 / a.rep + 1 : 0;

  const int start = s * a.part_tokens;
  const int wg_end = min(wg_lim, start + a.part_tokens);
  if (start >= wg_end) return;  // workgroup-uniform
  const int pshift = MODE != kBlocks16 ? a.block_shift : 0;
  const int pool_bs = SUB ? BS << pshift : GATHER ? BS >> pshift : BS;
  const int blk0 = start / pool_bs;
  const int nent = (wg_end - start + pool_bs - 1) / pool_bs;
  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk0;
  TableSlice tab;
  __shared__ int32_t stab[GATHER ? pa::kMaxSmallBlockPartition : 1];
  if constexpr (GATHER)
    stage_table(stab, bt, nent);
  else
    tab.load(bt, nent, lane);
  const int end = min(wlim, start + a.part_tokens);  // this wave's keys
  if (start >= end) return;  // no barrier follows
  const int nblk = (end - start + BS - 1) / BS;

  // The query of column c at dims 16i + 4gq .. +4, scaled into log2 units.
  f4 qv[NKL];
  {
    const float* qp = (const float*)a.query + qrow * D + 4 * gq;
#pragma unroll
    for (int i = 0; i < NKL; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(qp + 16 * i);
      qv[i] = live ? f4{v.x * a.qscale, v.y * a.qscale, v.z * a.qscale, v.w * a.qscale} : f4{0.f, 0.f, 0.f, 0.f};
    }
  }

  // Byte offsets inside a block: K row c, V rows 4gq + r.
  const size_t row_stride = a.row_stride, block_stride = (size_t)a.block_stride;
  const size_t hoff = (size_t)g * a.head_stride;
  const size_t kin = hoff + (size_t)4 * gq * 4;
  const size_t vin = hoff + (size_t)DV * c * 4;
  // where a row of step j lies: (table entry, row inside its block)
  auto row_addr = [&](int j, int t) -> size_t {
    if constexpr (GATHER) {
      const int e = min((j << pshift) + t / pool_bs, nent - 1);
      return (size_t)(uint32_t)stab[e] * block_stride + (size_t)(t % pool_bs) * row_stride;
    } else if constexpr (SUB) {
      return (size_t)(uint32_t)tab.get(j >> pshift) * block_stride +
             ((size_t)(j & ((1 << pshift) - 1)) * BS + t) * row_stride;
    } else {
      return (size_t)(uint32_t)tab.get(j) * block_stride + (size_t)t * row_stride;
    }
  };
  auto load_step = [&](int j, f4* kr, f4* vr) {
    const uint8_t* kp = a.k_pool + row_addr(j, c) + kin;
#pragma unroll
    for (int i = 0; i < NKL; ++i) kr[i] = *reinterpret_cast<const f4*>(kp + 64 * i);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint8_t* vp = a.v_pool + row_addr(j, 4 * gq + r) + vin;
#pragma unroll
      for (int h = 0; h < NVL; ++h) vr[r * NVL + h] = *reinterpret_cast<const f4*>(vp + 16 * h);
    }
  };

  f4 acc[DV];
#pragma unroll
  for (int t = 0; t < DV; ++t) acc[t] = f4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  auto process = [&](const f4* kr, const f4* vr, int tok0) {
    // Four independent accumulation chains (dims 16i + 4gq + j, one chain per
    // j) summed in pairs at the end: the MFMAs need not wait on each other,
    // and each fp32 sum runs over a quarter of the products.
    f4 sp[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < NKL; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sp[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(kr[i][j], qv[i][j], sp[j], 0, 0, 0);
    const f4 sacc = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    const bool partial = tok0 + BS > lim_min;
    float sc[4];
    bool ok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      ok[r] = !partial || tok0 + 4 * gq + r < lim;
      sc[r] = ok[r] ? sacc[r] : -INFINITY;
    }
    const float mn = fmaxf(m, rows_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]))));
    const float alpha = mn == -INFINITY ? 1.f : fast_exp2(m - mn);
    m = mn;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = ok[r] ? fast_exp2(sc[r] - mn) : 0.f;
    l = fmaf(l, alpha, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
    for (int t = 0; t < DV; ++t) acc[t] *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // rows past the wave's last key (stale, even NaN) must not reach the MFMA
      const bool vok = !partial || tok0 + 4 * gq + r < end;
#pragma unroll
      for (int t = 0; t < DV; ++t) {
        const float v = vok ? vr[r * NVL + t / 4][t % 4] : 0.f;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(v, p[r], acc[t], 0, 0, 0);
      }
    }
  };

  f4 ka[NKL], va[4 * NVL], kb[NKL], vb[4 * NVL];
  load_step(0, ka, va);
  for (int j = 0; j < nblk; j += 2) {
    if (j + 1 < nblk) load_step(j + 1, kb, vb);
    process(ka, va, start + j * BS);
    if (j + 1 >= nblk) break;
    if (j + 2 < nblk) load_step(j + 2, ka, va);
    process(kb, vb, start + (j + 1) * BS);
  }

  const float lt = rows_sum(l);
  if (!live) return;
  // lane (gq, c) holds dims (D/16)(4gq + i) + t, i.e. D/4 consecutive dims from 4 (D/16) gq
  float o[DPL];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < DV; ++t) o[DV * i + t] = acc[t][i];
  const int col_parts = (lim + a.part_tokens - 1) / a.part_tokens;
  if (s >= col_parts) return;
  if (col_parts == 1) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) o[e] *= inv;
    store_row<DT_F32, DPL>((uint8_t*)a.out + qrow * ROWB + (size_t)DPL * gq * 4, o);
  } else {
    const size_t idx = qrow * a.num_parts + s;
    float* dst = a.ws_acc + idx * D + DPL * gq;
#pragma unroll
    for (int e = 0; e < DPL; e += 4) *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
    if (gq == 0) a.ws_ml[idx] = make_float2(m, lt);
  }
}

// ------------------------------------------------------------------ MFMA decode (16-bit K/V)
//
// The query-head group of one KV head against a 16-token block is a small
// dense contraction, done on the matrix cores:
//   QK:  S[token][head]  = K[16 x D] . Q^T[D x 16]     mfma_f32_16x16x32 (D/32 of them)
//   PV:  O^T[dim][head] += V^T[16dims x 16] . P^T      mfma_f32_16x16x16 (D/16 of them)
// Heads occupy the 16 MFMA columns (a group of up to 16 query heads; unused
// columns hold zeros).  Lane l = 16*gq + col.
//  * K is loaded straight into the QK A-operand layout: lane l holds 16 bytes
//    (dims 32c + 8gq ..+8) of MFMA row col, and row col is token
//    4*(col%4) + col/4.  With that row order the score tile comes back as
//    lane (gq, head col) holding tokens 4i + gq in register i, which is the
//    PV B operand in place (k = 4gq + i <-> token 4i + gq, n = head col).
//  * V is loaded row-coalesced: load i gives lane l token 4i + gq, dims
//    (D/16)*col .. +D/16.  Element t of the four loads, paired by v_perm, is
//    the PV A operand of tile t (row col <-> dim (D/16)*col + t).
//  * Accumulator tile t: lane (gq, col) register r = O[head col][dim
//    (D/16)*(4gq + r) + t]; a lane owns dims 4*(D/16)*gq .. +4*(D/16) of its
//    head, so the softmax rescale factor of a head is lane-local.
// The running max of a head is kept uniform over the four row groups (a
// permlane max per block); denominators are per-lane partial sums.

// Pool block sizes (the MFMA tile always takes 16-token steps):
//  * kBlocks16: blocks and steps coincide;
//  * kBlocksLarge: blocks of 16 << a.block_shift tokens; a step is a window of
//    16 rows inside one block (table entry step >> shift, row offset
//    16 * (step & mask));
//  * kBlocksSmall: blocks of 16 >> a.block_shift tokens; a step's 16 rows
//    come from 1 << shift blocks, so every lane addresses its own row's block
//    (direct-to-LDS and V loads from per-lane global addresses).

template <int DT, int D, int NBUF, int WPW, int MODE>
__global__ __launch_bounds__(64 * WPW) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr bool SUB = MODE == kBlocksLarge;
  constexpr bool GATHER = MODE == kBlocksSmall;
  using Ops = MfmaOps<DT>;
  constexpr int BS = pa::kBlockSize;
  constexpr int ROWB = D * 2;
  constexpr int NKC = D / 32;  // QK k-chunks
  constexpr int VPL = D / 16;  // V elements per lane and row = PV output tiles
  constexpr int DPL = 4 * VPL; // output dims owned by a lane
  constexpr int CPR = ROWB / 16;  // 16-byte chunks per K row
  constexpr int NLI = BS * CPR / 64;  // K load instructions per block
  constexpr int KBYTES = BS * ROWB;   // one K block of one head
  using VT = typename VRow<VPL>::T;
  auto kswz = [](int t) { return kswz_t<CPR>(t); };
  static_assert(BS == 16, "the MFMA tiling assumes 16-token blocks");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = logical % a.groups;
  const int seq_part = logical / a.groups;
  const int s = seq_part % a.num_parts;
  const int b = seq_part / a.num_parts;
  const int unit = grp * WPW + wave;
  const int g = unit / a.chunks;
  const int repc = a.rep / a.chunks;
  const int h0 = g * a.rep + (unit % a.chunks) * repc;
  const int gq = lane >> 4, col = lane & 15;
  const bool live = col < repc;  // this lane's column is a real query head
  uint8_t* const out_row = (uint8_t*)a.out + ((size_t)b * a.num_heads + h0 + (live ? col : 0)) * ROWB + gq * DPL * 2;

  const int L = a.context_lens[b];
  const int start = s * a.part_tokens;
  if (start >= L) {
    if (s == 0 && live) {  // empty context: zeros
      float z[DPL] = {};
      store_row<DT, DPL>(out_row, z);
    }
    return;
  }
  const int end = min(L, start + a.part_tokens);
  const int seq_parts = (L + a.part_tokens - 1) / a.part_tokens;
  const int pshift = MODE != kBlocks16 ? a.block_shift : 0;
  const int pool_bs = SUB ? BS << pshift : GATHER ? BS >> pshift : BS;  // tokens per pool block
  const int blk0 = start / pool_bs;  // partitions start on a pool block
  const int nblk = (end - start + BS - 1) / BS;  // 16-token steps
  // table entries: 1..kMaxPartitionBlocks (kMaxSmallBlockPartition for small blocks)
  const int nent = MODE == kBlocks16 ? nblk : (end - start + pool_bs - 1) / pool_bs;
  const int last = nblk - 1;

  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq + blk0;
  // Blocks of 16 tokens or more: the partition's table slice in VGPR lanes,
  // read per block with readlane.  Small blocks (up to 1024 entries per
  // partition): the table in LDS, shared by the workgroup's waves (they all
  // serve the same sequence and partition), read per row by each lane.
  TableSlice tab;
  __shared__ int32_t stab[GATHER ? pa::kMaxSmallBlockPartition : 1];
  if constexpr (GATHER)
    stage_table(stab, bt, nent);
  else
    tab.load(bt, nent, lane);

  // Q^T as the QK B operand: column col = head h0 + col, k-chunk c = dims 32c + 8gq .. +8.
  uint4 qop[NKC];
  {
    const uint8_t* qp = (const uint8_t*)a.query + ((size_t)b * a.num_heads + h0 + (live ? col : 0)) * ROWB + gq * 16;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + c * 64);
      qop[c] = live ? v : make_uint4(0, 0, 0, 0);
    }
  }

  // Byte offsets inside one block (< 2^32).
  //  K: direct-to-LDS loads, NLI instructions of whole rows; load n, lane l fills
  //     LDS slot 64n + l = (token t, position q) with the row's 16-byte chunk
  //     q ^ f(t), so the row-order MFMA reads below hit 16 distinct bank groups.
  //  V: row-coalesced into registers, row gq (+4i).
  const uint32_t row_stride = a.row_stride;
  const uint32_t hoff = (uint32_t)g * a.head_stride;
  const size_t step_stride = (size_t)BS * row_stride;  // 16-token steps inside a larger block
  uint32_t kdma[NLI];
#pragma unroll
  for (int n = 0; n < NLI; ++n) {
    const int slot = 64 * n + lane, t = slot / CPR, q = slot % CPR;
    kdma[n] = (uint32_t)t * row_stride + hoff + (uint32_t)((q ^ kswz(t)) * 16);
  }
  uint32_t kread[NKC];  // QK A operand: token 4*(col%4) + col/4, chunk 4c + gq
  {
    const int t = 4 * (col & 3) + (col >> 2);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kread[c] = (uint32_t)(t * CPR + ((4 * c + gq) ^ kswz(t))) * 16;
  }
  const uint32_t voff = (uint32_t)gq * row_stride + hoff + col * VPL * 2;
  // Small blocks: for each row a lane loads, which block of the step holds it
  // and the byte offset inside that block.
  int kblk[GATHER ? NLI : 1], vblk[GATHER ? 4 : 1];
  uint32_t kin[GATHER ? NLI : 1], vin[GATHER ? 4 : 1];
  if constexpr (GATHER) {
#pragma unroll
    for (int n = 0; n < NLI; ++n) {
      const int slot = 64 * n + lane, t = slot / CPR, q = slot % CPR;
      kblk[n] = t / pool_bs;
      kin[n] = (uint32_t)(t % pool_bs) * row_stride + hoff + (uint32_t)((q ^ kswz(t)) * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + gq;
      vblk[i] = t / pool_bs;
      vin[i] = (uint32_t)(t % pool_bs) * row_stride + hoff + col * VPL * 2;
    }
  }
  // One LDS object per ring slot, so that the compiler's wait counting can
  // tell a slot being read from the slots whose loads are still in flight.
  __shared__ __attribute__((aligned(1024))) uint8_t kslot0[NBUF > 0 ? WPW : 1][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot1[NBUF > 1 ? WPW : 1][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot2[NBUF > 2 ? WPW : 1][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot3[NBUF > 3 ? WPW : 1][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot4[NBUF > 4 ? WPW : 1][KBYTES];
  static_assert(NBUF >= 2 && NBUF <= 5, "ring depth");
  auto slot_base = [&](int slot) -> uint8_t* {
    return slot == 0   ? &kslot0[wave][0]
           : slot == 1 ? &kslot1[wave][0]
           : slot == 2 ? &kslot2[wave][0]
           : slot == 3 ? &kslot3[wave][0]
                       : &kslot4[wave][0];
  };

  f32x4 acc[VPL];
#pragma unroll
  for (int t = 0; t < VPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;  // running max (log2 units) and partial denominator of head col

  // One block: K rows into ring slot `slot` of this wave's LDS, V rows into
  // registers; scalar buffer descriptors over the block (an offset past the
  // block would read zeros).
  // Past the partition's last block the loads are still issued (so every
  // wait stays an exact count) but through an empty descriptor: they return
  // zeros without touching memory.
  auto load_block = [&](int j, int slot, VT* vr) {
    const bool real = j <= last;
    const int jj = real ? j : last;
    if constexpr (GATHER) {  // per-lane rows; past the end the last step is re-read (cached, masked)
      size_t kb[NLI], vb[4];
      step_block_bases<NLI>(stab, jj, pshift, nent, (size_t)a.block_stride, kblk, kb);
      step_block_bases<4>(stab, jj, pshift, nent, (size_t)a.block_stride, vblk, vb);
#pragma unroll
      for (int n = 0; n < NLI; ++n)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(a.k_pool + kb[n] + kin[n]),
            (__attribute__((address_space(3))) void*)(slot_base(slot) + n * 1024), 16, 0, kKCpol);
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = *reinterpret_cast<const VT*>(a.v_pool + vb[i] + vin[i]);
      return;
    }
    const size_t off = SUB ? (size_t)(uint32_t)tab.get(jj >> pshift) * (size_t)a.block_stride +
                                 (size_t)(jj & ((1 << pshift) - 1)) * step_stride
                           : (size_t)(uint32_t)tab.get(jj) * (size_t)a.block_stride;
    const uint32_t span = real ? a.span : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_block_rsrc(a.k_pool + off, span);
    const __amdgpu_buffer_rsrc_t rv = make_block_rsrc(a.v_pool + off, span);
#pragma unroll
    for (int n = 0; n < NLI; ++n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(slot_base(slot) + n * 1024), 16, (int)kdma[n], 0, 0,
          kKCpol);
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = buffer_load_v<VT>(rv, voff + (uint32_t)(4 * i) * row_stride);
  };

  // One block; `valid` = context tokens in it (16 for inner blocks, fewer for
  // the sequence's last, 0 for the ring's overrun).  Branch free.
  // The QK A operand of ring slot `slot`, from LDS.
  auto read_k = [&](int slot, uint4* kr) {
    const uint8_t* kb = slot_base(slot);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kr[c] = *reinterpret_cast<const uint4*>(kb + kread[c]);
  };

  auto process = [&](const uint4* kr, const VT* vr, int valid) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) sacc = Ops::qk(kr[c], qop[c], sacc);
    float sc[4];
    VT vm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = 4 * i + gq < valid;
      sc[i] = ok ? sacc[i] * a.qscale : -INFINITY;
      vm[i] = ok ? vr[i] : VT{};  // garbage (even NaN) past the context must not reach the MFMA
    }
    const float mn = fmaxf(m, rows_max(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]))));
    const float alpha = fast_exp2(m - mn);  // 0 on the first block (m = -inf), 1 while the max stays
    m = mn;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - mn);
    const uint2 pb = make_uint2(Ops::pack(p[0], p[1]), Ops::pack(p[2], p[3]));
    // the denominator sums the same dtype-rounded weights that P.V multiplies
    l = fmaf(l, alpha, Ops::sum_pair(pb.x) + Ops::sum_pair(pb.y));
#pragma unroll
    for (int t = 0; t < VPL; ++t) {
      const int w = t >> 1;
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low 16-bit halves
      const uint2 va = make_uint2(__builtin_amdgcn_perm(vword<VPL>(vm[1], w), vword<VPL>(vm[0], w), sel),
                                  __builtin_amdgcn_perm(vword<VPL>(vm[3], w), vword<VPL>(vm[2], w), sel));
      acc[t] *= alpha;
      acc[t] = Ops::pv(va, pb, acc[t]);
    }
  };

  // Ring of NBUF buffers (LDS for K, registers for V): NBUF-1 blocks are in
  // flight while one is computed.  Every step issues its loads
  // unconditionally (past the last block through an empty descriptor, and
  // the steps past the end run fully masked), so each wait is an exact count.
  VT vr[NBUF][4];
  const int tok0 = start;
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) load_block(u, u, vr[u]);
  for (int j = 0; j < nblk; j += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int jj = j + u;
      uint4 kr[NKC];
      read_k(u, kr);  // this block's K, before its slot's neighbour is refilled
      load_block(jj + NBUF - 1, (u + NBUF - 1) % NBUF, vr[(u + NBUF - 1) % NBUF]);
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch issued ahead of this block's math
      process(kr, vr[u], max(0, min(BS, end - (tok0 + jj * BS))));
    }
  }

  const float lt = rows_sum(l);  // denominator of head col
  if (!live) return;
  if (seq_parts == 1) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float o[DPL];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < VPL; ++t) o[VPL * r + t] = acc[t][r] * inv;
    store_row<DT, DPL>(out_row, o);
  } else {
    const size_t idx = ((size_t)b * a.num_heads + h0 + col) * a.num_parts + s;
    float* dst = a.ws_acc + idx * D + gq * DPL;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int t = 0; t < VPL; t += 4) {
        *reinterpret_cast<float4*>(dst + VPL * r + t) =
            make_float4(acc[t][r], acc[t + 1][r], acc[t + 2][r], acc[t + 3][r]);
      }
    if (gq == 0) a.ws_ml[idx] = make_float2(m, lt);
  }
}

// One wave per (sequence, query head): merges the partials of a sequence that
// spans more than one partition.
template <int DT, int D>
__global__ __launch_bounds__(256) void combine_kernel(void* __restrict__ out, const float* __restrict__ ws_acc,
                                                      const float2* __restrict__ ws_ml,
                                                      const int32_t* __restrict__ context_lens, int num_seqs,
                                                      int num_heads, int part_tokens, int num_parts) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (idx >= num_seqs * num_heads) return;
  const int b = idx / num_heads;
  const int L = context_lens[b];
  const int np = L > 0 ? (L + part_tokens - 1) / part_tokens : 0;
  if (np <= 1) return;  // written by the partition kernel
  merge_partials<DT, D>((uint8_t*)out + (size_t)idx * D * ElemBytes<DT>::value, ws_acc + (size_t)idx * num_parts * D,
                        ws_ml + (size_t)idx * num_parts, np, lane);
}

// ------------------------------------------------------------------ dispatch

using DecodeFn = void (*)(const DecodeArgs);

#ifndef PA_MFMA_RING
#define PA_MFMA_RING 4
#endif
constexpr int kRing = PA_MFMA_RING;  // ring depth (blocks) of the MFMA decode kernel

template <int DT, int D, int MODE>
DecodeFn pick_rep(int repc) {
  switch (repc) {
    case 1: return decode_partition_kernel<DT, D, 1, MODE>;
    case 2: return decode_partition_kernel<DT, D, 2, MODE>;
    case 3: return decode_partition_kernel<DT, D, 3, MODE>;
    case 4: return decode_partition_kernel<DT, D, 4, MODE>;
    case 5: return decode_partition_kernel<DT, D, 5, MODE>;
    case 6: return decode_partition_kernel<DT, D, 6, MODE>;
    case 7: return decode_partition_kernel<DT, D, 7, MODE>;
    case 8: return decode_partition_kernel<DT, D, 8, MODE>;
    default: return nullptr;
  }
}

template <int DT, int D>
DecodeFn pick_rep_bs(int repc, int block_size) {
  if (block_size == pa::kBlockSize) return pick_rep<DT, D, kBlocks16>(repc);
  if (block_size > pa::kBlockSize) return pick_rep<DT, D, kBlocksLarge>(repc);
  return pick_rep<DT, D, kBlocksSmall>(repc);
}

template <int DT, int D, int MODE>
DecodeFn pick_mfma(int wpw) {
  switch (wpw) {
    case 1: return decode_mfma_kernel<DT, D, kRing, 1, MODE>;
    case 2: return decode_mfma_kernel<DT, D, kRing, 2, MODE>;
    case 4: return decode_mfma_kernel<DT, D, kRing, 4, MODE>;
#if PA_DECODE_MAX_WPW >= 8
    case 8: return decode_mfma_kernel<DT, D, kRing, 8, MODE>;
#endif
    default: return nullptr;
  }
}

template <int DT, int D>
DecodeFn pick_mfma_bs(int wpw, int block_size) {
  if (block_size == pa::kBlockSize) return pick_mfma<DT, D, kBlocks16>(wpw);
  if (block_size > pa::kBlockSize) return pick_mfma<DT, D, kBlocksLarge>(wpw);
  return pick_mfma<DT, D, kBlocksSmall>(wpw);
}

#ifndef PA_MHA_VALU
#define PA_MHA_VALU 0
#endif

// fp32: VALU kernel (one instantiation per heads-per-wave); fp16/bf16: MFMA
// kernel (one per waves-per-workgroup).  A build with PA_MHA_VALU=1 runs
// 16-bit batches without query-head groups (MHA) on the VALU kernel too.
DecodeFn pick_decode(int dtype, int d, const pa::DecodeGrid& g, int block_size) {
  if (PA_MHA_VALU && dtype != PA_F32 && g.rep == 1) {
    if (dtype == PA_F16) return d == 64 ? pick_rep_bs<DT_F16, 64>(1, block_size) : pick_rep_bs<DT_F16, 128>(1, block_size);
    return d == 64 ? pick_rep_bs<DT_BF16, 64>(1, block_size) : pick_rep_bs<DT_BF16, 128>(1, block_size);
  }
  switch (dtype) {
    case PA_F32:
      return d == 64 ? pick_rep_bs<DT_F32, 64>(g.repc, block_size) : pick_rep_bs<DT_F32, 128>(g.repc, block_size);
    case PA_F16:
      return d == 64 ? pick_mfma_bs<DT_F16, 64>(g.wpw, block_size) : pick_mfma_bs<DT_F16, 128>(g.wpw, block_size);
    case PA_BF16:
      return d == 64 ? pick_mfma_bs<DT_BF16, 64>(g.wpw, block_size) : pick_mfma_bs<DT_BF16, 128>(g.wpw, block_size);
    default: return nullptr;
  }
}

using CombineFn = void (*)(void*, const float*, const float2*, const int32_t*, int, int, int, int);

CombineFn pick_combine(int dtype, int d) {
  const bool d64 = d == 64;
  switch (dtype) {
    case PA_F32: return d64 ? combine_kernel<DT_F32, 64> : combine_kernel<DT_F32, 128>;
    case PA_F16: return d64 ? combine_kernel<DT_F16, 64> : combine_kernel<DT_F16, 128>;
    case PA_BF16: return d64 ? combine_kernel<DT_BF16, 64> : combine_kernel<DT_BF16, 128>;
    default: return nullptr;
  }
}

struct DecodePlan {
  int ps = 0, parts = 0;
  size_t need = 0;
};

// Host checks, the partition count and the partial bytes it needs; no HIP
// call unless partition_req == 0.
int plan_decode(const void* out, const void* query, const void* k_pool, const void* v_pool,
                const int32_t* block_tables, const int32_t* context_lens, const pa::DecodeShape& shp,
                float scale, int32_t partition_req, DecodePlan* plan) {
  int rc = pa::check_decode(out, query, k_pool, v_pool, block_tables, context_lens, shp, scale);
  if (rc != PA_OK) return rc;
  if (partition_req != 0 && pa::partition_size(shp, partition_req, 256, 1) < 0) return PA_ERR_INVALID_ARG;
  int cus = 256, per_cu = 1;
  if (partition_req == 0) {
    cus = pa::device_cu_count();
    const pa::DecodeGrid g = pa::decode_grid(shp);
    DecodeFn fn = pick_decode(shp.dtype, shp.head_dim, g, shp.block_size);
    if (!fn) return PA_ERR_UNSUPPORTED;
    per_cu = pa::resident_per_cu(reinterpret_cast<const void*>(fn), 64 * g.wpw);
    if (cus <= 0 || per_cu <= 0) return PA_ERR_HIP;
  }
  const int ps = pa::partition_size(shp, partition_req, cus, per_cu);
  if (ps <= 0) return -ps;
  plan->ps = ps;
  plan->parts = pa::num_partitions(shp.max_context_len, ps);
  plan->need = pa::workspace_bytes(shp.num_seqs, shp.num_heads, shp.head_dim, plan->parts);
  return PA_OK;
}

// PA_ERR_WORKSPACE unless `bytes` at `workspace` hold the plan's partials.
int check_workspace(const DecodePlan& plan, const void* workspace, size_t bytes) {
  return plan.need > 0 && (workspace == nullptr || bytes < plan.need) ? PA_ERR_WORKSPACE : PA_OK;
}

float2* ml_region(void* workspace, const pa::DecodeShape& shp, int parts) {
  if (parts <= 1) return nullptr;
  return reinterpret_cast<float2*>(static_cast<float*>(workspace) +
                                   (size_t)shp.num_seqs * shp.num_heads * parts * shp.head_dim);
}

int launch_partitions(void* out, const void* query, const pa::PoolView& pv, const int32_t* block_tables,
                      const int32_t* context_lens, const pa::DecodeShape& shp, float scale, void* workspace,
                      const DecodePlan& plan, void* stream) {
  const pa::DecodeGrid gd = pa::decode_grid(shp);
  const int64_t grid = (int64_t)shp.num_seqs * plan.parts * gd.groups;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  DecodeFn fn = pick_decode(shp.dtype, shp.head_dim, gd, shp.block_size);
  if (!fn) return PA_ERR_UNSUPPORTED;

  DecodeArgs a;
  a.out = out;
  a.query = query;
  a.k_pool = pv.k;
  a.v_pool = pv.v;
  a.block_stride = pv.block_stride;
  a.row_stride = (uint32_t)pv.row_stride;
  a.head_stride = (uint32_t)pv.head_stride;
  a.span = (uint32_t)pv.step_span(shp.head_dim * pa::elem_bytes(shp.dtype), shp.num_kv_heads);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = nullptr;
  a.num_seqs = shp.num_seqs;
  a.ctiles = 0;  // column mode only
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = ml_region(workspace, shp, plan.parts);
  a.num_heads = shp.num_heads;
  a.num_kv_heads = shp.num_kv_heads;
  a.rep = gd.rep;
  a.chunks = gd.chunks;
  a.max_blocks_per_seq = shp.max_blocks_per_seq;
  a.block_shift = pa::block_shift(shp.block_size);
  a.part_tokens = plan.ps;
  a.num_parts = plan.parts;
  a.groups = gd.groups;
  a.qscale = scale * 1.44269504088896340736f;  // log2(e)
  return pa::launch_kernel(fn, dim3((unsigned)grid), dim3(64 * gd.wpw), static_cast<hipStream_t>(stream), a);
}

int launch_combine(void* out, const int32_t* context_lens, const pa::DecodeShape& shp, void* workspace,
                   const DecodePlan& plan, void* stream) {
  if (plan.parts <= 1) return PA_OK;
  CombineFn cf = pick_combine(shp.dtype, shp.head_dim);
  if (!cf) return PA_ERR_UNSUPPORTED;
  const int64_t waves = (int64_t)shp.num_seqs * shp.num_heads;
  return pa::launch_kernel(cf, dim3((unsigned)((waves + 3) / 4)), dim3(256), static_cast<hipStream_t>(stream), out,
                           static_cast<const float*>(workspace), ml_region(workspace, shp, plan.parts),
                           context_lens, shp.num_seqs, shp.num_heads, plan.ps, plan.parts);
}

}  // namespace

namespace pa {

int device_cu_count() {
  static std::atomic<int> cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return -1;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int D>
DecodeFn pick_columns_mfma(int block_size) {
  if (block_size == kBlockSize) return columns_f32_mfma_kernel<D, kBlocks16>;
  if (block_size > kBlockSize) return columns_f32_mfma_kernel<D, kBlocksLarge>;
  return columns_f32_mfma_kernel<D, kBlocksSmall>;
}

// fp32 column mode: the matrix-core tile (16 columns per wave), or with
// PA_F32_COLUMNS_MFMA=0 the VALU tile (cols_per_wave(head_dim) columns).
DecodeFn pick_columns(const PrefillShape& s) {
  if (s.d.dtype != PA_F32) return nullptr;
  const int cols = cols_per_wave(s.d.head_dim);
  if (kColumnsMfma) return s.d.head_dim == 64 ? pick_columns_mfma<64>(s.d.block_size) : pick_columns_mfma<128>(s.d.block_size);
  return s.d.head_dim == 64 ? pick_rep_bs<DT_F32, 64>(cols, s.d.block_size)
                            : pick_rep_bs<DT_F32, 128>(cols, s.d.block_size);
}

const void* columns_kernel(const PrefillShape& s, int* threads) {
  *threads = 64 * column_grid(s).wpw;
  return reinterpret_cast<const void*>(pick_columns(s));
}

int launch_columns(void* out, const void* query, const PoolView& pv, const int32_t* block_tables,
                   const int32_t* context_lens, const int32_t* query_start_loc, const PrefillShape& s, float scale,
                   void* ws_acc, void* ws_ml, int part_tokens, int num_parts, void* stream) {
  const ColumnGrid cg = column_grid(s);
  const int64_t grid = cg.items * num_parts;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  DecodeFn fn = pick_columns(s);
  if (!fn) return PA_ERR_UNSUPPORTED;
  const DecodeShape& d = s.d;
  DecodeArgs a;
  a.out = out;
  a.query = query;
  a.k_pool = pv.k;
  a.v_pool = pv.v;
  a.block_stride = pv.block_stride;
  a.row_stride = (uint32_t)pv.row_stride;
  a.head_stride = (uint32_t)pv.head_stride;
  a.span = (uint32_t)pv.step_span(d.head_dim * elem_bytes(d.dtype), d.num_kv_heads);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.num_seqs = d.num_seqs;
  a.ctiles = cg.ctiles;
  a.ws_acc = static_cast<float*>(ws_acc);
  a.ws_ml = static_cast<float2*>(ws_ml);
  a.num_heads = d.num_heads;
  a.num_kv_heads = d.num_kv_heads;
  a.rep = d.num_heads / d.num_kv_heads;
  a.chunks = 0;  // decode mode only
  a.groups = 0;
  a.max_blocks_per_seq = d.max_blocks_per_seq;
  a.block_shift = block_shift(d.block_size);
  a.part_tokens = part_tokens;
  a.num_parts = num_parts;
  a.qscale = scale * 1.44269504088896340736f;  // log2(e)
  return launch_kernel(fn, dim3((unsigned)grid), dim3(64 * cg.wpw), static_cast<hipStream_t>(stream), a);
}

// Workgroups of `fn` (with `threads` threads) resident per compute unit, cached
// per (device, kernel).  0 on failure.
int resident_per_cu(const void* fn, int threads) {
  struct Entry { int dev; const void* fn; int n; };
  static Entry cache[256];
  static int used = 0;
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i)
      if (cache[i].dev == dev && cache[i].fn == fn) return cache[i].n;
  }
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, threads, 0) != hipSuccess)
    return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (used < 256) cache[used++] = Entry{dev, fn, n};
  return n;
}

}  // namespace pa

// ------------------------------------------------------------------ C ABI

extern "C" int pa_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables, const int32_t* context_lens,
                               const int32_t* query_start_loc, int32_t num_seqs, int32_t max_blocks_per_seq,
                               int32_t block_size, int64_t num_tokens, void* stream) {
  if (num_seqs == 0 && num_tokens == 0) return PA_OK;  // an empty batch
  int rc = pa::check_slot_mapping(slot_mapping, block_tables, context_lens, query_start_loc, num_seqs,
                                  max_blocks_per_seq, block_size, num_tokens);
  if (rc != PA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (!query_start_loc)
    return pa::launch_kernel(slot_mapping_decode_kernel, dim3((num_seqs + 255) / 256), dim3(256), st, slot_mapping,
                             block_tables, context_lens, num_seqs, max_blocks_per_seq, block_size);
  return pa::launch_kernel(slot_mapping_varlen_kernel, dim3(num_seqs), dim3(64), st, slot_mapping, block_tables,
                           context_lens, query_start_loc, max_blocks_per_seq, block_size, num_tokens);
}

namespace {

template <typename V>
int launch_reshape(const void* key, const void* value, const pa::PoolView& pv, const int64_t* slots,
                   int64_t num_tokens, int num_kv_heads, int head_bytes, int block_size, int64_t num_slots,
                   int threads, hipStream_t st) {
  constexpr int64_t W = sizeof(V);
  return pa::launch_kernel(reshape_and_cache_kernel<V>, dim3((unsigned)num_tokens, 2), dim3(threads), st,
                           (const V*)key, (const V*)value, (V*)const_cast<uint8_t*>(pv.k),
                           (V*)const_cast<uint8_t*>(pv.v), slots, (int)(head_bytes / W), num_kv_heads, block_size,
                           pv.block_stride / W, pv.row_stride / W, pv.head_stride / W, num_slots);
}

}  // namespace

extern "C" int pa_reshape_and_cache_layout(const void* key, const void* value, void* k_pool, void* v_pool,
                                           const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                           pa_dtype dtype, pa_kv_layout layout, void* stream) {
  pa::PoolView pv;
  int rc = pa::check_reshape(key, value, k_pool, layout == PA_KV_FUSED ? k_pool : v_pool, slot_mapping, num_tokens,
                             num_kv_heads, head_dim, block_size, num_blocks, dtype);
  if (rc != PA_OK) return rc;
  rc = pa::pool_view(k_pool, v_pool, (int)layout, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
  if (num_tokens == 0) return PA_OK;
  const int head_bytes = head_dim * pa::elem_bytes(dtype);
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
    return launch_reshape<V>(key, value, pv, slot_mapping, num_tokens, num_kv_heads, head_bytes, block_size,
                             num_slots, threads, st);
  };
  switch (vec) {
    case 16: return run(uint4{});
    case 8: return run(uint2{});
    case 4: return run(uint32_t{});
    case 2: return run(uint16_t{});
    default: return run(uint8_t{});
  }
}

extern "C" int pa_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const int64_t* slot_mapping, int64_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int64_t num_blocks, pa_dtype dtype,
                                    void* stream) {
  if (!v_pool) return PA_ERR_INVALID_ARG;
  return pa_reshape_and_cache_layout(key, value, k_pool, v_pool, slot_mapping, num_tokens, num_kv_heads, head_dim,
                                     block_size, num_blocks, dtype, PA_KV_SPLIT, stream);
}

extern "C" int pa_decode_attention_layout(void* out, const void* query, const void* k_pool, const void* v_pool,
                                          const int32_t* block_tables, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                          int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                          int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                                          size_t workspace_bytes, int32_t partition_size, pa_kv_layout layout,
                                          void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch
  const pa::DecodeShape shp{num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            max_context_len, (int)dtype};
  pa::PoolView pv;
  int rc = pa::check_decode(out, query, k_pool, layout == PA_KV_FUSED ? k_pool : v_pool, block_tables,
                            context_lens, shp, scale);
  if (rc != PA_OK) return rc;
  rc = pa::pool_view(k_pool, v_pool, (int)layout, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
  DecodePlan plan;
  rc = plan_decode(out, query, pv.k, pv.v, block_tables, context_lens, shp, scale, partition_size, &plan);
  if (rc == PA_OK) rc = check_workspace(plan, workspace, workspace_bytes);
  if (rc != PA_OK) return rc;
  rc = launch_partitions(out, query, pv, block_tables, context_lens, shp, scale, workspace, plan, stream);
  if (rc != PA_OK) return rc;
  return launch_combine(out, context_lens, shp, workspace, plan, stream);
}

extern "C" int pa_decode_attention_ex(void* out, const void* query, const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, int32_t max_context_len,
                                      float scale, pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                      int32_t partition_size, void* stream) {
  if (!v_pool) return PA_ERR_INVALID_ARG;
  return pa_decode_attention_layout(out, query, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                                    num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len, scale,
                                    dtype, workspace, workspace_bytes, partition_size, PA_KV_SPLIT, stream);
}

extern "C" int pa_decode_attention(void* out, const void* query, const void* k_pool, const void* v_pool,
                                   const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                   int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                   pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return pa_decode_attention_ex(out, query, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                                num_kv_heads, head_dim, block_size, max_blocks_per_seq, max_context_len, scale,
                                dtype, workspace, workspace_bytes, 0, stream);
}

extern "C" int pa_decode_partitions(void* out, const void* query, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t max_blocks_per_seq, int32_t max_context_len, float scale,
                                    pa_dtype dtype, void* workspace, size_t workspace_bytes,
                                    int32_t partition_size, void* stream) {
  if (partition_size == 0) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;  // an empty batch
  const pa::DecodeShape shp{num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            max_context_len, (int)dtype};
  DecodePlan plan;
  int rc = plan_decode(out, query, k_pool, v_pool, block_tables, context_lens, shp, scale, partition_size, &plan);
  if (rc == PA_OK) rc = check_workspace(plan, workspace, workspace_bytes);
  if (rc != PA_OK) return rc;
  pa::PoolView pv;
  rc = pa::pool_view(k_pool, v_pool, PA_KV_SPLIT, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
  return launch_partitions(out, query, pv, block_tables, context_lens, shp, scale, workspace, plan, stream);
}

extern "C" int pa_decode_combine(void* out, const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                                 int32_t head_dim, int32_t max_context_len, int32_t partition_size, pa_dtype dtype,
                                 const void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch
  int rc = pa::check_combine(out, context_lens, num_seqs, num_heads, head_dim, max_context_len, partition_size,
                             (int)dtype);
  if (rc != PA_OK) return rc;
  const pa::DecodeShape shp{num_seqs, num_heads, 1, head_dim, pa::kBlockSize, 1, max_context_len, (int)dtype};
  DecodePlan plan;
  plan.ps = partition_size;
  plan.parts = pa::num_partitions(max_context_len, partition_size);
  plan.need = pa::workspace_bytes(num_seqs, num_heads, head_dim, plan.parts);
  rc = check_workspace(plan, workspace, workspace_bytes);
  if (rc != PA_OK) return rc;
  return launch_combine(out, context_lens, shp, const_cast<void*>(workspace), plan, stream);
}

extern "C" int32_t pa_decode_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                            pa_dtype dtype, const int32_t* host_context_lens) {
  const pa::DecodeShape shp{num_seqs, num_heads, num_kv_heads, head_dim, block_size, 1 << 30, max_context_len,
                            (int)dtype};
  const int rc = pa::check_partition_query(shp);
  if (rc != PA_OK) return -rc;
  const pa::DecodeGrid g = pa::decode_grid(shp);
  DecodeFn fn = pick_decode(shp.dtype, shp.head_dim, g, shp.block_size);
  if (!fn) return -PA_ERR_UNSUPPORTED;
  const int cus = pa::device_cu_count();
  const int per_cu = pa::resident_per_cu(reinterpret_cast<const void*>(fn), 64 * g.wpw);
  if (cus <= 0 || per_cu <= 0) return -PA_ERR_HIP;
  return pa::partition_size(shp, 0, cus, per_cu, host_context_lens);
}

// ------------------------------------------------------------------ decode without a workspace argument
//
// For callers that cannot allocate device memory: the split-context partials
// live in `scratch`, one copy per GPU, held until the process ends.  In host
// code the name `scratch` only stands in for the symbol; its device address
// comes from hipGetSymbolAddress, once per device, with that device current.

static __device__ __align__(256) uint8_t scratch[PA_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;

// Device address of the current device's `scratch`, or nullptr on a HIP error.
void* scratch_on_current_device() {
  static std::atomic<void*> addr[kScratchDevices] = {};
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" int pa_decode_attention_noalloc(void* out, const void* query, const void* k_pool, const void* v_pool,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, float scale, pa_dtype dtype,
                                           int32_t partition_size, void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch
  if (!v_pool) return PA_ERR_INVALID_ARG;
  const pa::DecodeShape shp{num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                            max_context_len, (int)dtype};
  pa::PoolView pv;
  int rc = pa::check_decode(out, query, k_pool, v_pool, block_tables, context_lens, shp, scale);
  if (rc != PA_OK) return rc;
  rc = pa::pool_view(k_pool, v_pool, PA_KV_SPLIT, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
  DecodePlan plan;
  rc = plan_decode(out, query, pv.k, pv.v, block_tables, context_lens, shp, scale, partition_size, &plan);
  if (rc != PA_OK) return rc;
  if (plan.need > PA_DECODE_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return PA_ERR_HIP;
  }
  rc = launch_partitions(out, query, pv, block_tables, context_lens, shp, scale, ws, plan, stream);
  if (rc != PA_OK) return rc;
  return launch_combine(out, context_lens, shp, ws, plan, stream);
}
