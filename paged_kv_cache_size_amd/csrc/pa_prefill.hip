// Paged attention for several new tokens per sequence on gfx950: varlen
// prefill, chunked prefill, and batches that mix prefill chunks with decode
// steps.  Sequence b contributes the query rows query_start_loc[b] ..
// query_start_loc[b+1]; they are the last n_b positions of its context of
// length L_b, and the row at position p attends causally to positions 0..p
// (handbook "分页 KV Cache", section "分页注意力": seq_lens is the context after
// this step, query_start_loc delimits each sequence's new tokens, and the mask
// keeps, for new token i, the positions up to L_b - n_b + i).
//
// The tile is the decode MFMA tile with its 16 columns re-purposed: a column
// is a (new token, query head) pair of one KV head's group instead of one
// query head of the single new token.  Per pair of 16-token blocks (32 keys):
//   QK:  S^T[key][column]  = K[16 x D] . Q^T[D x 16]   mfma_f32_16x16x32 (D/32 per block)
//   PV:  O^T[dim][column] += V^T[16 x 32] . P^T          mfma_f32_16x16x32 (D/16)
// K goes through LDS in a swizzled row order.  The per-wave tile pairs V rows
// (loaded into registers) by v_perm; the cooperative tile reads V transposed
// from LDS (ds_read_b64_tr_b16).  Causality is a per-column key limit applied
// to the probabilities; V rows past the partition's last key are zeroed, so
// stale slots never reach the MFMA.
// Long contexts split into partitions like decode; the partials are merged per
// (query row, head) by the combine kernel below.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "pa.h"
#include "pa_device.h"
#include "pa_host.h"
#include "pa_runtime.h"

namespace {

struct PrefillArgs {
  void* out;                 // [T, H, D]
  const void* query;         // [T, H, D]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start_loc;  // [B + 1]; null: sequence b owns row b alone
  const int32_t* table_rows;       // [B] block-table row of sequence b; null: row b
  const int32_t* key_begin;        // [B] first key of sequence b's range; null: 0
  float* ws_acc;                   // [T, H, slots, D]
  float2* ws_ml;                   // [T, H, slots] (running max in log2 units, denominator)
  int num_heads, num_kv_heads, rep, repc, chunks, max_blocks_per_seq;
  int block_shift;  // pool blocks of 16 << shift (kBlocksLarge) or 16 >> shift (kBlocksSmall) tokens
  int part_tokens, num_parts, groups, tiles;  // tiles: 16-column tiles per (sequence, wave unit)
  int causal;          // 1: row i sits at position L - n + i; 0: every row sees the whole key range
  int partial_base;    // < 0: final rows, partials only for split rows; >= 0: every partition's
  int partial_stride;  //   partials go to slot partial_base + s of partial_stride slots per row
  float qscale;        // |scale| * log2(e)
  int qneg;            // scale < 0: the query's signs are flipped as it is loaded, so qscale >= 0
  // pool geometry in bytes (layout): K row (block p, token t, head h) at
  // k_pool + p*block_stride + t*row_stride + h*head_stride, V likewise;
  // span = what one block may touch from its first byte
  int64_t block_stride;
  uint32_t row_stride, head_stride, span;
};

// A finite floor for the running max: a column whose keys all lie beyond this
// block (or partition) keeps m at the floor, so alpha = 2^0 and p = 2^-inf = 0
// instead of the NaN that -inf - -inf would give.
constexpr float kMaxFloor = -3.0e38f;
constexpr float kRescaleLog2 = 8.f;  // lazy rescale threshold, log2 units

// NaN-propagating maximum: v_maximum3_f32 on gfx950, which unlike fmaxf needs
// no quieting of its inputs.  Masked scores enter as -inf, so only a NaN
// input can make the result NaN.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max8(const float (&x)[8]) {
  return vmax(vmax(vmax(vmax(x[0], x[1]), x[2]), vmax(vmax(x[3], x[4]), x[5])), vmax(vmax(x[6], x[7]), -INFINITY));
}
__device__ __forceinline__ float rows_maximum(float x) {  // over the 4 row groups of a 16x16 tile
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The online-softmax update of one column tile for a pair of 16-key blocks
// (the per-wave tile; the cooperative tile runs the same update phased over
// its tiles, with one branch for all their rescales).  x[i]: the lane's raw score (scale not applied) of key 4(i%4) + gq of block
// i/4; ok[i] (boundary steps only): that key is visible to the lane's column.
// Moves the running max m (log2 units) when a score exceeds it by more than
// 2^8 (probabilities stay <= 256, exact in fp32 sums) and then rescales l and
// the accumulators - a rare, wave-uniform branch; adds the probabilities, as
// rounded to the 16-bit type, to l and returns them packed as the P.V B
// operand.  Absent keys get p = 0 by a
// select after the exponential (not a -inf score, which times a zero scale
// would be NaN).  qscale >= 0, so the max of the raw scores scales to the max
// of the scaled ones.
template <int DT, int VPL, bool kInterior>
__device__ __forceinline__ uint4 softmax_pair(const float (&x)[8], const bool (&ok)[8], float qscale, float& m,
                                              float& l, f32x4* acc) {
  using Ops = MfmaOps<DT>;
  float xm[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xm[i] = kInterior || ok[i] ? x[i] : -INFINITY;
  const float smax = rows_maximum(max8(xm)) * qscale;
  if (__ballot(smax > m + kRescaleLog2)) {
    const float mn = fmaxf(m, smax);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    l *= alpha;
#pragma unroll
    for (int t = 0; t < VPL; ++t) acc[t] *= alpha;
  }
  const float nm = -m;
  float p[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float e = fast_exp2(fmaf(x[i], qscale, nm));
    p[i] = kInterior || ok[i] ? e : 0.f;
  }
  const uint4 pk =
      make_uint4(Ops::pack(p[0], p[1]), Ops::pack(p[2], p[3]), Ops::pack(p[4], p[5]), Ops::pack(p[6], p[7]));
  // the denominator sums the same dtype-rounded weights that P.V multiplies
  l += (Ops::sum_pair(pk.x) + Ops::sum_pair(pk.y)) + (Ops::sum_pair(pk.z) + Ops::sum_pair(pk.w));
  return pk;
}

// A query operand chunk (8 16-bit values) as loaded, with every sign flipped
// when the scale is negative.
__device__ __forceinline__ uint4 query_chunk(const uint8_t* p, bool live, int qneg) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t f = qneg ? 0x80008000u : 0u;
  return live ? make_uint4(v.x ^ f, v.y ^ f, v.z ^ f, v.w ^ f) : make_uint4(0, 0, 0, 0);
}

// Four consecutive output elements from four floats (8 bytes for 16-bit
// types, 16 for fp32).
template <int DT>
__device__ __forceinline__ void store4(uint8_t* dst, const float (&f)[4]) {
  if constexpr (DT == DT_F32) {
    *reinterpret_cast<float4*>(dst) = make_float4(f[0], f[1], f[2], f[3]);
  } else {
    auto bits = [](float x) { return DT == DT_BF16 ? float_to_bf16_bits(x) : float_to_f16_bits(x); };
    *reinterpret_cast<uint2*>(dst) = make_uint2(bits(f[0]) | (bits(f[1]) << 16), bits(f[2]) | (bits(f[3]) << 16));
  }
}

// ds_read_b64_tr_b16: within each 16-lane group, lane 4a + b receives element
// b of the four 16-bit elements addressed by lanes a, a + 4, a + 8, a + 12.
__device__ __forceinline__ uint2 lds_read_tr16(const uint8_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)((__attribute__((address_space(3))) uint8_t*)p));
  return __builtin_bit_cast(uint2, r);
}

// XOR swizzle of a V row's 16-byte chunks in LDS for the transposed reads:
// a 32-lane half of one read touches 8 rows (4 rows of two row groups) at the
// same pair of chunks; row t's chunks are moved by 2*f(t) with f distinct
// over those rows, so the 8 pairs land on distinct banks.  (Rows of 8 chunks
// pair up by parity inside 256 bytes, so f keeps only the row's group.)
template <int CPR>
__device__ __forceinline__ int vswz_t(int t) {
  return 2 * ((((t >> 2) & 3) | ((t & 1) << 2)) & (CPR / 2 - 1));
}

// The end of one column's work in one partition: lane (gq, col) holds
// accumulator tile t register r = O[col][dim (D/16)(4gq + r) + t] (V rows
// paired in registers) or O[col][dim 16t + 4gq + r] (kTr: V read transposed
// from LDS), the column's running max m (log2 units) and denominator lt.
//  * slot mode (partial_base >= 0): partials into slot partial_base + s,
//    m = -inf when the column saw no key;
//  * a column whose keys fit one partition: its output row;
//  * otherwise: partials for the combine kernel.
template <int DT, int D, bool kTr = false>
__device__ __forceinline__ void store_column(const PrefillArgs& a, const f32x4* acc, float m, float lt, size_t qrow,
                                             int s, int col_parts, int gq) {
  constexpr int VPL = D / 16, DPL = 4 * VPL, ROWB = D * 2, EB = DT == DT_F32 ? 4 : 2;
  auto store_partial = [&](size_t idx, float mm) {
    if constexpr (kTr) {
      float* dst = a.ws_acc + idx * D + 4 * gq;
#pragma unroll
      for (int t = 0; t < VPL; ++t)
        *reinterpret_cast<float4*>(dst + 16 * t) = make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    } else {
      float* dst = a.ws_acc + idx * D + gq * DPL;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < VPL; t += 4)
          *reinterpret_cast<float4*>(dst + VPL * r + t) =
              make_float4(acc[t][r], acc[t + 1][r], acc[t + 2][r], acc[t + 3][r]);
    }
    if (gq == 0) a.ws_ml[idx] = make_float2(mm, lt);
  };
  if (a.partial_base >= 0) {
    store_partial(qrow * a.partial_stride + a.partial_base + s, lt > 0.f ? m : -INFINITY);
    return;
  }
  if (s >= col_parts) return;  // no keys of this column here
  if (col_parts == 1) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if constexpr (kTr) {
      uint8_t* dst = (uint8_t*)a.out + qrow * ROWB + 4 * gq * EB;
#pragma unroll
      for (int t = 0; t < VPL; ++t) {
        const float o[4] = {acc[t][0] * inv, acc[t][1] * inv, acc[t][2] * inv, acc[t][3] * inv};
        store4<DT>(dst + 16 * t * EB, o);
      }
    } else {
      float o[DPL];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int t = 0; t < VPL; ++t) o[VPL * r + t] = acc[t][r] * inv;
      store_row<DT, DPL>((uint8_t*)a.out + qrow * ROWB + gq * DPL * 2, o);
    }
  } else {
    store_partial(qrow * a.num_parts + s, m);
  }
}

// Marks one column's slot empty (m = -inf, l = 0, acc = 0) in slot mode.
template <int D>
__device__ __forceinline__ void store_empty_slot(const PrefillArgs& a, size_t qrow, int s, int gq) {
  constexpr int DPL = D / 4;
  const size_t idx = qrow * a.partial_stride + a.partial_base + s;
  float* dst = a.ws_acc + idx * D + gq * DPL;
#pragma unroll
  for (int i = 0; i < DPL; i += 4) *reinterpret_cast<float4*>(dst + i) = make_float4(0.f, 0.f, 0.f, 0.f);
  if (gq == 0) a.ws_ml[idx] = make_float2(-INFINITY, 0.f);
}

template <int DT, int D, int NBUF, int WPW, int MODE>
__global__ __launch_bounds__(64 * WPW) void prefill_mfma_kernel(const PrefillArgs a) {
  constexpr bool SUB = MODE == kBlocksLarge;
  constexpr bool GATHER = MODE == kBlocksSmall;
  using Ops = MfmaOps<DT>;
  constexpr int BS = pa::kBlockSize;
  constexpr int ROWB = D * 2;
  constexpr int NKC = D / 32;      // QK k-chunks
  constexpr int VPL = D / 16;      // V elements per lane and row = PV output tiles
  constexpr int CPR = ROWB / 16;   // 16-byte chunks per K row
  constexpr int NLI = BS * CPR / 64;  // K load instructions per block
  constexpr int KBYTES = BS * ROWB;
  using VT = typename VRow<VPL>::T;
  static_assert(BS == 16, "the MFMA tiling assumes 16-token blocks");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int rest = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = rest % a.groups;
  rest /= a.groups;
  const int s = rest % a.num_parts;
  rest /= a.num_parts;
  const int tile = rest % a.tiles;
  const int b = rest / a.tiles;
  const int unit = grp * WPW + wave;
  const int g = unit / a.chunks;
  const int gq = lane >> 4, col = lane & 15;

  const int q0 = a.query_start_loc ? a.query_start_loc[b] : b;
  const int n = a.query_start_loc ? a.query_start_loc[b + 1] - q0 : 1;  // query rows of this sequence
  const int L = a.context_lens[b];
  const int kb = a.key_begin ? a.key_begin[b] : 0;  // keys [kb, L)
  const int trow = a.table_rows ? a.table_rows[b] : b;
  const int first_tok = (16 * tile) / a.repc;
  if (first_tok >= n) return;  // the whole wave lies past this sequence's new tokens
  const int last_tok = min(n - 1, (16 * tile + 15) / a.repc);

  // This lane's column: new token ti, query head h, position pos.
  const int cc = 16 * tile + col;
  const int ti = cc / a.repc;
  const bool live = ti < n;
  const int h = g * a.rep + (unit % a.chunks) * a.repc + cc % a.repc;
  const int pos = a.causal ? L - n + ti : L - 1;  // last key this column sees
  const size_t qrow = ((size_t)(q0 + (live ? ti : 0)) * a.num_heads + h);

  const int start = kb + s * a.part_tokens;
  const int pend = min(L, start + a.part_tokens);
  const int end = min(pend, a.causal ? L - n + last_tok + 1 : L);  // keys any column of the wave sees here
  if (start >= end) {  // no column's keys in this partition
    if (a.partial_base >= 0 && live) store_empty_slot<D>(a, qrow, s, gq);  // the merge reads every slot
    return;
  }
  const int lim = live ? min(pend, pos + 1) : 0;  // this column's keys are [start, lim)
  const int col_parts = (pos - kb + a.part_tokens) / a.part_tokens;  // partitions holding its keys
  const int pshift = MODE != kBlocks16 ? a.block_shift : 0;
  const int pool_bs = SUB ? BS << pshift : GATHER ? BS >> pshift : BS;  // tokens per pool block
  const int blk0 = start / pool_bs;  // partitions start on a pool block
  const int nblk = (end - start + BS - 1) / BS;  // 16-token steps
  const int nent = MODE == kBlocks16 ? nblk : (end - start + pool_bs - 1) / pool_bs;  // 1..kMaxPartitionBlocks
  const int last = nblk - 1;

  const int32_t* bt = a.block_tables + (size_t)trow * a.max_blocks_per_seq + blk0;
  TableSlice tab;  // blocks of 16 tokens or more: the slice in VGPR lanes
  __shared__ int32_t stab[GATHER ? pa::kMaxSmallBlockPartition : 1];  // small blocks: in LDS
  if constexpr (GATHER)
    stage_table(stab, bt, nent);
  else
    tab.load(bt, nent, lane);

  uint4 qop[NKC];
  {
    const uint8_t* qp = (const uint8_t*)a.query + qrow * ROWB + gq * 16;
#pragma unroll
    for (int c = 0; c < NKC; ++c) qop[c] = query_chunk(qp + c * 64, live, a.qneg);
  }

  const uint32_t row_stride = a.row_stride;
  const uint32_t hoff = (uint32_t)g * a.head_stride;
  const size_t block_stride = (size_t)a.block_stride;
  uint32_t kdma[NLI];
#pragma unroll
  for (int i = 0; i < NLI; ++i) {
    const int slot = 64 * i + lane, t = slot / CPR, q = slot % CPR;
    kdma[i] = (uint32_t)t * row_stride + hoff + (uint32_t)((q ^ kswz_t<CPR>(t)) * 16);
  }
  uint32_t kread[NKC];  // QK A operand: token 4*(col%4) + col/4, chunk 4c + gq
  {
    const int t = 4 * (col & 3) + (col >> 2);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kread[c] = (uint32_t)(t * CPR + ((4 * c + gq) ^ kswz_t<CPR>(t))) * 16;
  }
  const uint32_t voff = (uint32_t)gq * row_stride + hoff + col * VPL * 2;
  const size_t step_stride = (size_t)BS * row_stride;  // 16-token windows inside a larger block
  // Small blocks: for each row a lane loads, its block within the step and
  // its byte offset inside that block.
  int kblk[GATHER ? NLI : 1], vblk[GATHER ? 4 : 1];
  uint32_t kin[GATHER ? NLI : 1], vin[GATHER ? 4 : 1];
  if constexpr (GATHER) {
#pragma unroll
    for (int i = 0; i < NLI; ++i) {
      const int slot = 64 * i + lane, t = slot / CPR, q = slot % CPR;
      kblk[i] = t / pool_bs;
      kin[i] = (uint32_t)(t % pool_bs) * row_stride + hoff + (uint32_t)((q ^ kswz_t<CPR>(t)) * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * i + gq;
      vblk[i] = t / pool_bs;
      vin[i] = (uint32_t)(t % pool_bs) * row_stride + hoff + col * VPL * 2;
    }
  }
  __shared__ __attribute__((aligned(1024))) uint8_t kslot0[WPW][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot1[WPW][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot2[NBUF > 2 ? WPW : 1][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot3[NBUF > 3 ? WPW : 1][KBYTES];
  static_assert(NBUF >= 2 && NBUF <= 4, "ring depth");
  auto slot_base = [&](int slot) -> uint8_t* {
    return slot == 0 ? &kslot0[wave][0] : slot == 1 ? &kslot1[wave][0] : slot == 2 ? &kslot2[wave][0] : &kslot3[wave][0];
  };

  f32x4 acc[VPL];
#pragma unroll
  for (int t = 0; t < VPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kMaxFloor, l = 0.f;

  // Loads past the partition's last step go through an empty descriptor
  // (zeros, no memory access), so every wait stays an exact count; with small
  // blocks (per-lane addresses) they re-read the last step's rows instead
  // (masked).
  auto load_block = [&](int j, int slot, VT* vr) {
    const bool real = j <= last;
    const int jj = real ? j : last;
    if constexpr (GATHER) {
      size_t kbase[NLI], vbase[4];
      step_block_bases<NLI>(stab, jj, pshift, nent, block_stride, kblk, kbase);
      step_block_bases<4>(stab, jj, pshift, nent, block_stride, vblk, vbase);
#pragma unroll
      for (int i = 0; i < NLI; ++i)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(a.k_pool + kbase[i] + kin[i]),
            (__attribute__((address_space(3))) void*)(slot_base(slot) + i * 1024), 16, 0, kKCpol);
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = *reinterpret_cast<const VT*>(a.v_pool + vbase[i] + vin[i]);
      return;
    }
    const size_t off = SUB ? (size_t)(uint32_t)tab.get(jj >> pshift) * (uint32_t)block_stride +
                                 (size_t)(jj & ((1 << pshift) - 1)) * step_stride
                           : (size_t)(uint32_t)tab.get(jj) * (uint32_t)block_stride;  // stride <= 2^31 (host check)
    const uint32_t span = real ? a.span : 0u;
    const __amdgpu_buffer_rsrc_t rk = make_block_rsrc(a.k_pool + off, span);
    const __amdgpu_buffer_rsrc_t rv = make_block_rsrc(a.v_pool + off, span);
#pragma unroll
    for (int i = 0; i < NLI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(slot_base(slot) + i * 1024), 16, (int)kdma[i], 0, 0,
          kKCpol);
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = buffer_load_v<VT>(rv, voff + (uint32_t)(4 * i) * row_stride);
  };
  auto read_k = [&](int slot, uint4* kr) {
    const uint8_t* kb = slot_base(slot);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kr[c] = *reinterpret_cast<const uint4*>(kb + kread[c]);
  };
  // Keys [start, safe) are visible to every live column of the wave: steps
  // wholly below `safe` need no masks.
  const int safe = min(pend, a.causal ? L - n + first_tok + 1 : L);

  // Two blocks (32 keys) whose first key is `key0`.  Lane (gq, col) register i
  // of the block-A (block-B) score tile holds key key0 + 4i + gq (+ 16) of
  // column col.  P.V runs on mfma_f32_16x16x32 with the contraction index
  // k = 8gq + j <-> key 4(j % 4) + gq of block A (j < 4) or B (j >= 4): the
  // lane's own score registers are its B operand, its own V rows its A operand.
  auto step = [&](const uint4* kra, const uint4* krb, const VT* va_rows, const VT* vb_rows, int key0,
                  auto interior) {
    constexpr bool kInterior = decltype(interior)::value;
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      sa = Ops::qk(kra[c], qop[c], sa);
      sb = Ops::qk(krb[c], qop[c], sb);
    }
    const float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
    VT v[8] = {va_rows[0], va_rows[1], va_rows[2], va_rows[3], vb_rows[0], vb_rows[1], vb_rows[2], vb_rows[3]};
    bool ok[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = key0 + (i >> 2) * 16 + 4 * (i & 3) + gq;
      ok[i] = key < lim;
      if constexpr (!kInterior)
        v[i] = key < end ? v[i] : VT{};  // rows past the last key (stale, even NaN) must not reach the MFMA
    }
    const uint4 pb = softmax_pair<DT, VPL, kInterior>(x, ok, a.qscale, m, l, acc);
#pragma unroll
    for (int t = 0; t < VPL; ++t) {
      const int w = t >> 1;
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low 16-bit halves
      const uint4 vt = make_uint4(__builtin_amdgcn_perm(vword<VPL>(v[1], w), vword<VPL>(v[0], w), sel),
                                  __builtin_amdgcn_perm(vword<VPL>(v[3], w), vword<VPL>(v[2], w), sel),
                                  __builtin_amdgcn_perm(vword<VPL>(v[5], w), vword<VPL>(v[4], w), sel),
                                  __builtin_amdgcn_perm(vword<VPL>(v[7], w), vword<VPL>(v[6], w), sel));
      acc[t] = Ops::qk(vt, pb, acc[t]);
    }
  };
  auto run_step = [&](const uint4* kra, const uint4* krb, const VT* va_rows, const VT* vb_rows, int key0) {
    if (key0 + 2 * BS <= safe) step(kra, krb, va_rows, vb_rows, key0, std::true_type{});
    else step(kra, krb, va_rows, vb_rows, key0, std::false_type{});
  };

  // Ring of 4 blocks (K in LDS slots, V in register sets), consumed two at a
  // time: while a pair is computed the next pair's loads are in flight.  Loads
  // past the partition go through an empty descriptor, so every wait is an
  // exact count; steps past the end run fully masked.
  static_assert(NBUF == 4, "the pair ring has four slots");
  VT vr[4][4];
  load_block(0, 0, vr[0]);
  load_block(1, 1, vr[1]);
  load_block(2, 2, vr[2]);
  for (int j = 0; j < nblk; j += 4) {
    uint4 ka[NKC], kb2[NKC];
    read_k(0, ka);
    read_k(1, kb2);
    load_block(j + 3, 3, vr[3]);
    __builtin_amdgcn_sched_barrier(0);
    run_step(ka, kb2, vr[0], vr[1], start + j * BS);
    load_block(j + 4, 0, vr[0]);
    read_k(2, ka);
    read_k(3, kb2);
    load_block(j + 5, 1, vr[1]);
    __builtin_amdgcn_sched_barrier(0);
    run_step(ka, kb2, vr[2], vr[3], start + (j + 2) * BS);
    load_block(j + 6, 2, vr[2]);
  }

  const float lt = rows_sum(l);
  if (live) store_column<DT, D>(a, acc, m, lt, qrow, s, col_parts, gq);
}


// Cooperative form for wide column ranges (long varlen rows, chunked
// prefill): the waves of a workgroup take 16 * TILES consecutive columns each
// of one (sequence, KV head unit) and share one copy of each K/V block.  The
// blocks stream through an LDS ring of 2 * NP blocks, K and V each with its
// own chunk swizzle, filled by direct-to-LDS loads that the waves split
// between them; one barrier per two-block step publishes a pair and frees the
// pair read in the step before.  Each wave reads K (the QK A operand) and V
// transposed (the P.V A operand) from LDS once per step and applies them to
// all of its tiles.
// Arithmetic per tile follows prefill_mfma_kernel (32-key steps, P.V on
// 16x16x32, lazily moved running max, mask-free interior steps), ordered by
// phase over the wave's tiles, with the softmax denominators summed by an
// extra MFMA per tile.
// WAVES waves of TILES 16-column tiles each: 128 columns for long runs of new
// tokens (4 x 2; 8 waves measured 6% slower), 64 or 32 for short ones (2 x 2,
// 2 x 1).
template <int DT, int D, int NP, int MODE, int WAVES, int TILES>
__global__ __launch_bounds__(64 * WAVES) void prefill_wg_kernel(const PrefillArgs a) {
  constexpr int kWaveTiles = TILES;               // 16-column MFMA tiles per wave
  constexpr int kWaveCols = 16 * kWaveTiles;      // columns per wave
  constexpr int kWgWaves = WAVES;                 // waves per workgroup
  constexpr int kWgCols = kWaveCols * kWgWaves;   // columns per workgroup
  // The 2-wave shapes cover every column of a (sequence, unit) in one
  // workgroup, so each K block is read once: K streams non-temporal as in
  // decode.  The 4-wave shape's column groups re-read a sequence's blocks
  // through L2, so its loads keep the default policy.
  constexpr int kKPol = WAVES == 2 ? kKCpol : 0;
  constexpr bool SUB = MODE == kBlocksLarge;
  constexpr bool GATHER = MODE == kBlocksSmall;
  using Ops = MfmaOps<DT>;
  constexpr int BS = pa::kBlockSize;
  constexpr int ROWB = D * 2;
  constexpr int NKC = D / 32;
  constexpr int VPL = D / 16;
  constexpr int CPR = ROWB / 16;            // 16-byte chunks per row
  constexpr int KI = BS * CPR / 64;         // load instructions per block for K (and for V)
  // load instructions per block and wave: K and V split over the waves (with
  // more waves than instructions the last waves issue none)
  constexpr int DPW = (2 * KI + kWgWaves - 1) / kWgWaves;
  constexpr int KBYTES = BS * ROWB;
  static_assert(BS == 16 && (2 * KI) % DPW == 0, "tile shape");
  static_assert(NP == 3 || NP == 4, "the ring is unrolled for three or four pairs");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: scalar load shares, no waterfall
  const int gq = lane >> 4, col = lane & 15;
  int rest = xcd_remap(blockIdx.x, gridDim.x);
  const int s = rest % a.num_parts;
  rest /= a.num_parts;
  const int k = rest % a.tiles;  // column group
  rest /= a.tiles;
  const int unit = rest % a.groups;  // (KV head, chunk of query heads)
  const int b = rest / a.groups;
  const int g = unit / a.chunks;

  const int q0 = a.query_start_loc ? a.query_start_loc[b] : b;
  const int n = a.query_start_loc ? a.query_start_loc[b + 1] - q0 : 1;
  const int L = a.context_lens[b];
  const int kb = a.key_begin ? a.key_begin[b] : 0;
  const int trow = a.table_rows ? a.table_rows[b] : b;
  if ((kWgCols * k) / a.repc >= n) return;  // the whole workgroup lies past this sequence's rows
  const int last_tok = min(n - 1, (kWgCols * k + kWgCols - 1) / a.repc);
  const int start = kb + s * a.part_tokens;
  const int pend = min(L, start + a.part_tokens);
  const int end = min(pend, a.causal ? L - n + last_tok + 1 : L);  // keys any column here sees

  // This lane's two columns.
  int pos[kWaveTiles], lim[kWaveTiles], col_parts[kWaveTiles];
  bool live[kWaveTiles];
  size_t qrow[kWaveTiles];
#pragma unroll
  for (int tt = 0; tt < kWaveTiles; ++tt) {
    const int cc = kWgCols * k + kWaveCols * wave + 16 * tt + col;
    const int ti = cc / a.repc;
    live[tt] = ti < n;
    const int h = g * a.rep + (unit % a.chunks) * a.repc + cc % a.repc;
    pos[tt] = a.causal ? L - n + ti : L - 1;
    qrow[tt] = (size_t)(q0 + (live[tt] ? ti : 0)) * a.num_heads + h;
    lim[tt] = live[tt] ? min(pend, pos[tt] + 1) : 0;
    col_parts[tt] = (pos[tt] - kb + a.part_tokens) / a.part_tokens;
  }
  if (start >= end) {  // uniform over the workgroup
    if (a.partial_base >= 0)
#pragma unroll
      for (int tt = 0; tt < kWaveTiles; ++tt)
        if (live[tt]) store_empty_slot<D>(a, qrow[tt], s, gq);
    return;
  }
  // Steps wholly below `safe` need no masks for this wave's columns.
  const int wave_tok = (kWgCols * k + kWaveCols * wave) / a.repc;
  const int safe = wave_tok < n ? min(pend, a.causal ? L - n + wave_tok + 1 : L) : end;
  const int pshift = MODE != kBlocks16 ? a.block_shift : 0;
  const int pool_bs = SUB ? BS << pshift : GATHER ? BS >> pshift : BS;  // tokens per pool block
  const int blk0 = start / pool_bs;  // partitions start on a pool block
  const int nblk = (end - start + BS - 1) / BS;  // 16-token steps
  const int nent = MODE == kBlocks16 ? nblk : (end - start + pool_bs - 1) / pool_bs;
  const int last = nblk - 1;

  const int32_t* bt = a.block_tables + (size_t)trow * a.max_blocks_per_seq + blk0;
  TableSlice tab;  // blocks of 16 tokens or more: the slice in VGPR lanes
  TableWindow twin;  // read forward only: the steps' blocks come in order
  __shared__ int32_t stab[GATHER ? pa::kMaxSmallBlockPartition : 1];  // small blocks: in LDS
  if constexpr (GATHER) {
    stage_table(stab, bt, nent);
  } else {
    tab.load(bt, nent, lane);
    twin.init(tab);
  }

  uint4 qop[kWaveTiles][NKC];
#pragma unroll
  for (int tt = 0; tt < kWaveTiles; ++tt) {
    const uint8_t* qp = (const uint8_t*)a.query + qrow[tt] * ROWB + gq * 16;
#pragma unroll
    for (int c = 0; c < NKC; ++c) qop[tt][c] = query_chunk(qp + c * 64, live[tt], a.qneg);
  }

  // This wave's share of every block's loads: instructions wave*DPW ..
  // +DPW of the 2*KI (the first KI fill K, the rest V); lane l of
  // instruction i fills LDS chunk 64*(i mod KI) + l = (row t, position q):
  // K with the row's chunk q ^ swizzle(t), V with chunk q.
  const uint32_t row_stride = a.row_stride;
  const uint32_t hoff = (uint32_t)g * a.head_stride;
  const size_t block_stride = (size_t)a.block_stride;
  const size_t step_stride = (size_t)BS * row_stride;  // 16-token windows inside a larger block
  uint32_t goff[DPW];
  bool is_k[DPW], has[DPW];
  int lds_off[DPW], rblk[DPW];  // rblk: with small blocks, the row's block within the step
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int ins = wave * DPW + i;
    has[i] = (2 * KI) % kWgWaves == 0 || ins < 2 * KI;  // every wave loads when the split is even
    is_k[i] = ins < KI;
    const int idx = is_k[i] ? ins : ins - KI;
    const int sl = 64 * idx + lane, t = sl / CPR, q = sl % CPR;
    const int tr = GATHER ? t % pool_bs : t;  // the row inside its pool block
    rblk[i] = GATHER ? t / pool_bs : 0;
    goff[i] = (uint32_t)tr * row_stride + hoff + (uint32_t)((q ^ (is_k[i] ? kswz_t<CPR>(t) : vswz_t<CPR>(t))) * 16);
    lds_off[i] = idx * 1024;
  }
  uint32_t kread[NKC];  // QK A operand: token 4*(col%4) + col/4, chunk 4c + gq
  {
    const int t = 4 * (col & 3) + (col >> 2);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kread[c] = (uint32_t)(t * CPR + ((4 * c + gq) ^ kswz_t<CPR>(t))) * 16;
  }
  // P.V A operand of output tile t (dims 16t + col) by transposed reads: this
  // lane addresses row 4(col / 4) + gq, dims 16t + 4(col % 4) .. + 3, so that
  // lane (gq, col) receives that dim of rows gq, gq + 4, gq + 8, gq + 12.
  uint32_t vtr[VPL];
  {
    const int r = 4 * (col >> 2) + gq;
#pragma unroll
    for (int t = 0; t < VPL; ++t)
      vtr[t] = (uint32_t)(r * ROWB + ((2 * t + ((col & 3) >> 1)) ^ vswz_t<CPR>(r)) * 16 + (col & 1) * 8);
  }

  constexpr int XB = NP > 3 ? KBYTES : 16;  // slots 6 and 7 exist with four pairs
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[KBYTES], ks1[KBYTES], ks2[KBYTES], ks3[KBYTES],
      ks4[KBYTES], ks5[KBYTES], ks6[XB], ks7[XB];
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[KBYTES], vs1[KBYTES], vs2[KBYTES], vs3[KBYTES],
      vs4[KBYTES], vs5[KBYTES], vs6[XB], vs7[XB];
  auto kslot = [&](int x) -> uint8_t* {
    return x == 0 ? ks0 : x == 1 ? ks1 : x == 2 ? ks2 : x == 3 ? ks3 : x == 4 ? ks4 : x == 5 ? ks5 : x == 6 ? ks6 : ks7;
  };
  auto vslot = [&](int x) -> uint8_t* {
    return x == 0 ? vs0 : x == 1 ? vs1 : x == 2 ? vs2 : x == 3 ? vs3 : x == 4 ? vs4 : x == 5 ? vs5 : x == 6 ? vs6 : vs7;
  };

  f32x4 acc[kWaveTiles][VPL];
#pragma unroll
  for (int tt = 0; tt < kWaveTiles; ++tt)
#pragma unroll
    for (int t = 0; t < VPL; ++t) acc[tt][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[kWaveTiles], mth[kWaveTiles];  // running max (log2 units), and m + kRescaleLog2
  f32x4 lacc[kWaveTiles];  // every register: the column's denominator
#pragma unroll
  for (int tt = 0; tt < kWaveTiles; ++tt) {
    m[tt] = kMaxFloor;
    mth[tt] = kMaxFloor + kRescaleLog2;
    lacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Loads past the partition go through an empty descriptor (zeros, no
  // memory access), so every wait count is exact; with small blocks
  // (per-lane addresses) they re-read the last step's rows instead, which
  // the step past `end` never uses.
  // A wave's loads are all of K or all of V (its DPW instructions never
  // straddle the K | V boundary), so one pool base and descriptor serve it.
  static_assert(KI % DPW == 0, "a wave's share of a block's loads is of one kind");
  const bool wave_k = is_k[0];
  const uint8_t* const wave_pool = wave_k ? a.k_pool : a.v_pool;
  const uint32_t bstride32 = (uint32_t)a.block_stride;  // <= 2^31 (checked on the host)
  auto load_block = [&](int j, int x) {
    const bool real = j <= last;
    const int jj = real ? j : last;
    if constexpr (GATHER) {
      size_t base[DPW];
      step_block_bases<DPW>(stab, jj, pshift, nent, block_stride, rblk, base);
#pragma unroll
      for (int i = 0; i < DPW; ++i) {
        if (!has[i]) continue;
        const uint8_t* src = (is_k[i] ? a.k_pool : a.v_pool) + base[i] + goff[i];
        auto* dst = (__attribute__((address_space(3))) void*)((is_k[i] ? kslot(x) : vslot(x)) + lds_off[i]);
        if (is_k[i])  // wave-uniform
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src, dst, 16, 0, kKPol);
        else
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src, dst, 16, 0, 0);
      }
      return;
    }
    const size_t off = SUB ? (size_t)(uint32_t)twin.get(tab, jj >> pshift) * bstride32 +
                                 (size_t)(jj & ((1 << pshift) - 1)) * step_stride
                           : (size_t)(uint32_t)twin.get(tab, jj) * bstride32;
    const uint32_t span = real ? a.span : 0u;
    const __amdgpu_buffer_rsrc_t r = make_block_rsrc(wave_pool + off, span);
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      if (!has[i]) continue;
      if (wave_k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(kslot(x) + lds_off[i]),
                                                 16, (int)goff[i], 0, 0, kKPol);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(vslot(x) + lds_off[i]),
                                                 16, (int)goff[i], 0, 0, 0);
    }
  };

  // One pair of blocks from ring slots xa, xb whose first key is key0.
  auto step = [&](int xa, int xb, int key0, auto interior) {
    constexpr bool kInterior = decltype(interior)::value;
    uint4 kra[NKC], krb[NKC];
    uint2 va[VPL], vb[VPL];  // keys 4k + gq of block A (B), k = 0..3, at dim 16t + col
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      kra[c] = *reinterpret_cast<const uint4*>(kslot(xa) + kread[c]);
      krb[c] = *reinterpret_cast<const uint4*>(kslot(xb) + kread[c]);
    }
#pragma unroll
    for (int t = 0; t < VPL; ++t) {
      va[t] = lds_read_tr16(vslot(xa) + vtr[t]);
      vb[t] = lds_read_tr16(vslot(xb) + vtr[t]);
    }
    if constexpr (!kInterior) {  // rows past the last key (stale, even NaN) must not reach the MFMA
      auto keep = [&](int k0) {
        return (k0 + gq < end ? 0xffffu : 0u) | (k0 + 4 + gq < end ? 0xffff0000u : 0u);
      };
      const uint2 ma = make_uint2(keep(key0), keep(key0 + 8)), mb = make_uint2(keep(key0 + 16), keep(key0 + 24));
#pragma unroll
      for (int t = 0; t < VPL; ++t) {
        va[t] = make_uint2(va[t].x & ma.x, va[t].y & ma.y);
        vb[t] = make_uint2(vb[t].x & mb.x, vb[t].y & mb.y);
      }
    }
    // Scores of every tile first, so the second tile's QK MFMAs overlap the
    // first tile's max; then one wave-uniform branch for all tiles' rare
    // rescales; then each tile's probabilities and its P.V MFMAs, so the next
    // tile's exponentials overlap this tile's matrix work.
    float x[kWaveTiles][8];
#pragma unroll
    for (int tt = 0; tt < kWaveTiles; ++tt) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NKC; ++c) {
        sa = Ops::qk(kra[c], qop[tt][c], sa);
        sb = Ops::qk(krb[c], qop[tt][c], sb);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[tt][i] = sa[i];
        x[tt][4 + i] = sb[i];
      }
    }
    auto visible = [&](int tt, int i) {
      return kInterior || key0 + (i >> 2) * 16 + 4 * (i & 3) + gq < lim[tt];
    };
    // The test for a move looks at the lane's own 8 scores: some lane's max
    // passes the threshold exactly when its column's max does (scaling by
    // qscale >= 0 and rounding keep the order), so the column max across the
    // four lane groups is taken only inside the rare branch.
    float lmax[kWaveTiles];
    bool move = false;
#pragma unroll
    for (int tt = 0; tt < kWaveTiles; ++tt) {
      float xm[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) xm[i] = visible(tt, i) ? x[tt][i] : -INFINITY;
      lmax[tt] = max8(xm);
      move = move || lmax[tt] * a.qscale > mth[tt];
    }
    if (__ballot(move)) {  // rare: some column's max moved by more than 2^8
#pragma unroll
      for (int tt = 0; tt < kWaveTiles; ++tt) {
        const float mn = fmaxf(m[tt], rows_maximum(lmax[tt]) * a.qscale);
        const float alpha = fast_exp2(m[tt] - mn);
        m[tt] = mn;
        mth[tt] = mn + kRescaleLog2;
        lacc[tt] *= alpha;
#pragma unroll
        for (int t = 0; t < VPL; ++t) acc[tt][t] *= alpha;
      }
    }
    // The P.V MFMAs issue at raised wave priority: the wave's independent
    // MFMAs go out back to back while the SIMD's other wave (another
    // workgroup's) runs its softmax beside them.  Measured 3% faster on
    // chunked prefill; the same around the QK MFMAs gained nothing.
    // The softmax denominators come from the matrix core too: a 16 x 32 block
    // of ones times P^T gives every row of lacc the column's sum of the same
    // rounded probabilities P.V weighs, one MFMA per tile instead of 8 adds.
    constexpr uint32_t one2 = DT == DT_BF16 ? 0x3f803f80u : 0x3c003c00u;  // two 16-bit 1.0
    const uint4 ones = make_uint4(one2, one2, one2, one2);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int tt = 0; tt < kWaveTiles; ++tt) {
      const float nm = -m[tt];
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e = fast_exp2(fmaf(x[tt][i], a.qscale, nm));
        p[i] = visible(tt, i) ? e : 0.f;  // absent keys: a select, not -inf * scale
      }
      const uint4 pb = make_uint4(Ops::pack(p[0], p[1]), Ops::pack(p[2], p[3]), Ops::pack(p[4], p[5]),
                                  Ops::pack(p[6], p[7]));
#pragma unroll
      for (int t = 0; t < VPL; ++t)
        acc[tt][t] = Ops::qk(make_uint4(va[t].x, va[t].y, vb[t].x, vb[t].y), pb, acc[tt][t]);
      lacc[tt] = Ops::qk(ones, pb, lacc[tt]);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // One ring step over pair p, held in ring pair `sp` (slots 2sp, 2sp+1):
  // wait for this wave's loads of it, barrier (every wave's loads of it have
  // landed and every wave has finished the previous step), refill the
  // previous step's pair with the blocks 2*(NP-1) ahead, then compute.
  auto ring_step = [&](auto sp, int p, auto interior) {
    constexpr int xa = 2 * decltype(sp)::value, xp = 2 * ((decltype(sp)::value + NP - 1) % NP);
    wait_vmcnt<(NP - 2) * 2 * DPW>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    load_block(2 * p + 2 * (NP - 1), xp);
    load_block(2 * p + 2 * (NP - 1) + 1, xp + 1);
    __builtin_amdgcn_sched_barrier(0);
    step(xa, xa + 1, start + 2 * p * BS, interior);
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;

  // Pairs with a key below `end` run, the others are never started (the
  // step count is the same for every wave, so the barriers match).  Pairs
  // wholly below this wave's `safe` take the unmasked step, in whole turns of
  // the ring, so that loop is straight-line code; the rest (the causal edge,
  // the partition's last pair, a turn's remainder) take the masked one, also
  // in turns of the ring (a step chosen per pair by its slot would keep the
  // registers of every slot's variant live: occupancy 1 instead of 2).
  const int npairs = (nblk + 1) / 2;
  const int nint = min(npairs, max(0, (safe - start) / (2 * BS)));
#pragma unroll
  for (int x = 0; x < 2 * (NP - 1); ++x) load_block(x, x);
  int p = 0;
  for (; p + NP <= nint; p += NP) {
    ring_step(C0{}, p, std::true_type{});
    ring_step(C1{}, p + 1, std::true_type{});
    ring_step(C2{}, p + 2, std::true_type{});
    if constexpr (NP == 4) ring_step(C3{}, p + 3, std::true_type{});
  }
  for (; p < npairs; p += NP) {
    ring_step(C0{}, p, std::false_type{});
    if (p + 1 < npairs) ring_step(C1{}, p + 1, std::false_type{});
    if (p + 2 < npairs) ring_step(C2{}, p + 2, std::false_type{});
    if constexpr (NP == 4)
      if (p + 3 < npairs) ring_step(C3{}, p + 3, std::false_type{});
  }
  wait_vmcnt<0>();  // no load into this workgroup's LDS outlives it

#pragma unroll
  for (int tt = 0; tt < kWaveTiles; ++tt) {
    const float lt = lacc[tt][0];
    if (live[tt]) store_column<DT, D, true>(a, acc[tt], m[tt], lt, qrow[tt], s, col_parts[tt], gq);
  }
}

// One wave per (query row, head): the sequence of row t is found by binary
// search over query_start_loc; rows whose keys fit one partition were written
// by the partition kernel.
template <int DT, int D>
__global__ __launch_bounds__(256) void prefill_combine_kernel(void* __restrict__ out, const float* __restrict__ ws_acc,
                                                              const float2* __restrict__ ws_ml,
                                                              const int32_t* __restrict__ context_lens,
                                                              const int32_t* __restrict__ query_start_loc,
                                                              int num_seqs, int num_tokens, int num_heads,
                                                              int part_tokens, int num_parts) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (idx >= num_tokens * num_heads) return;
  const int t = idx / num_heads;
  int lo = 0, hi = num_seqs;  // largest b with query_start_loc[b] <= t
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (query_start_loc[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int q0 = query_start_loc[lo], n = query_start_loc[lo + 1] - q0;
  if (t >= q0 + n) return;  // a row no sequence owns
  const int pos = context_lens[lo] - n + (t - q0);
  const int np = (pos + part_tokens) / part_tokens;
  if (np <= 1) return;
  merge_partials<DT, D>((uint8_t*)out + (size_t)idx * D * ElemBytes<DT>::value, ws_acc + (size_t)idx * num_parts * D,
                        ws_ml + (size_t)idx * num_parts, np, lane);
}

// One wave per (row, head): merges `slots` partials (empty ones hold m = -inf).
template <int DT, int D>
__global__ __launch_bounds__(256) void merge_slots_kernel(void* __restrict__ out, const float* __restrict__ ws_acc,
                                                          const float2* __restrict__ ws_ml, int rows_heads,
                                                          int slots) {
  const int lane = threadIdx.x & 63;
  const int idx = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (idx >= rows_heads) return;
  merge_partials<DT, D>((uint8_t*)out + (size_t)idx * D * ElemBytes<DT>::value, ws_acc + (size_t)idx * slots * D,
                        ws_ml + (size_t)idx * slots, slots, lane);
}

using PrefillFn = void (*)(const PrefillArgs);
using MergeSlotsFn = void (*)(void*, const float*, const float2*, int, int);

MergeSlotsFn pick_merge_slots(int dtype, int d) {
  switch (dtype) {
    case PA_F16: return d == 64 ? merge_slots_kernel<DT_F16, 64> : merge_slots_kernel<DT_F16, 128>;
    case PA_BF16: return d == 64 ? merge_slots_kernel<DT_BF16, 64> : merge_slots_kernel<DT_BF16, 128>;
    default: return nullptr;
  }
}
using PrefillCombineFn = void (*)(void*, const float*, const float2*, const int32_t*, const int32_t*, int, int, int,
                                  int, int);
constexpr int kPrefillRing = 4;

template <int DT, int D, int MODE>
PrefillFn pick_prefill_wpw(int wpw) {
  switch (wpw) {
    case 1: return prefill_mfma_kernel<DT, D, kPrefillRing, 1, MODE>;
    case 2: return prefill_mfma_kernel<DT, D, kPrefillRing, 2, MODE>;
    case 4: return prefill_mfma_kernel<DT, D, kPrefillRing, 4, MODE>;
    default: return nullptr;
  }
}

template <int DT, int D>
PrefillFn pick_prefill_bs(int wpw, int block_size) {
  if (block_size == pa::kBlockSize) return pick_prefill_wpw<DT, D, kBlocks16>(wpw);
  if (block_size > pa::kBlockSize) return pick_prefill_wpw<DT, D, kBlocksLarge>(wpw);
  return pick_prefill_wpw<DT, D, kBlocksSmall>(wpw);
}

#ifndef PA_PREFILL_PAIRS
#define PA_PREFILL_PAIRS 3
#endif
// Ring pairs of the cooperative tile: the 4-wave shape (compute bound) keeps
// three (48 KiB of LDS; a fourth measured the same).  The 2-wave shapes of
// pa_prefill_attention (bandwidth bound: several new tokens per sequence,
// grids of many workgroups per compute unit) take four, one more pair of
// loads in flight (8 and 16 new tokens per sequence: 5% and 3% faster); the
// cascade's prefix pass keeps three, so that three workgroups fit a compute
// unit (2400-token prompts: 86 us with three, 104 us with four).
constexpr int kPrefillPairs = PA_PREFILL_PAIRS;
constexpr int kPrefillPairsDeep = 4;

template <int DT, int D, int WAVES, int TILES, bool DEEP>
PrefillFn pick_prefill_wide_bs(int block_size) {
  constexpr int NP = WAVES == 2 && DEEP ? kPrefillPairsDeep : kPrefillPairs;
  if (block_size == pa::kBlockSize) return prefill_wg_kernel<DT, D, NP, kBlocks16, WAVES, TILES>;
  if (block_size > pa::kBlockSize) return prefill_wg_kernel<DT, D, NP, kBlocksLarge, WAVES, TILES>;
  return prefill_wg_kernel<DT, D, NP, kBlocksSmall, WAVES, TILES>;
}

template <int DT, int D>
PrefillFn pick_prefill_wide_shape(const pa::PrefillGrid& g, int block_size, bool deep) {
  if (g.waves == 2 && g.wave_tiles == 1)
    return deep ? pick_prefill_wide_bs<DT, D, 2, 1, true>(block_size) : pick_prefill_wide_bs<DT, D, 2, 1, false>(block_size);
  if (g.waves == 2 && g.wave_tiles == 2)
    return deep ? pick_prefill_wide_bs<DT, D, 2, 2, true>(block_size) : pick_prefill_wide_bs<DT, D, 2, 2, false>(block_size);
  if (g.waves == pa::kPrefillWgWaves && g.wave_tiles == pa::kPrefillWaveTiles)
    return pick_prefill_wide_bs<DT, D, pa::kPrefillWgWaves, pa::kPrefillWaveTiles, false>(block_size);
  return nullptr;
}

// deep: the 2-wave shapes with four ring pairs (see kPrefillPairsDeep).
PrefillFn pick_prefill_wide(int dtype, int d, const pa::PrefillGrid& g, int block_size, bool deep) {
  switch (dtype) {
    case PA_F16:
      return d == 64 ? pick_prefill_wide_shape<DT_F16, 64>(g, block_size, deep)
                     : pick_prefill_wide_shape<DT_F16, 128>(g, block_size, deep);
    case PA_BF16:
      return d == 64 ? pick_prefill_wide_shape<DT_BF16, 64>(g, block_size, deep)
                     : pick_prefill_wide_shape<DT_BF16, 128>(g, block_size, deep);
    default: return nullptr;
  }
}

PrefillFn pick_prefill(int dtype, int d, int wpw, int block_size) {
  switch (dtype) {
    case PA_F16:
      return d == 64 ? pick_prefill_bs<DT_F16, 64>(wpw, block_size) : pick_prefill_bs<DT_F16, 128>(wpw, block_size);
    case PA_BF16:
      return d == 64 ? pick_prefill_bs<DT_BF16, 64>(wpw, block_size) : pick_prefill_bs<DT_BF16, 128>(wpw, block_size);
    default: return nullptr;
  }
}

PrefillCombineFn pick_prefill_combine(int dtype, int d) {
  switch (dtype) {
    case PA_F32: return d == 64 ? prefill_combine_kernel<DT_F32, 64> : prefill_combine_kernel<DT_F32, 128>;
    case PA_F16: return d == 64 ? prefill_combine_kernel<DT_F16, 64> : prefill_combine_kernel<DT_F16, 128>;
    case PA_BF16: return d == 64 ? prefill_combine_kernel<DT_BF16, 64> : prefill_combine_kernel<DT_BF16, 128>;
    default: return nullptr;
  }
}

size_t prefill_workspace(const pa::PrefillShape& s, int parts) {
  return pa::workspace_bytes(s.num_tokens, s.d.num_heads, s.d.head_dim, parts);
}

// fp32: the column tile - the columns of a (sequence, KV head) are its (new
// token, query head) pairs, 16 per wave on the matrix cores, each with its
// own causal key limit; the waves of a workgroup take consecutive columns,
// so a sequence's rows share each K/V read of a wave and its workgroup's
// waves read the same blocks together.  Partials merged as for the 16-bit
// tiles.
int prefill_rows(void* out, const void* query, const pa::PoolView& pv, const int32_t* block_tables,
                 const int32_t* context_lens, const int32_t* query_start_loc, const pa::PrefillShape& shp,
                 float scale, void* workspace, size_t workspace_bytes, int32_t partition_size, void* stream) {
  const pa::DecodeShape& d = shp.d;
  const pa::ColumnGrid cg = pa::column_grid(shp);
  int cus = 256, per_cu = 1;
  if (partition_size == 0) {
    int threads = 0;
    const void* fn = pa::columns_kernel(shp, &threads);
    if (!fn) return PA_ERR_UNSUPPORTED;
    cus = pa::device_cu_count();
    per_cu = pa::resident_per_cu(fn, threads);
    if (cus <= 0 || per_cu <= 0) return PA_ERR_HIP;
  }
  const int ps = pa::prefill_partition_size_for(shp, cg.items, cg.wpw, partition_size, cus, per_cu);
  if (ps <= 0) return -ps;
  const int parts = pa::num_partitions(d.max_context_len, ps);
  const size_t need = prefill_workspace(shp, parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  float* ws_acc = parts > 1 ? static_cast<float*>(workspace) : nullptr;
  float2* ws_ml = parts > 1 ? reinterpret_cast<float2*>(static_cast<float*>(workspace) +
                                                        (size_t)shp.num_tokens * d.num_heads * parts * d.head_dim)
                            : nullptr;
  int rc = pa::launch_columns(out, query, pv, block_tables, context_lens, query_start_loc, shp, scale, ws_acc,
                              ws_ml, ps, parts, stream);
  if (rc != PA_OK || parts <= 1) return rc;
  PrefillCombineFn cf = pick_prefill_combine(d.dtype, d.head_dim);
  if (!cf) return PA_ERR_UNSUPPORTED;
  const int64_t waves = (int64_t)shp.num_tokens * d.num_heads;
  return pa::launch_kernel(cf, dim3((unsigned)((waves + 3) / 4)), dim3(256), static_cast<hipStream_t>(stream), out,
                           ws_acc, ws_ml, context_lens, query_start_loc, d.num_seqs, shp.num_tokens, d.num_heads, ps,
                           parts);
}

// Scores are scaled by |scale| (in log2 units for exp2); a negative scale
// flips the query's signs instead, so the tiles' running max of the raw
// scores stays the max of the scaled ones.
void set_scale(PrefillArgs* a, float scale) {
  a->qscale = std::fabs(scale) * 1.44269504088896340736f;  // log2(e)
  a->qneg = scale < 0.f;
}

void set_pool(PrefillArgs* a, const pa::PoolView& pv, const pa::DecodeShape& s) {
  a->k_pool = pv.k;
  a->v_pool = pv.v;
  a->block_shift = pa::block_shift(s.block_size);
  a->block_stride = pv.block_stride;
  a->row_stride = (uint32_t)pv.row_stride;
  a->head_stride = (uint32_t)pv.head_stride;
  a->span = (uint32_t)pv.step_span(s.head_dim * pa::elem_bytes(s.dtype), s.num_kv_heads);
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" size_t pa_prefill_workspace_bytes(int32_t num_tokens, int32_t num_heads, int32_t head_dim,
                                             int32_t max_context_len, int32_t block_size, int32_t partition_size) {
  if (num_tokens <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || block_size <= 0) return 0;
  pa::PrefillShape s{{1, num_heads, 1, head_dim, block_size, 1 << 30, max_context_len, PA_BF16}, num_tokens, 1};
  int parts;
  if (partition_size == 0) {
    int lo = 1;
    pa::prefill_partition_bounds(s, &lo, &parts);
  } else {
    if (pa::validate_prefill_partition(partition_size, block_size) < 0) return 0;
    parts = pa::num_partitions(max_context_len, partition_size);
  }
  return prefill_workspace(s, parts);
}

extern "C" int pa_prefill_attention_layout(void* out, const void* query, const void* k_pool, const void* v_pool,
                                           const int32_t* block_tables, const int32_t* context_lens,
                                           const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                           int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                                           int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                           int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                                           size_t workspace_bytes, int32_t partition_size, pa_kv_layout layout,
                                           void* stream) {
  if (num_tokens == 0) return PA_OK;  // no new tokens
  const pa::PrefillShape shp{{num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              max_context_len, (int)dtype},
                             num_tokens,
                             max_query_len};
  int rc = pa::check_prefill(out, query, k_pool, layout == PA_KV_FUSED ? k_pool : v_pool, block_tables,
                             context_lens, query_start_loc, shp, scale);
  if (rc != PA_OK) return rc;
  pa::PoolView pv;
  rc = pa::pool_view(k_pool, v_pool, (int)layout, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
  if (dtype == PA_F32)
    return prefill_rows(out, query, pv, block_tables, context_lens, query_start_loc, shp, scale, workspace,
                        workspace_bytes, partition_size, stream);
  const pa::DecodeGrid gd = pa::decode_grid(shp.d);
  const pa::PrefillGrid pg = pa::prefill_grid(shp);
  PrefillFn fn = pg.wide ? pick_prefill_wide(shp.d.dtype, shp.d.head_dim, pg, block_size, true)
                         : pick_prefill(shp.d.dtype, shp.d.head_dim, gd.wpw, block_size);
  if (!fn) return PA_ERR_UNSUPPORTED;
  int cus = 256, per_cu = 1;
  if (partition_size == 0) {
    cus = pa::device_cu_count();
    per_cu = pa::resident_per_cu(reinterpret_cast<const void*>(fn), 64 * pg.waves);
    if (cus <= 0 || per_cu <= 0) return PA_ERR_HIP;
  }
  const int ps = pa::prefill_partition_size(shp, partition_size, cus, per_cu);
  if (ps <= 0) return -ps;
  const int parts = pa::num_partitions(max_context_len, ps);
  const size_t need = prefill_workspace(shp, parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const int64_t grid = pg.items * parts;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;

  PrefillArgs a;
  set_pool(&a, pv, shp.d);
  a.out = out;
  a.query = query;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start_loc = query_start_loc;
  a.table_rows = nullptr;
  a.key_begin = nullptr;
  a.causal = 1;
  a.partial_base = -1;
  a.partial_stride = parts;
  a.ws_acc = parts > 1 ? static_cast<float*>(workspace) : nullptr;
  a.ws_ml = parts > 1 ? reinterpret_cast<float2*>(static_cast<float*>(workspace) +
                                                  (size_t)num_tokens * num_heads * parts * head_dim)
                      : nullptr;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.rep = gd.rep;
  a.repc = gd.repc;
  a.chunks = gd.chunks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.part_tokens = ps;
  a.num_parts = parts;
  a.groups = pg.groups;
  a.tiles = pg.tiles;
  set_scale(&a, scale);
  hipStream_t st = static_cast<hipStream_t>(stream);
  rc = pa::launch_kernel(fn, dim3((unsigned)grid), dim3(64 * pg.waves), st, a);
  if (rc != PA_OK || parts <= 1) return rc;
  PrefillCombineFn cf = pick_prefill_combine(shp.d.dtype, shp.d.head_dim);
  if (!cf) return PA_ERR_UNSUPPORTED;
  const int64_t waves = (int64_t)num_tokens * num_heads;
  return pa::launch_kernel(cf, dim3((unsigned)((waves + 3) / 4)), dim3(256), st, out, a.ws_acc, a.ws_ml,
                           context_lens, query_start_loc, num_seqs, num_tokens, num_heads, ps, parts);
}

extern "C" int pa_prefill_attention(void* out, const void* query, const void* k_pool, const void* v_pool,
                                    const int32_t* block_tables, const int32_t* context_lens,
                                    const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                    int32_t max_query_len, int32_t num_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
                                    int32_t max_context_len, float scale, pa_dtype dtype, void* workspace,
                                    size_t workspace_bytes, int32_t partition_size, void* stream) {
  if (!v_pool) return PA_ERR_INVALID_ARG;
  return pa_prefill_attention_layout(out, query, k_pool, v_pool, block_tables, context_lens, query_start_loc,
                                     num_seqs, num_tokens, max_query_len, num_heads, num_kv_heads, head_dim,
                                     block_size, max_blocks_per_seq, max_context_len, scale, dtype, workspace,
                                     workspace_bytes, partition_size, PA_KV_SPLIT, stream);
}

// ------------------------------------------------------------------ shared-prefix decode

extern "C" size_t pa_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                                   int32_t max_context_len, int32_t max_prefix_len) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || max_prefix_len < 0 ||
      max_prefix_len > max_context_len)
    return 0;
  const int slots = pa::shared_prefix_slots(max_context_len, max_prefix_len);
  return (size_t)num_seqs * num_heads * slots * ((size_t)head_dim + 2) * sizeof(float);
}

extern "C" int pa_decode_attention_shared_prefix_layout(
    void* out, const void* query, const void* k_pool, const void* v_pool, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* group_start, const int32_t* prefix_lens,
    const int32_t* seq_prefix_lens, int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_prefix_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, pa_kv_layout layout, void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch
  const pa::PrefillShape shp{{num_seqs, num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                              max_context_len, (int)dtype},
                             num_seqs,
                             1};
  int rc = pa::check_shared_prefix(out, query, k_pool, layout == PA_KV_FUSED ? k_pool : v_pool, block_tables,
                                   context_lens, group_start, prefix_lens, seq_prefix_lens, shp, num_groups,
                                   max_group_size, max_prefix_len, scale);
  if (rc != PA_OK) return rc;
  const int p1 = pa::num_partitions(std::max(max_prefix_len, 1), pa::kSharedPrefixPartition);
  const int slots = pa::shared_prefix_slots(max_context_len, max_prefix_len);
  const int p2 = slots - p1;
  const size_t need = pa_shared_prefix_workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, max_prefix_len);
  if (workspace == nullptr || workspace_bytes < need) return PA_ERR_WORKSPACE;
  const pa::DecodeGrid gd = pa::decode_grid(shp.d);
  PrefillFn fn = pick_prefill(shp.d.dtype, shp.d.head_dim, gd.wpw, block_size);
  MergeSlotsFn mf = pick_merge_slots(shp.d.dtype, shp.d.head_dim);
  if (!fn || !mf) return PA_ERR_UNSUPPORTED;

  pa::PoolView pv;
  rc = pa::pool_view(k_pool, v_pool, (int)layout, block_size, num_kv_heads, head_dim, (int)dtype, &pv);
  if (rc != PA_OK) return rc;
#ifndef PA_SHARED_PREFIX_SINGLE
#define PA_SHARED_PREFIX_SINGLE 1
#endif
  if (PA_SHARED_PREFIX_SINGLE) {  // one launch when the batch fits it, else the passes below
    rc = pa::launch_shared_prefix_single(out, query, pv, block_tables, context_lens, group_start, prefix_lens, shp.d,
                                         num_groups, max_group_size, scale, stream);
    if (rc != PA_ERR_UNSUPPORTED) return rc;
  }
  PrefillArgs a;
  set_pool(&a, pv, shp.d);
  a.out = out;
  a.query = query;
  a.block_tables = block_tables;
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = reinterpret_cast<float2*>(static_cast<float*>(workspace) + (size_t)num_seqs * num_heads * slots * head_dim);
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.rep = gd.rep;
  a.repc = gd.repc;
  a.chunks = gd.chunks;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.part_tokens = pa::kSharedPrefixPartition;
  a.groups = gd.groups;
  a.partial_stride = slots;
  set_scale(&a, scale);
  hipStream_t st = static_cast<hipStream_t>(stream);

  // Prefix pass: one "sequence" per group whose rows are the members' queries
  // and whose keys are the shared prefix, read through the first member's
  // table; no causal limit inside the prefix (every member's position lies
  // past it).
  // A group whose members bring more than 16 (member, query head) columns
  // per KV head runs the cooperative tile, whose waves share one read of
  // each prefix block - when that still gives two workgroups per compute
  // unit; fewer, larger groups keep the per-wave tile's parallelism.
  a.context_lens = prefix_lens;
  a.query_start_loc = group_start;
  a.table_rows = group_start;
  a.key_begin = nullptr;
  a.causal = 0;
  a.num_parts = p1;
  a.partial_base = 0;
  pa::PrefillShape pre = shp;
  pre.d.num_seqs = num_groups;
  pre.max_query_len = max_group_size;
  pa::PrefillGrid pg = pa::prefill_grid(pre);
  if (pg.wide && pg.items * p1 < 2 * (int64_t)std::max(1, pa::device_cu_count())) {
    pg.wide = false;
    pg.tiles = (int)(((int64_t)max_group_size * gd.repc + 15) / 16);
    pg.groups = gd.groups;
    pg.waves = gd.wpw;
    pg.items = (int64_t)num_groups * pg.tiles * pg.groups;
  }
  PrefillFn pfn = pg.wide ? pick_prefill_wide(shp.d.dtype, shp.d.head_dim, pg, block_size, false) : fn;
  if (!pfn) return PA_ERR_UNSUPPORTED;
  a.groups = pg.groups;
  a.tiles = pg.tiles;
  int64_t grid = pg.items * p1;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  rc = pa::launch_kernel(pfn, dim3((unsigned)grid), dim3(64 * pg.waves), st, a);
  if (rc != PA_OK) return rc;

  // Suffix pass: every sequence's own keys past its group's prefix.
  a.context_lens = context_lens;
  a.query_start_loc = nullptr;
  a.table_rows = nullptr;
  a.key_begin = seq_prefix_lens;
  a.causal = 1;
  a.num_parts = p2;
  a.partial_base = p1;
  a.groups = gd.groups;
  a.tiles = 1;
  grid = (int64_t)num_seqs * p2 * gd.groups;
  if (grid > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  rc = pa::launch_kernel(fn, dim3((unsigned)grid), dim3(64 * gd.wpw), st, a);
  if (rc != PA_OK) return rc;

  const int64_t waves = (int64_t)num_seqs * num_heads;
  return pa::launch_kernel(mf, dim3((unsigned)((waves + 3) / 4)), dim3(256), st, out, a.ws_acc, a.ws_ml,
                           (int)waves, slots);
}

extern "C" int pa_decode_attention_shared_prefix(
    void* out, const void* query, const void* k_pool, const void* v_pool, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* group_start, const int32_t* prefix_lens,
    const int32_t* seq_prefix_lens, int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
    int32_t num_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq,
    int32_t max_context_len, int32_t max_prefix_len, float scale, pa_dtype dtype, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (num_seqs == 0) return PA_OK;  // an empty batch: every pointer may be NULL
  if (!v_pool) return PA_ERR_INVALID_ARG;
  return pa_decode_attention_shared_prefix_layout(out, query, k_pool, v_pool, block_tables, context_lens, group_start,
                                                  prefix_lens, seq_prefix_lens, num_seqs, num_groups, max_group_size,
                                                  num_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                                  max_context_len, max_prefix_len, scale, dtype, workspace,
                                                  workspace_bytes, PA_KV_SPLIT, stream);
}
