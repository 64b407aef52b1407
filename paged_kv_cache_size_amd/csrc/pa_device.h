// Device helpers shared by the libpa kernels (gfx950, wave64): storage
// conversions, lane exchanges, the on-chip block-table slice, the XCD-aware
// workgroup remap, buffer descriptors and the MFMA operand helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_host.h"

namespace {

constexpr int DT_F32 = PA_F32, DT_F16 = PA_F16, DT_BF16 = PA_BF16;

template <int DT>
struct ElemBytes { static constexpr int value = (DT == DT_F32) ? 4 : 2; };

// ------------------------------------------------------------------ numerics

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float f16_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// 16 bytes of storage -> 16 / elem floats
template <int DT>
__device__ __forceinline__ void unpack16(const uint4 v, float* f) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(w[i]);
  } else if constexpr (DT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = f16_bits_to_float(w[i] & 0xffffu);
      f[2 * i + 1] = f16_bits_to_float(w[i] >> 16);
    }
  }
}

// float -> storage bits, round to nearest even
__device__ __forceinline__ uint32_t float_to_bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t float_to_f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

template <int DT, int N>
__device__ __forceinline__ void store_row(uint8_t* dst, const float* f) {
  // N floats -> N elements of storage, written as 16-byte vectors
  if constexpr (DT == DT_F32) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<uint4*>(dst + 4 * i) =
          make_uint4(__float_as_uint(f[i]), __float_as_uint(f[i + 1]), __float_as_uint(f[i + 2]),
                     __float_as_uint(f[i + 3]));
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const uint32_t lo = DT == DT_BF16 ? float_to_bf16_bits(f[2 * i]) : float_to_f16_bits(f[2 * i]);
      const uint32_t hi = DT == DT_BF16 ? float_to_bf16_bits(f[2 * i + 1]) : float_to_f16_bits(f[2 * i + 1]);
      w[i] = lo | (hi << 16);
    }
#pragma unroll
    for (int i = 0; i < N / 2; i += 4)
      *reinterpret_cast<uint4*>(dst + 4 * i) = make_uint4(w[i], w[i + 1], w[i + 2], w[i + 3]);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ lane exchange

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over aligned groups of G lanes (G = 8, 16 or 32); every lane of a group
// ends with the same bits (each step adds a pair in both orders).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm(1,0,3,2): partner lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm(2,3,0,1): partner lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: lane i <-> 7 - i within 8 lanes
  if constexpr (G >= 16) x += dpp<0x140>(x);  // row_mirror: lane i <-> 15 - i within 16
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  static_assert(G == 8 || G == 16 || G == 32, "group size");
  return x;
}

// Reduce over the lanes that differ only in bits >= log2(G) (the row groups).
template <int G>
__device__ __forceinline__ float across_groups_max(float x) {
#pragma unroll
  for (int m = G; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
template <int G>
__device__ __forceinline__ float across_groups_sum(float x) {
#pragma unroll
  for (int m = G; m < 64; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// A partition's block-table slice, staged on chip: entry j sits in lane j % 64
// of register j / 64, so one wave holds up to 64 * kTabRegs entries.
constexpr int kTabRegs = pa::kMaxPartitionBlocks / 64;
struct TableSlice {
  int r[kTabRegs];
  __device__ __forceinline__ void load(const int32_t* bt, int n, int lane) {
#pragma unroll
    for (int k = 0; k < kTabRegs; ++k) r[k] = (64 * k + lane < n) ? bt[64 * k + lane] : 0;
  }
  // entry j (wave-uniform j < 64 * kTabRegs), as a scalar: one readlane per
  // register and scalar selects (no dynamic register indexing)
  __device__ __forceinline__ int get(int j) const {
    const int lane = j & 63, k = j >> 6;
    int v = __builtin_amdgcn_readlane(r[0], lane);
#pragma unroll
    for (int i = 1; i < kTabRegs; ++i) {
      const int e = __builtin_amdgcn_readlane(r[i], lane);
      v = (k == i) ? e : v;
    }
    return v;
  }
};

// A forward-moving view of a TableSlice for callers that ask for entries in
// non-decreasing order: it keeps the register holding the 64 entries around
// the last one asked for, so an entry costs one readlane; moving on to the
// next register is a rare wave-uniform branch.
struct TableWindow {
  int w = 0;     // entries base .. base + 63
  int base = 0;  // a multiple of 64, wave-uniform
  __device__ __forceinline__ void init(const TableSlice& t) {
    w = t.r[0];
    base = 0;
  }
  // entry j (wave-uniform, base <= j < 64 * kTabRegs)
  __device__ __forceinline__ int get(const TableSlice& t, int j) {
    if (j - base >= 64) {
      const int k = j >> 6;
      int v = t.r[0];
#pragma unroll
      for (int i = 1; i < kTabRegs; ++i) {
        int c = t.r[i];
        asm("" : "+v"(c));  // a plain select per register, not an indexed (scratch) array access
        v = (k == i) ? c : v;
      }
      w = v;
      base = k << 6;
    }
    return __builtin_amdgcn_readlane(w, j - base);
  }
};

// Pool block sizes against the 16-token steps of the MFMA tiles:
//  * kBlocks16: blocks and steps coincide;
//  * kBlocksLarge: blocks of 16 << shift tokens; a step is a window of 16
//    rows inside one block (table entry step >> shift, rows 16 * (step & mask));
//  * kBlocksSmall: blocks of 16 >> shift tokens; a step's 16 rows come from
//    1 << shift blocks, so every lane addresses its own row's block.
constexpr int kBlocks16 = 0, kBlocksLarge = 1, kBlocksSmall = 2;

// kBlocksSmall: the partition's table (up to kMaxSmallBlockPartition
// entries) staged in LDS by the whole workgroup - every wave of a workgroup
// serves the same sequence and partition - then read per row by each lane.
// Callers reach this from every wave of the workgroup (it ends in a barrier).
__device__ __forceinline__ void stage_table(int32_t* stab, const int32_t* bt, int nent) {
  for (int k = threadIdx.x; k < nent; k += blockDim.x) stab[k] = bt[k];
  __syncthreads();
}
// Byte offset of the pool block holding each of N rows a lane touches in
// step jj; blk[i] = index of row i's block within the step (row / block
// size).  The step's blocks are table entries (jj << shift) + k, clamped to
// the partition's last entry (nent - 1) past its end, so every address stays
// inside a block the caller owns.
template <int N>
__device__ __forceinline__ void step_block_bases(const int32_t* stab, int jj, int shift, int nent,
                                                 size_t block_stride, const int* blk, size_t* base) {
  const int e0 = jj << shift;
#pragma unroll
  for (int i = 0; i < N; ++i) base[i] = (size_t)(uint32_t)stab[min(e0 + blk[i], nent - 1)] * block_stride;
}

// s_waitcnt vmcnt(N), the other counters left free (gfx9 field layout:
// vmcnt[3:0] and [15:14], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup id -> logical id such that each XCD (workgroups are dealt to the
// 8 XCDs round-robin) receives one contiguous range of logical ids; a bijection
// whatever the hardware order.
__device__ __forceinline__ int xcd_remap(int i, int n) {
  const int xcd = i & 7, k = i >> 3, per = n >> 3, rem = n & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

// ------------------------------------------------------------------ MFMA helpers

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

#ifndef PA_K_CPOL
#define PA_K_CPOL 2
#endif
#ifndef PA_V_CPOL
#define PA_V_CPOL 0
#endif
// Cache-policy bits of the K and V stream loads (gfx950: 1 = sc0, 2 = nt, 16 = sc1).
// Measured on MI355X: marking one of the two streams non-temporal is fastest
// (~10% over neither, ~4% over both), and keeps shared prompt blocks of
// forked sequences cacheable through the other stream.
constexpr int kKCpol = PA_K_CPOL, kVCpol = PA_V_CPOL;

// Raw buffer descriptor over `bytes` bytes from `base` (gfx9 data format word).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_block_rsrc(const uint8_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, (int)bytes, 0x00020000);
}
template <typename VT>
__device__ __forceinline__ VT buffer_load_v(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(VT) == 16)
    return __builtin_bit_cast(VT, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kVCpol));
  else
    return __builtin_bit_cast(VT, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kVCpol));
}

// XOR swizzle of a K row's 16-byte chunks in LDS for the matrix-core tiles,
// whose lane in MFMA column col reads token t = 4 (col % 4) + col / 4 at
// chunk 4c + gq: token t's chunk k sits at position k ^ kswz(t).  Rows of 16
// chunks: kswz(t) = col(t) = 4 (t % 4) + t / 4, so a lane reads chunk
// (4c + gq) ^ col - measured on gfx950 with four waves reading two blocks
// each, 71 clocks per wave and block pair, against 98 for k ^ t, which the
// 16-byte reads' lane grouping turns into two-way bank conflicts.  Rows of 8
// chunks: two rows share 16 positions, kswz(t) = t / 2.
template <int CPR>
__device__ __forceinline__ int kswz_t(int t) {
  return CPR == 16 ? ((t & 3) << 2) | (t >> 2) : (t >> 1) & (CPR - 1);
}

template <int DT>
struct MfmaOps;

template <>
struct MfmaOps<DT_BF16> {
  static __device__ __forceinline__ f32x4 qk(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // v_cvt_pk_bf16_f32, nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  // the sum of the two values a pack() word holds, as the matrix core reads them
  static __device__ __forceinline__ float sum_pair(uint32_t w) { return bf16_lo(w) + bf16_hi(w); }
};

template <>
struct MfmaOps<DT_F16> {
  static __device__ __forceinline__ f32x4 qk(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    return float_to_f16_bits(lo) | (float_to_f16_bits(hi) << 16);
  }
  static __device__ __forceinline__ float sum_pair(uint32_t w) {
    return f16_bits_to_float(w & 0xffffu) + f16_bits_to_float(w >> 16);
  }
};

// Max over the four 16-lane rows (lanes l, l^16, l^32, l^48), every lane ends equal.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}


template <int VPL>
struct VRow;  // V elements per lane and row
template <>
struct VRow<8> { using T = uint4; };
template <>
struct VRow<4> { using T = uint2; };

template <int VPL>
__device__ __forceinline__ uint32_t vword(const typename VRow<VPL>::T& v, int w) {
  if constexpr (VPL == 8) return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
  else return w == 0 ? v.x : v.y;
}

// ------------------------------------------------------------------ split-KV merge

// One wave merges np partition partials of one (query row, head):
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s with M = max_s m_s
// (m in log2 units), in a fixed order.  acc: np x D floats, ml: np (m, l).
template <int DT, int D>
__device__ __forceinline__ void merge_partials(uint8_t* out_row, const float* __restrict__ acc,
                                               const float2* __restrict__ ml, int np, int lane) {
  constexpr int EB = ElemBytes<DT>::value;
  constexpr int DPL = D / 64;  // dims per lane
  float M = -INFINITY;
  for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[p].x);
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) M = fmaxf(M, __shfl_xor(M, x));
  if (M == -INFINITY) M = 0.f;  // every partial empty: weights 2^-inf = 0, output 0
  float den = 0.f;
  for (int p = lane; p < np; p += 64) den += ml[p].y * fast_exp2(ml[p].x - M);
#pragma unroll
  for (int x = 1; x < 64; x <<= 1) den += __shfl_xor(den, x);

  // partials in chunks of 8 whose loads are all issued before any is used
  // (the loads, not the arithmetic, bound this loop); summed in partition order
  constexpr int kChunk = 8;
  float o[DPL] = {};
  for (int p0 = 0; p0 < np; p0 += kChunk) {
    float f[kChunk], v[kChunk][DPL];
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int p = min(p0 + i, np - 1);  // past np: a weight of 0 on a valid address
      f[i] = p0 + i < np ? ml[p].x : -INFINITY;
#pragma unroll
      for (int d = 0; d < DPL; ++d) v[i][d] = acc[(size_t)p * D + lane * DPL + d];
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const float w = fast_exp2(f[i] - M);
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[d] = fmaf(w, v[i][d], o[d]);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  uint8_t* dst = out_row + lane * DPL * EB;
#pragma unroll
  for (int d = 0; d < DPL; ++d) {
    const float v = o[d] * inv;
    if constexpr (DT == DT_F32) reinterpret_cast<float*>(dst)[d] = v;
    else if constexpr (DT == DT_BF16) reinterpret_cast<uint16_t*>(dst)[d] = (uint16_t)float_to_bf16_bits(v);
    else reinterpret_cast<uint16_t*>(dst)[d] = (uint16_t)float_to_f16_bits(v);
  }
}

}  // namespace
