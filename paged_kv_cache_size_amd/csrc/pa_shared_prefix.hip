// Decode over groups of sequences that share their leading blocks, in one
// launch: forks of one prompt (parallel sampling) hold the prompt's blocks by
// reference count and only their own tails differ ("KV cache: capacity
// derivation, paging and reclamation", section on shared prefixes and
// reference counts; xxqk.cn PagedAttention article, block-level sharing and
// copy-on-write).  Attention over a member's context is attention over the
// shared blocks followed by its own blocks, so the shared blocks can be read
// once for every member.
//
// A workgroup takes one (group, KV head, set of members): the set's members
// and query heads fill the 16 columns of the matrix-core decode tile (16 /
// heads-per-KV-head members per set).  The set's key steps are the shared
// blocks - every column takes them - then each member's own blocks, which
// only that member's columns take (the others' probabilities are 0 there).
// The NW waves of the workgroup split that list of steps evenly, each with
// its own online softmax over its part, and merge their partial states
// through LDS at the end, so no partial leaves the workgroup and no second
// launch merges them.  Per step the operands are the decode tile's: QK on
// mfma_f32_16x16x32, P.V on mfma_f32_16x16x16, K through an LDS ring filled
// by direct-to-LDS loads, V in registers; the running max moves lazily (by
// more than 2^8 only, as in the prefill tiles) and masks are selects on the
// scores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pa.h"
#include "pa_device.h"
#include "pa_host.h"
#include "pa_runtime.h"

namespace {

struct GroupArgs {
  void* out;                    // [B, H, D]
  const void* query;            // [B, H, D]
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* block_tables;  // [B, max_blocks_per_seq]
  const int32_t* context_lens;  // [B]
  const int32_t* group_start;   // [groups + 1]: group g is sequences group_start[g] .. [g+1]-1
  const int32_t* prefix_lens;   // [groups]: shared tokens, whole blocks
  int num_heads, num_kv_heads, rep, repc, chunks, max_blocks_per_seq;
  int mpw;   // members per set: the 16 columns hold mpw members x repc query heads
  int sets;  // sets per group
  float qscale;  // scale * log2(e): scores in log2 units for exp2
  // pool geometry in bytes: K row (block p, token t, head h) at k_pool +
  // p*block_stride + t*row_stride + h*head_stride, V likewise; span = what
  // one 16-token block may touch from its first byte
  int64_t block_stride;
  uint32_t row_stride, head_stride, span;
};

constexpr int kAllMembers = 0xff;  // step tag of a shared block: every member's columns take it

template <int DT, int D, int NBUF, int NW>
__global__ __launch_bounds__(64 * NW) void shared_prefix_kernel(const GroupArgs a) {
  using Ops = MfmaOps<DT>;
  constexpr int BS = pa::kBlockSize;
  constexpr int ROWB = D * 2;
  constexpr int NKC = D / 32;         // QK k-chunks
  constexpr int VPL = D / 16;         // V elements per lane and row = P.V output tiles
  constexpr int DPL = 4 * VPL;        // output dims owned by a lane
  constexpr int CPR = ROWB / 16;      // 16-byte chunks per K row
  constexpr int NLI = BS * CPR / 64;  // K load instructions per block
  constexpr int KBYTES = BS * ROWB;   // one K block of one head
  using VT = typename VRow<VPL>::T;
  static_assert(NBUF >= 3 && NBUF <= 4, "ring depth; the merge reuses three slots");
  static_assert(32 * DPL * 4 == KBYTES, "half a wave's accumulators fill one ring slot");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int gq = lane >> 4, col = lane & 15;
  int rest = xcd_remap(blockIdx.x, gridDim.x);
  const int set = rest % a.sets;  // sets of one (group, KV head) run side by side: shared blocks meet in L2
  rest /= a.sets;
  const int chunk = rest % a.chunks;
  rest /= a.chunks;
  const int g = rest % a.num_kv_heads;
  const int grp = rest / a.num_kv_heads;

  // The group's members are dealt to as few sets as hold them, in equal
  // shares (6 members of at most 4 per set: 3 + 3), so that the sets' step
  // lists - the shared blocks plus their members' own - come out even.
  const int row0 = a.group_start[grp];
  const int members = a.group_start[grp + 1] - row0;
  const int used_sets = (members + a.mpw - 1) / a.mpw;
  const int share = used_sets > 0 ? (members + used_sets - 1) / used_sets : 0;
  const int m0 = set * share;  // the set's first member
  const int nm = min(share, members - m0);
  if (set >= used_sets || nm <= 0) return;  // workgroup-uniform: a smaller group than the largest
  const int P = a.prefix_lens[grp] / BS;  // shared blocks
  const int mi = col / a.repc;            // this lane's member within the set
  const bool live = mi < nm;              // nm <= mpw: the set's columns fit the 16
  const int row = row0 + m0 + (live ? mi : 0);
  const int head = g * a.rep + chunk * a.repc + col % a.repc;
  uint8_t* const out_row = (uint8_t*)a.out + ((size_t)row * a.num_heads + head) * ROWB + gq * DPL * 2;

  // Q^T as the QK B operand: column col = (member mi, head), k-chunk c =
  // dims 32c + 8gq .. +8 (loaded first: it needs only the group's rows).
  uint4 qop[NKC];
  {
    const uint8_t* qp = (const uint8_t*)a.query + ((size_t)row * a.num_heads + head) * ROWB + gq * 16;
#pragma unroll
    for (int c = 0; c < NKC; ++c) {
      const uint4 v = *reinterpret_cast<const uint4*>(qp + c * 64);
      qop[c] = live ? v : make_uint4(0, 0, 0, 0);
    }
  }

  // The set's steps: the P shared blocks, then each member's blocks past
  // them.  Member k's context length sits in lane k (one load for all).
  const int len_lane = lane < nm ? a.context_lens[row0 + m0 + lane] : 0;
  auto len_of = [&](int k) { return __builtin_amdgcn_readlane(len_lane, k); };
  auto own_steps = [&](int L) { return max(0, (L + BS - 1) / BS - P); };
  int total = P;
  for (int k = 0; k < nm; ++k) total += own_steps(len_of(k));
  const int per = (total + NW - 1) / NW;  // <= 64 * kTabRegs (the host picks NW so)
  const int j0 = min(total, wave * per);
  const int nsteps = min(total, j0 + per) - j0;  // this wave's share
  const int last = nsteps - 1;

  // This wave's steps staged in VGPR lanes (step e in lane e % 64 of
  // register e / 64): the physical block, and a tag (member << 8 | rows of
  // the block inside that member's context).
  TableSlice tab, tag;
#pragma unroll
  for (int k = 0; k < kTabRegs; ++k) {
    const int e = 64 * k + lane;
    int blk = 0, t = 0;
    if (e < nsteps) {
      // the step's table row and entry first (lengths only), then one load
      const int j = j0 + e;
      int trow = row0, bi = j;
      t = (kAllMembers << 8) | BS;
      if (j >= P) {
        int left = j - P;
        for (int kk = 0; kk < nm; ++kk) {
          const int L = len_of(kk);
          const int own = own_steps(L);
          if (left < own) {
            trow = row0 + m0 + kk;
            bi = P + left;
            t = (kk << 8) | min(BS, L - bi * BS);
            break;
          }
          left -= own;
        }
      }
      blk = a.block_tables[(size_t)trow * a.max_blocks_per_seq + bi];
    }
    tab.r[k] = blk;
    tag.r[k] = t;
  }


  // K: direct-to-LDS loads of whole rows, chunk q of token t at position
  // q ^ kswz(t) (the decode tile's layout); V: rows gq + 4i into registers.
  const uint32_t row_stride = a.row_stride;
  const uint32_t hoff = (uint32_t)g * a.head_stride;
  uint32_t kdma[NLI];
#pragma unroll
  for (int n = 0; n < NLI; ++n) {
    const int slot = 64 * n + lane, t = slot / CPR, q = slot % CPR;
    kdma[n] = (uint32_t)t * row_stride + hoff + (uint32_t)((q ^ kswz_t<CPR>(t)) * 16);
  }
  uint32_t kread[NKC];  // QK A operand: token 4*(col%4) + col/4, chunk 4c + gq
  {
    const int t = 4 * (col & 3) + (col >> 2);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kread[c] = (uint32_t)(t * CPR + ((4 * c + gq) ^ kswz_t<CPR>(t))) * 16;
  }
  const uint32_t voff = (uint32_t)gq * row_stride + hoff + col * VPL * 2;

  __shared__ __attribute__((aligned(1024))) uint8_t ks0[NW][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks1[NW][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks2[NW][KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t ks3[NBUF > 3 ? NW : 1][KBYTES];
  auto slot_base = [&](int x) -> uint8_t* {
    return x == 0 ? &ks0[wave][0] : x == 1 ? &ks1[wave][0] : x == 2 ? &ks2[wave][0] : &ks3[wave][0];
  };

  f32x4 acc[VPL];
#pragma unroll
  for (int t = 0; t < VPL; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max (log2 units; a finite floor until the first key), the
  // threshold that moves it, and the partial denominator of this lane's column
  constexpr float kFloor = -3.0e38f, kLazyLog2 = 8.f;
  float m = kFloor, mth = kFloor + kLazyLog2, l = 0.f;

  // Step j: K into ring slot `slot`, V into registers.  Past the wave's
  // last step the loads go through an empty descriptor (zeros, no memory
  // access), so every wait stays an exact count.
  // both read forward only: the loads' entries and the steps' tags come in order
  TableWindow twin, tagw;
  twin.init(tab);
  tagw.init(tag);
  auto load_block = [&](int j, int slot, VT* vr) {
    const bool real = j <= last;
    const int jj = real ? j : max(last, 0);
    const size_t off = (size_t)(uint32_t)twin.get(tab, jj) * (uint32_t)a.block_stride;  // stride <= 2^31 (host check)
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
  auto read_k = [&](int slot, uint4* kr) {
    const uint8_t* kb = slot_base(slot);
#pragma unroll
    for (int c = 0; c < NKC; ++c) kr[c] = *reinterpret_cast<const uint4*>(kb + kread[c]);
  };

  // One step tagged t: rows past its valid count never reach the sums (V
  // zeroed, weight 0), and columns of other members take weight 0.
  auto process = [&](const uint4* kr, const VT* vr, int t) {
    const int member = t >> 8, valid = t & 0xff;
    const bool act = live && (member == kAllMembers || member == mi);
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NKC; ++c) sacc = Ops::qk(kr[c], qop[c], sacc);
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] = act && 4 * i + gq < valid ? sacc[i] * a.qscale : -INFINITY;
    // rows past the block's valid count (stale, even NaN) must not reach the
    // MFMA: only a member's last block has any (a wave-uniform test)
    VT vm[4];
    if (valid < BS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) vm[i] = 4 * i + gq < valid ? vr[i] : VT{};
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) vm[i] = vr[i];
    }
    // The running max moves only when a score passes it by more than 2^8
    // (log2 units), so weights stay <= 256 and the rescale of the
    // accumulators is a rare wave-uniform branch; each lane tests its own
    // four scores, and the column max across the lane groups is taken only
    // inside the branch.  The max is finite from the start (a floor), so an
    // absent key's score of -inf gives weight exp2(-inf) = 0 with no select.
    const float smax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    if (__ballot(smax > mth)) {
      const float mn = fmaxf(m, rows_max(smax));
      const float alpha = fast_exp2(m - mn);  // 0 while m is the floor
      m = mn;
      mth = mn + kLazyLog2;
      l *= alpha;
#pragma unroll
      for (int tt = 0; tt < VPL; ++tt) acc[tt] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sc[i] - m);
    const uint2 pb = make_uint2(Ops::pack(p[0], p[1]), Ops::pack(p[2], p[3]));
    // the denominator sums the same dtype-rounded weights that P.V multiplies
    l += Ops::sum_pair(pb.x) + Ops::sum_pair(pb.y);
#pragma unroll
    for (int tt = 0; tt < VPL; ++tt) {
      const int w = tt >> 1;
      const uint32_t sel = (tt & 1) ? 0x07060302u : 0x05040100u;  // high or low 16-bit halves
      const uint2 va = make_uint2(__builtin_amdgcn_perm(vword<VPL>(vm[1], w), vword<VPL>(vm[0], w), sel),
                                  __builtin_amdgcn_perm(vword<VPL>(vm[3], w), vword<VPL>(vm[2], w), sel));
      acc[tt] = Ops::pv(va, pb, acc[tt]);
    }
  };

  VT vr[NBUF][4];
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) load_block(u, u, vr[u]);
  for (int j = 0; j < nsteps; j += NBUF) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int jj = j + u;
      uint4 kr[NKC];
      read_k(u, kr);
      load_block(jj + NBUF - 1, (u + NBUF - 1) % NBUF, vr[(u + NBUF - 1) % NBUF]);
      __builtin_amdgcn_sched_barrier(0);
      process(kr, vr[u], jj <= last ? tagw.get(tag, jj) : 0);
    }
  }
  float lt = rows_sum(l);
  wait_vmcnt<0>();  // the ring's last loads have landed: its slots are free for the merge

  if constexpr (NW > 1) {
    // Every wave leaves its state in its own ring slots (accumulators of
    // lanes 0-31 in slot 0, 32-63 in slot 1, register r of all eight tiles
    // together; (max, denominator) of each column in slot 2); then wave w
    // merges register r = w of every wave (dims 32 gq + 8w .. +8 of column
    // col) with the softmax rescaling and stores that quarter of the rows.
    static_assert(NW == 4 || NW == 2, "merge split");
    auto acc_at = [&](int v) {
      uint8_t* base = lane < 32 ? &ks0[v][0] : &ks1[v][0];
      return reinterpret_cast<float4*>(base + (lane & 31) * DPL * 4);
    };
    auto ml_at = [&](int v) { return reinterpret_cast<float2*>(&ks2[v][0]); };
    {
      float4* dst = acc_at(wave);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int tt = 0; tt < VPL; tt += 4)
          dst[(r * VPL + tt) / 4] = make_float4(acc[tt][r], acc[tt + 1][r], acc[tt + 2][r], acc[tt + 3][r]);
      if (gq == 0) ml_at(wave)[col] = make_float2(m, lt);
    }
    __syncthreads();
    if (!live) return;
    float mv[NW], fv[NW];
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float2 ml = ml_at(v)[col];
      mv[v] = ml.x;
      fv[v] = ml.y;
      M = fmaxf(M, ml.x);
    }
    float den = 0.f;
    constexpr int RPW = 4 / NW;  // accumulator registers each wave merges
    float o[RPW * VPL];
#pragma unroll
    for (int i = 0; i < RPW * VPL; ++i) o[i] = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float f = mv[v] == -INFINITY ? 0.f : fast_exp2(mv[v] - M);
      den = fmaf(f, fv[v], den);
      const float4* src = acc_at(v);
#pragma unroll
      for (int i = 0; i < RPW * VPL; i += 4) {
        const float4 x = src[(wave * RPW * VPL + i) / 4];
        o[i] = fmaf(f, x.x, o[i]);
        o[i + 1] = fmaf(f, x.y, o[i + 1]);
        o[i + 2] = fmaf(f, x.z, o[i + 2]);
        o[i + 3] = fmaf(f, x.w, o[i + 3]);
      }
    }
    const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
    for (int i = 0; i < RPW * VPL; ++i) o[i] *= inv;
    // this wave's NO consecutive dims of the lane's row segment in the query
    // dtype (nearest even): 8-byte or 16-byte stores
    constexpr int NO = RPW * VPL;
    static_assert(NO == 4 || NO % 8 == 0, "a wave stores 8 bytes or whole 16-byte chunks of each row");
    uint8_t* const dst = out_row + wave * NO * 2;
    if constexpr (NO == 4) {
      *reinterpret_cast<uint2*>(dst) = make_uint2(Ops::pack(o[0], o[1]), Ops::pack(o[2], o[3]));
    } else {
#pragma unroll
      for (int i = 0; i < NO; i += 8)
        *reinterpret_cast<uint4*>(dst + 2 * i) = make_uint4(Ops::pack(o[i], o[i + 1]), Ops::pack(o[i + 2], o[i + 3]),
                                                            Ops::pack(o[i + 4], o[i + 5]), Ops::pack(o[i + 6], o[i + 7]));
    }
  } else {
    if (!live) return;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float o[DPL];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int tt = 0; tt < VPL; ++tt) o[VPL * r + tt] = acc[tt][r] * inv;
    store_row<DT, DPL>(out_row, o);
  }
}

using GroupFn = void (*)(const GroupArgs);

constexpr int kGroupRing = 4;

template <int DT, int D>
GroupFn pick_group_nw(int nw) {
  switch (nw) {
    case 1: return shared_prefix_kernel<DT, D, kGroupRing, 1>;
    case 2: return shared_prefix_kernel<DT, D, kGroupRing, 2>;
    case 4: return shared_prefix_kernel<DT, D, kGroupRing, 4>;
    default: return nullptr;
  }
}

GroupFn pick_group(int dtype, int d, int nw) {
  switch (dtype) {
    case PA_F16: return d == 64 ? pick_group_nw<DT_F16, 64>(nw) : pick_group_nw<DT_F16, 128>(nw);
    case PA_BF16: return d == 64 ? pick_group_nw<DT_BF16, 64>(nw) : pick_group_nw<DT_BF16, 128>(nw);
    default: return nullptr;
  }
}

}  // namespace

namespace pa {

int launch_shared_prefix_single(void* out, const void* query, const PoolView& pv, const int32_t* block_tables,
                                const int32_t* context_lens, const int32_t* group_start, const int32_t* prefix_lens,
                                const DecodeShape& s, int num_groups, int max_group_size, float scale,
                                void* stream) {
  const SharedPrefixGrid sg = shared_prefix_grid(s, num_groups, max_group_size, device_cu_count());
  if (sg.waves == 0) return PA_ERR_UNSUPPORTED;
  GroupFn fn = pick_group(s.dtype, s.head_dim, sg.waves);
  if (!fn) return PA_ERR_UNSUPPORTED;
  const DecodeGrid dg = decode_grid(s);
  GroupArgs a;
  a.out = out;
  a.query = query;
  a.k_pool = pv.k;
  a.v_pool = pv.v;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.group_start = group_start;
  a.prefix_lens = prefix_lens;
  a.num_heads = s.num_heads;
  a.num_kv_heads = s.num_kv_heads;
  a.rep = dg.rep;
  a.repc = dg.repc;
  a.chunks = dg.chunks;
  a.max_blocks_per_seq = s.max_blocks_per_seq;
  a.mpw = sg.members_per_set;
  a.sets = sg.sets;
  a.qscale = scale * 1.44269504088896340736f;  // log2(e)
  a.block_stride = pv.block_stride;
  a.row_stride = (uint32_t)pv.row_stride;
  a.head_stride = (uint32_t)pv.head_stride;
  a.span = (uint32_t)pv.step_span(s.head_dim * elem_bytes(s.dtype), s.num_kv_heads);
  if (sg.items > 0x7fffffffLL) return PA_ERR_INVALID_ARG;
  return launch_kernel(fn, dim3((unsigned)sg.items), dim3(64 * sg.waves), static_cast<hipStream_t>(stream), a);
}

}  // namespace pa
