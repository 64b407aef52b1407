// Host-side argument checks and partition policy of libpa (no HIP calls).
#include "pa_host.h"

#include <algorithm>
#include <cmath>
#include <functional>
#include <vector>

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
  if (!decode_block_size_ok(s.block_size, s.dtype)) return PA_ERR_UNSUPPORTED;
  // grid: num_seqs * partitions * head groups workgroups must fit a 32-bit grid
  if ((int64_t)s.num_seqs * s.num_heads > (int64_t)1 << 30) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

bool decode_block_size_ok(int block_size, int dtype) {
  (void)dtype;  // every dtype's tiles take 16-token steps over any of these block sizes
  if (block_size <= 0 || (block_size & (block_size - 1)) != 0) return false;  // powers of two
  return block_size >= kMinDecodeBlock && block_size <= kMaxDecodeBlock;
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
  g.wpw = (kDecodeMaxWpw >= 8 && s.dtype != PA_F32 && g.units % 8 == 0) ? 8
          : g.units % 4 == 0                                                ? 4
          : g.units % 2 == 0                                                ? 2
                                                                            : 1;
  g.groups = g.units / g.wpw;
  return g;
}

namespace {

// Cost-model constants, in block steps (the time a workgroup takes for one
// 16-token block while every resident workgroup streams, i.e. at the HBM
// bound): a workgroup's fixed cost (table and query loads, ring fill, final
// stores), a partition past its sequence's end (exits at once), the merge
// launch, and how much faster a workgroup runs once so few remain that HBM is
// no longer saturated (its own loads in flight then bound it).  Fitted to
// launches on MI355X over partition sizes 128..4096 on uniform (256 x 4096
// tokens), ragged (200 sequences, 120..3400 tokens) and small (64 sequences)
// batches: the chosen size is within 2.5% of the best measured on each.
constexpr int kItemSetupQ = 16;  // quarter steps: every cost is a whole number of them
constexpr int kEmptyItemQ = 1;
constexpr double kItemSetup = kItemSetupQ / 4.0;
constexpr double kEmptyItem = kEmptyItemQ / 4.0;
constexpr double kMergeLaunch = 1.5;
constexpr double kMaxSpeedup = 2.0;

// Duration of the partition kernel in block steps.  Workgroups are dealt to
// the 8 XCDs round-robin and the kernel remaps them so that each XCD takes one
// contiguous range of (sequence, partition, head group) items, in order, as its
// slots free up.  All running workgroups share HBM equally: with `active` of
// the `slots` running each advances at min(kMaxSpeedup, slots / active) blocks
// per step.  Since they all advance at the same rate, the items finish in the
// order of (work done when they started + their work), a whole number of
// quarter steps: a bucket queue over that key replays the launch in
// O(items + makespan).
double simulate_partitions(const DecodeShape& s, const DecodeGrid& g, const int32_t* lens, int64_t pb,
                           int64_t parts, int64_t slots) {
  const int bs = kBlockSize;  // the kernels' step: 16 tokens, whatever the pool's block size
  const int64_t items = (int64_t)s.num_seqs * parts * g.groups;
  const int64_t xcd_slots = std::max<int64_t>(1, slots / 8);
  const int64_t per = items / 8, rem = items % 8;
  std::vector<int64_t> seq_blocks((size_t)s.num_seqs);
  for (int b = 0; b < s.num_seqs; ++b) {
    const int64_t len = lens ? std::max<int64_t>(0, lens[b]) : s.max_context_len;
    seq_blocks[(size_t)b] = (len + bs - 1) / bs;
  }
  // Per-XCD cursors over (sequence, partition, head group), advanced without
  // divisions.
  struct Cursor {
    int64_t left, b, part, grp;
  };
  Cursor cur[8];
  auto take = [&](Cursor& c) -> int64_t {  // quarter steps of the cursor's item; advance it
    const int64_t nblk = std::min<int64_t>(pb, seq_blocks[(size_t)c.b] - c.part * pb);
    --c.left;
    if (++c.grp == g.groups) {
      c.grp = 0;
      if (++c.part == parts) {
        c.part = 0;
        ++c.b;
      }
    }
    return nblk > 0 ? 4 * nblk + kItemSetupQ : kEmptyItemQ;
  };
  // One node per slot, reused by the slot's next item; head[key] lists the
  // nodes whose item ends when every running item has done `key` quarters.
  std::vector<int32_t> head, link, node_xcd;
  auto push = [&](int64_t key, int32_t node) {
    if (key >= (int64_t)head.size()) head.resize((size_t)std::max<int64_t>(key + 1, 2 * (int64_t)head.size()), -1);
    link[(size_t)node] = head[(size_t)key];
    head[(size_t)key] = node;
  };
  int64_t active = 0;
  for (int x = 0; x < 8; ++x) {
    const int64_t first = x * per + (x < rem ? x : rem);
    const int64_t seq_part = first / g.groups;
    cur[x] = {per + (x < rem ? 1 : 0), seq_part / parts, seq_part % parts, first % g.groups};
    for (int64_t k = 0; k < xcd_slots && cur[x].left > 0; ++k) {
      const int32_t node = (int32_t)node_xcd.size();
      node_xcd.push_back(x);
      link.push_back(-1);
      push(take(cur[x]), node);
      ++active;
    }
  }
  const double total = (double)(8 * xcd_slots);
  double t = 0.0;
  int64_t done = 0;
  for (int64_t key = 0; active > 0; ++key) {
    while (head[(size_t)key] >= 0) {
      const int32_t node = head[(size_t)key];
      head[(size_t)key] = link[(size_t)node];
      t += (double)(key - done) / 4.0 / std::min(kMaxSpeedup, total / (double)active);
      done = key;
      Cursor& c = cur[node_xcd[(size_t)node]];
      if (c.left > 0)
        push(key + take(c), node);  // at least one quarter later: never this bucket
      else
        --active;
    }
  }
  return t;
}

}  // namespace

namespace {

double merge_cost(const DecodeShape& s, const DecodeGrid& g, int64_t parts, int64_t slots) {
  if (parts <= 1) return 0.0;  // merge: read every partial once, write the output
  const double wg_block_bytes = (double)g.wpw * 2.0 * kBlockSize * s.head_dim * elem_bytes(s.dtype);
  return kMergeLaunch + 2.0 * (double)s.num_seqs * s.num_heads * parts * (s.head_dim + 2) * 4.0 /
                            ((double)slots * wg_block_bytes);
}

int64_t total_slots(int num_cus, int wg_per_cu) {
  return (int64_t)(num_cus > 0 ? num_cus : 256) * (wg_per_cu > 0 ? wg_per_cu : 1);
}

// A lower bound of decode_cost: the whole work spread evenly over the slots,
// and no less than the longest item.
double cost_lower_bound(const DecodeShape& s, const DecodeGrid& g, const int32_t* lens, int64_t pb,
                        int64_t parts, int64_t slots) {
  double work = 0.0;
  int64_t longest = 0;
  for (int b = 0; b < s.num_seqs; ++b) {
    const int64_t nblk = (std::max<int64_t>(0, lens[b]) + kBlockSize - 1) / kBlockSize;
    const int64_t used = std::min<int64_t>(parts, (nblk + pb - 1) / pb);
    work += (double)nblk + kItemSetup * used + kEmptyItem * (parts - used);
    longest = std::max(longest, std::min(nblk, pb));
  }
  const double spread = work * g.groups / slots;
  const double item = longest > 0 ? ((double)longest + kItemSetup) / kMaxSpeedup : 0.0;
  return std::max(spread, item) + merge_cost(s, g, parts, slots);
}

}  // namespace

double decode_cost(const DecodeShape& s, int64_t pb, const int32_t* lens, int num_cus, int wg_per_cu) {
  const DecodeGrid g = decode_grid(s);
  const int64_t slots = total_slots(num_cus, wg_per_cu);
  const int64_t nb = (s.max_context_len + kBlockSize - 1) / kBlockSize;
  const int64_t parts = (nb + pb - 1) / pb;
  double cost;
  if (lens) {
    cost = simulate_partitions(s, g, lens, pb, parts, slots);
  } else {  // every sequence at max_context_len: identical items in waves of `slots`
    const int64_t items = (int64_t)s.num_seqs * parts * g.groups;
    const double item = (double)pb + kItemSetup;
    const int64_t tail = items % slots;
    cost = (double)(items / slots) * item;
    if (tail > 0) cost += item / std::min(kMaxSpeedup, (double)slots / (double)tail);
  }
  return cost + merge_cost(s, g, parts, slots);
}

int partition_granule(int block_size) { return block_size > kBlockSize ? block_size : kBlockSize; }

int max_partition_tokens(int block_size) {
  return (block_size < kBlockSize ? kMaxSmallBlockPartition : kMaxPartitionBlocks) * block_size;
}

int max_prefill_partition_tokens(int block_size) { return max_partition_tokens(block_size); }

int block_shift(int block_size) {
  const int ratio = block_size >= kBlockSize ? block_size / kBlockSize : kBlockSize / block_size;
  int r = 0;
  while ((1 << r) < ratio) ++r;
  return r;
}

int validate_partition(int requested, int block_size) {
  const int gran = partition_granule(block_size);
  if (requested < gran || requested > max_partition_tokens(block_size) || requested % gran != 0)
    return -PA_ERR_INVALID_ARG;
  return requested;
}

int validate_prefill_partition(int requested, int block_size) {
  const int gran = partition_granule(block_size);
  if (requested < gran || requested > max_prefill_partition_tokens(block_size) || requested % gran != 0)
    return -PA_ERR_INVALID_ARG;
  return requested;
}

int partition_size(const DecodeShape& s, int requested, int num_cus, int wg_per_cu, const int32_t* lens) {
  if (requested != 0) return validate_partition(requested, s.block_size);
  // The model counts 16-token steps; a partition is a whole number of pool
  // blocks (spb steps each) and holds at most kMaxPartitionBlocks of them.
  // Without the lengths the batch is taken to be at max_context_len and the
  // partitions are kept short enough to balance a ragged one; with them the
  // launch is simulated and any size up to the table-slice limit may win.
  const int64_t spb = partition_granule(s.block_size) / kBlockSize;
  const int64_t max_steps = max_partition_tokens(s.block_size) / kBlockSize;
  int64_t cap = lens ? max_steps : std::min<int64_t>(kMaxAutoPartitionBlocks, max_steps);
  cap = std::max<int64_t>(spb, cap / spb * spb);
  const int64_t nb = (s.max_context_len + kBlockSize - 1) / kBlockSize;
  const int64_t bound = auto_partition_bound(s.max_context_len, s.block_size);
  struct Cand {
    int64_t pb;
    double lb;
  };
  std::vector<Cand> cands;
  const DecodeGrid g = decode_grid(s);
  const int64_t slots = total_slots(num_cus, wg_per_cu);
  for (int64_t parts = 1; parts <= bound; ++parts) {
    const int64_t pb = ((nb + parts - 1) / parts + spb - 1) / spb * spb;  // steps per partition
    if (pb > cap || (!cands.empty() && cands.back().pb == pb)) continue;
    const int64_t p = (nb + pb - 1) / pb;
    cands.push_back({pb, lens ? cost_lower_bound(s, g, lens, pb, p, slots) : 0.0});
  }
  if (cands.empty()) return (int)(std::min<int64_t>(cap, std::max<int64_t>(spb, nb)) * kBlockSize);
  // Simulate in order of the lower bound; stop once no bound can win.  Near
  // ties go to the longer partition (fewer partials to write and merge).
  std::stable_sort(cands.begin(), cands.end(), [](const Cand& x, const Cand& y) { return x.lb < y.lb; });
  int64_t best_pb = 0;
  double best = 0.0;
  for (const Cand& c : cands) {
    if (best_pb != 0 && c.lb >= best - 1e-9) break;
    const double cost = decode_cost(s, c.pb, lens, num_cus, wg_per_cu);
    if (best_pb == 0 || cost < best - 1e-9 || (cost < best + 1e-9 && c.pb > best_pb)) {
      best = cost;
      best_pb = c.pb;
    }
  }
  return (int)(best_pb * kBlockSize);
}

int check_partition_query(const DecodeShape& s) {
  static const int kFake = 0;
  return check_decode(&kFake, &kFake, &kFake, &kFake, &kFake, &kFake, s, 1.0f);
}

int auto_partition_bound(int max_context_len, int block_size) {
  const int least = block_size > kMinPartition ? block_size : kMinPartition;  // smallest automatic partition
  int b = (max_context_len + least - 1) / least;
  return b < 1 ? 1 : b;
}

int check_prefill(const void* out, const void* query, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start_loc,
                  const PrefillShape& s, float scale) {
  if (!query_start_loc) return PA_ERR_INVALID_ARG;
  const int rc = check_decode(out, query, k_pool, v_pool, block_tables, context_lens, s.d, scale);
  if (rc != PA_OK) return rc;
  if (s.num_tokens <= 0 || s.max_query_len <= 0 || s.max_query_len > s.num_tokens) return PA_ERR_INVALID_ARG;
  if (s.max_query_len > s.d.max_context_len) return PA_ERR_INVALID_ARG;
  if ((int64_t)s.num_tokens * s.d.num_heads > (int64_t)1 << 30) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int shared_prefix_slots(int max_context_len, int max_prefix_len) {
  const int p1 = num_partitions(max_prefix_len > 0 ? max_prefix_len : 1, kSharedPrefixPartition);
  const int p2 = num_partitions(max_context_len, kSharedPrefixPartition);
  return p1 + p2;
}

SharedPrefixGrid shared_prefix_grid(const DecodeShape& s, int num_groups, int max_group_size, int num_cus) {
  SharedPrefixGrid sg{0, 0, 0, 0};
  if (s.dtype == PA_F32 || s.block_size != kBlockSize || num_groups <= 0 || max_group_size <= 0) return sg;
  const DecodeGrid g = decode_grid(s);
  sg.members_per_set = kMaxRepPerWaveMfma / g.repc;
  sg.sets = (max_group_size + sg.members_per_set - 1) / sg.members_per_set;
  // steps of one set: at most members_per_set whole contexts; a wave holds
  // at most kMaxPartitionBlocks of them in its table slice
  const int64_t steps = (int64_t)sg.members_per_set * ((s.max_context_len + kBlockSize - 1) / kBlockSize);
  int waves = 1;
  while (waves <= 4 && (steps + waves - 1) / waves > kMaxPartitionBlocks) waves *= 2;
  if (waves > 4) return SharedPrefixGrid{0, 0, 0, 0};
  const int64_t units = (int64_t)num_groups * s.num_kv_heads * g.chunks * sg.sets;
  // more waves per set while the launch has at most four per SIMD's share
  // (two resident, two queued behind them: shorter waves finish the launch
  // more evenly; the 384-sequence parallel-sampling batch measured 63.6 us
  // with four waves per set against 65.3 us with two)
#ifndef PA_SHARED_PREFIX_WAVES_PER_CU
#define PA_SHARED_PREFIX_WAVES_PER_CU 16
#endif
  const int64_t target = (int64_t)(num_cus > 0 ? num_cus : 256) * PA_SHARED_PREFIX_WAVES_PER_CU;
  while (waves < 4 && units * waves * 2 <= target) waves *= 2;
  sg.waves = waves;
  sg.items = units;
  return sg;
}

int check_shared_prefix(const void* out, const void* query, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, const int32_t* group_start,
                        const int32_t* prefix_lens, const int32_t* seq_prefix_lens, const PrefillShape& s,
                        int num_groups, int max_group_size, int max_prefix_len, float scale) {
  if (!group_start || !prefix_lens || !seq_prefix_lens) return PA_ERR_INVALID_ARG;
  const int rc = check_decode(out, query, k_pool, v_pool, block_tables, context_lens, s.d, scale);
  if (rc != PA_OK) return rc;
  if (num_groups <= 0 || num_groups > s.d.num_seqs || max_group_size <= 0 || max_group_size > s.d.num_seqs)
    return PA_ERR_INVALID_ARG;
  if (max_prefix_len < 0 || max_prefix_len > s.d.max_context_len || max_prefix_len % s.d.block_size != 0)
    return PA_ERR_INVALID_ARG;
  if (s.d.dtype == PA_F32) return PA_ERR_UNSUPPORTED;  // both passes run the MFMA prefill tile
  // the passes split keys at kSharedPrefixPartition tokens, which must fit one table slice
  if (max_prefill_partition_tokens(s.d.block_size) < kSharedPrefixPartition) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

int prefill_tiles(const PrefillShape& s, const DecodeGrid& g) {
  return (int)(((int64_t)s.max_query_len * g.repc + 15) / 16);
}

PrefillGrid prefill_grid(const PrefillShape& s) {
  const DecodeGrid g = decode_grid(s.d);
  PrefillGrid p;
  const int64_t cols = (int64_t)s.max_query_len * g.repc;
  p.wide = cols >= kPrefillWideCols;
  p.wave_tiles = 1;
  if (p.wide) {
    if (cols <= 32) {
      p.waves = 2;
      p.wave_tiles = 1;
    } else if (cols <= 64) {
      p.waves = 2;
      p.wave_tiles = 2;
    } else {
      p.waves = kPrefillWgWaves;
      p.wave_tiles = kPrefillWaveTiles;
    }
    const int64_t wg_cols = 16 * p.wave_tiles * p.waves;
    p.tiles = (int)((cols + wg_cols - 1) / wg_cols);
    p.groups = g.units;
  } else {
    p.tiles = prefill_tiles(s, g);
    p.groups = g.groups;
    p.waves = g.wpw;
  }
  p.items = (int64_t)s.d.num_seqs * p.tiles * p.groups;
  return p;
}

int prefill_partition_bounds(const PrefillShape& s, int* min_parts, int* max_parts) {
  const int bs = s.d.block_size;
  const int64_t most = max_prefill_partition_tokens(bs);  // a multiple of the granule
  const int64_t lo = (s.d.max_context_len + most - 1) / most;
  int64_t hi = auto_partition_bound(s.d.max_context_len, bs);
  const size_t per_part = (size_t)s.num_tokens * s.d.num_heads * ((size_t)s.d.head_dim + 2) * sizeof(float);
  const int64_t cap = per_part > 0 ? (int64_t)(kPrefillWorkspaceCap / per_part) : hi;
  hi = std::min(hi, std::max<int64_t>(lo, cap));
  *min_parts = (int)std::max<int64_t>(1, lo);
  *max_parts = (int)std::max<int64_t>(*min_parts, hi);
  return PA_OK;
}

int cols_per_wave(int head_dim) {
  if (kColumnsMfma) return 16;
  return head_dim == 64 ? kMaxRepPerWaveValu : kMaxRepPerWaveValu / 2;
}

ColumnGrid column_grid(const PrefillShape& s) {
  const int64_t rep = s.d.num_heads / s.d.num_kv_heads;
  ColumnGrid g;
  g.cols = cols_per_wave(s.d.head_dim);
  const int64_t chunks = ((int64_t)s.max_query_len * rep + g.cols - 1) / g.cols;
  g.wpw = chunks >= 4 ? 4 : (chunks >= 2 ? 2 : 1);
  g.ctiles = (int)((chunks + g.wpw - 1) / g.wpw);
  g.items = (int64_t)s.d.num_seqs * s.d.num_kv_heads * g.ctiles;
  return g;
}

int prefill_partition_size(const PrefillShape& s, int requested, int num_cus, int wg_per_cu) {
  const PrefillGrid pg = prefill_grid(s);
  return prefill_partition_size_for(s, pg.items, pg.waves, requested, num_cus, wg_per_cu);
}

int prefill_partition_size_for(const PrefillShape& s, int64_t items_per_part, int waves, int requested,
                               int num_cus, int wg_per_cu) {
  const int bs = s.d.block_size;
  if (requested != 0) return validate_prefill_partition(requested, bs);
  // Partitions are whole granules (max(16, block size) tokens); costs count
  // 16-token steps.
  const int64_t gran = partition_granule(bs);
  const int64_t steps_per_gran = gran / kBlockSize;
  const int64_t slots = total_slots(num_cus, wg_per_cu);
  const int64_t ng = (s.d.max_context_len + gran - 1) / gran;
  int lo = 1, hi = 1;
  prefill_partition_bounds(s, &lo, &hi);
  int64_t best_pg = 0, prev_pg = 0;
  double best = 0.0;
  for (int64_t parts = lo; parts <= hi; ++parts) {
    const int64_t pgr = (ng + parts - 1) / parts;  // granules per partition
    if (pgr == prev_pg) continue;
    prev_pg = pgr;
    const int64_t p = (ng + pgr - 1) / pgr;
    if (p > hi || pgr * gran > max_prefill_partition_tokens(bs)) continue;
    const int64_t items = items_per_part * p;
    const double item = (double)(pgr * steps_per_gran) + kItemSetup;
    const int64_t tail = items % slots;
    double cost = (double)(items / slots) * item;
    if (tail > 0) cost += item / std::min(kMaxSpeedup, (double)slots / (double)tail);
    if (p > 1) {  // merge: every partial read once
      const double wg_step_bytes = (double)waves * 2.0 * kBlockSize * s.d.head_dim * elem_bytes(s.d.dtype);
      cost += kMergeLaunch + 2.0 * (double)s.num_tokens * s.d.num_heads * p * (s.d.head_dim + 2) * 4.0 /
                                 ((double)slots * wg_step_bytes);
    }
    if (best_pg == 0 || cost < best - 1e-9) {
      best = cost;
      best_pg = pgr;
    }
  }
  if (best_pg == 0) best_pg = std::min<int64_t>(max_prefill_partition_tokens(bs) / gran, ng);
  return (int)(best_pg * gran);
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
      partition_size > max_partition_tokens(kMaxDecodeBlock))
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

int pool_view(const void* k_pool, const void* v_pool, int layout, int block_size, int num_kv_heads, int head_dim,
              int dtype, PoolView* pv) {
  const int64_t e = elem_bytes(dtype);
  if (e == 0) return PA_ERR_UNSUPPORTED;
  if (!k_pool || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0) return PA_ERR_INVALID_ARG;
  const int64_t rowb = (int64_t)head_dim * e;
  const uint8_t* k = static_cast<const uint8_t*>(k_pool);
  if (layout == PA_KV_SPLIT) {
    if (!v_pool) return PA_ERR_INVALID_ARG;
    pv->k = k;
    pv->v = static_cast<const uint8_t*>(v_pool);
    pv->head_stride = rowb;
    pv->row_stride = (int64_t)num_kv_heads * rowb;
    pv->block_stride = (int64_t)block_size * pv->row_stride;
    return pv->block_stride <= kMaxBlockBytes ? PA_OK : PA_ERR_INVALID_ARG;
  }
  if (layout == PA_KV_FUSED) {
    if (v_pool) return PA_ERR_INVALID_ARG;  // the fused pool holds V itself
    pv->k = k;
    pv->v = k + rowb;
    pv->row_stride = 2 * rowb;
    pv->head_stride = (int64_t)block_size * pv->row_stride;
    pv->block_stride = (int64_t)num_kv_heads * pv->head_stride;
    return pv->block_stride <= kMaxBlockBytes ? PA_OK : PA_ERR_INVALID_ARG;
  }
  return PA_ERR_INVALID_ARG;
}

int check_convert_blocks(const void* dst_k, const void* dst_v, int dst_layout, int64_t dst_num_blocks,
                         const void* src_k, const void* src_v, int src_layout, int64_t src_num_blocks,
                         const int64_t* src, const int64_t* dst, int64_t num_pairs, int block_size,
                         int num_kv_heads, int head_dim, int dtype) {
  if (num_pairs < 0 || dst_num_blocks <= 0 || src_num_blocks <= 0) return PA_ERR_INVALID_ARG;
  if (num_pairs > 0 && (!src || !dst)) return PA_ERR_INVALID_ARG;
  if (num_pairs > 0x7fffffffLL) return PA_ERR_INVALID_ARG;  // one grid row per pair
  PoolView a, b;
  int rc = pool_view(dst_k, dst_v, dst_layout, block_size, num_kv_heads, head_dim, dtype, &a);
  if (rc != PA_OK) return rc;
  rc = pool_view(src_k, src_v, src_layout, block_size, num_kv_heads, head_dim, dtype, &b);
  if (rc != PA_OK) return rc;
  if ((int64_t)block_size * num_kv_heads * head_dim > (int64_t)1 << 30) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

int check_copy_blocks(const void* k_pool, const void* v_pool, const int64_t* src, const int64_t* dst,
                      int64_t num_pairs, int block_size, int num_kv_heads, int head_dim, int64_t num_blocks,
                      int dtype) {
  if (!k_pool || !v_pool || num_pairs < 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (num_pairs > 0 && (!src || !dst)) return PA_ERR_INVALID_ARG;
  if (num_pairs > 0x7fffffffLL) return PA_ERR_INVALID_ARG;  // one grid row per pair
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if ((int64_t)block_size * num_kv_heads * head_dim > (int64_t)1 << 30) return PA_ERR_INVALID_ARG;
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
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: not enough free blocks in the pool";
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
      pa::validate_partition(partition_size, block_size) <= 0)
    return 0;
  return pa::workspace_bytes(num_seqs, num_heads, head_dim,
                             pa::num_partitions(max_context_len, partition_size));
}

extern "C" int32_t pa_decode_plan_partition_size(int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, int32_t max_context_len, int32_t block_size,
                                                 pa_dtype dtype, const int32_t* host_context_lens,
                                                 int32_t num_cus, int32_t workgroups_per_cu) {
  const pa::DecodeShape shp{num_seqs, num_heads, num_kv_heads, head_dim, block_size, 1 << 30, max_context_len,
                            (int)dtype};
  const int rc = pa::check_partition_query(shp);
  if (rc != PA_OK) return -rc;
  if (num_cus <= 0 || workgroups_per_cu <= 0) return -PA_ERR_INVALID_ARG;
  return pa::partition_size(shp, 0, num_cus, workgroups_per_cu, host_context_lens);
}
