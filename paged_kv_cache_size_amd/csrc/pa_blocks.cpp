// Host-side block pool and sequences of libpa (no HIP calls).
//
// The pool is a fixed set of physical blocks with a FIFO free queue and one
// reference count per block (handbook "分页 KV Cache", section "块表与 slot
// mapping": BlockPool hands out blocks from the head of its free queue,
// returns None when short, and re-queues freed blocks at the tail).  A
// sequence owns an ordered block list and a token count.  Forking shares every
// block (one more reference each); appending to a sequence whose partly filled
// last block is shared first moves that block to a fresh one - copy-on-write -
// and reports the (source, destination) pair so the caller can copy the rows
// on the device with pa_copy_blocks ("KV cache: capacity derivation, paging
// and reclamation", section on shared prefixes and reference counts).
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <new>
#include <vector>

#include "pa.h"

struct pa_block_pool {
  int32_t block_size = 0;
  std::vector<int32_t> ref;     // references per physical block
  std::deque<int32_t> free_q;   // blocks with no reference, in hand-out order
  struct Seq {
    std::vector<int32_t> blocks;
    int64_t length = 0;
    bool live = false;
  };
  std::vector<Seq> seqs;
  std::vector<int32_t> spare;   // released sequence handles, reused first
};

namespace {

bool valid_seq(const pa_block_pool* p, int32_t s) {
  return p && s >= 0 && s < (int32_t)p->seqs.size() && p->seqs[(size_t)s].live;
}

void drop(pa_block_pool* p, int32_t b) {
  if (--p->ref[(size_t)b] == 0) p->free_q.push_back(b);
}

int32_t take(pa_block_pool* p) {
  const int32_t b = p->free_q.front();
  p->free_q.pop_front();
  p->ref[(size_t)b] = 1;
  return b;
}

}  // namespace

extern "C" pa_block_pool* pa_block_pool_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pa_block_pool* p = new (std::nothrow) pa_block_pool;
  if (!p) return nullptr;
  try {
    p->block_size = block_size;
    p->ref.assign((size_t)num_blocks, 0);
    std::vector<char> seen((size_t)num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order ? free_order[i] : i;
      if (b < 0 || b >= num_blocks || seen[(size_t)b]) {  // not a permutation
        delete p;
        return nullptr;
      }
      seen[(size_t)b] = 1;
      p->free_q.push_back(b);
    }
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

extern "C" void pa_block_pool_destroy(pa_block_pool* pool) { delete pool; }

extern "C" int32_t pa_block_pool_num_free(const pa_block_pool* pool) {
  return pool ? (int32_t)pool->free_q.size() : -1;
}

extern "C" int32_t pa_block_pool_ref_count(const pa_block_pool* pool, int32_t block) {
  if (!pool || block < 0 || block >= (int32_t)pool->ref.size()) return -1;
  return pool->ref[(size_t)block];
}

extern "C" int pa_block_pool_allocate(pa_block_pool* pool, int32_t n, int32_t* blocks) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PA_ERR_INVALID_ARG;
  if ((size_t)n > pool->free_q.size()) return PA_ERR_NO_BLOCKS;
  for (int32_t i = 0; i < n; ++i) blocks[i] = take(pool);
  return PA_OK;
}

extern "C" int pa_block_pool_free(pa_block_pool* pool, const int32_t* blocks, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !blocks)) return PA_ERR_INVALID_ARG;
  try {  // all or nothing: no block may be listed more often than it is referenced
    std::vector<int32_t> ids(blocks, blocks + n);
    std::sort(ids.begin(), ids.end());
    for (size_t i = 0, j; i < ids.size(); i = j) {
      for (j = i; j < ids.size() && ids[j] == ids[i]; ++j) {
      }
      if (ids[i] < 0 || ids[i] >= (int32_t)pool->ref.size() || (int64_t)(j - i) > pool->ref[(size_t)ids[i]])
        return PA_ERR_INVALID_ARG;
    }
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) drop(pool, blocks[i]);
  return PA_OK;
}

extern "C" int pa_seq_create(pa_block_pool* pool, int32_t* seq) {
  if (!pool || !seq) return PA_ERR_INVALID_ARG;
  try {
    int32_t h;
    if (!pool->spare.empty()) {
      h = pool->spare.back();
      pool->spare.pop_back();
    } else {
      h = (int32_t)pool->seqs.size();
      pool->seqs.emplace_back();
    }
    pool->seqs[(size_t)h] = pa_block_pool::Seq{{}, 0, true};
    *seq = h;
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

extern "C" int pa_seq_fork(pa_block_pool* pool, int32_t parent, int32_t* child) {
  if (!valid_seq(pool, parent) || !child) return PA_ERR_INVALID_ARG;
  int32_t h;
  const int rc = pa_seq_create(pool, &h);
  if (rc != PA_OK) return rc;
  pa_block_pool::Seq& c = pool->seqs[(size_t)h];
  const pa_block_pool::Seq& p = pool->seqs[(size_t)parent];
  c.blocks = p.blocks;
  c.length = p.length;
  for (int32_t b : c.blocks) ++pool->ref[(size_t)b];
  *child = h;
  return PA_OK;
}

extern "C" int pa_seq_append(pa_block_pool* pool, int32_t seq, int64_t num_tokens, int32_t* cow_src,
                             int32_t* cow_dst) {
  if (!valid_seq(pool, seq) || num_tokens < 0 || !cow_src || !cow_dst) return PA_ERR_INVALID_ARG;
  pa_block_pool::Seq& s = pool->seqs[(size_t)seq];
  const int64_t bs = pool->block_size;
  *cow_src = -1;
  *cow_dst = -1;
  if (num_tokens == 0) return PA_OK;
  const int64_t have = (int64_t)s.blocks.size();
  const int64_t after = (s.length + num_tokens + bs - 1) / bs;
  if (after > (int64_t)1 << 30) return PA_ERR_INVALID_ARG;
  const bool cow = s.length % bs != 0 && pool->ref[(size_t)s.blocks.back()] > 1;
  const int64_t need = (after - have) + (cow ? 1 : 0);
  if (need > (int64_t)pool->free_q.size()) return PA_ERR_NO_BLOCKS;  // nothing changed
  try {
    s.blocks.reserve((size_t)after);
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  if (cow) {  // the shared, partly filled last block moves to a private copy
    const int32_t src = s.blocks.back();
    const int32_t dst = take(pool);
    drop(pool, src);
    s.blocks.back() = dst;
    *cow_src = src;
    *cow_dst = dst;
  }
  while ((int64_t)s.blocks.size() < after) s.blocks.push_back(take(pool));
  s.length += num_tokens;
  return PA_OK;
}

extern "C" int pa_seq_release(pa_block_pool* pool, int32_t seq) {
  if (!valid_seq(pool, seq)) return PA_ERR_INVALID_ARG;
  pa_block_pool::Seq& s = pool->seqs[(size_t)seq];
  for (int32_t b : s.blocks) drop(pool, b);
  s = pa_block_pool::Seq{};
  try {
    pool->spare.push_back(seq);
  } catch (...) {
  }
  return PA_OK;
}

extern "C" int64_t pa_seq_length(const pa_block_pool* pool, int32_t seq) {
  return valid_seq(pool, seq) ? pool->seqs[(size_t)seq].length : -1;
}

extern "C" int pa_seq_block_table(const pa_block_pool* pool, int32_t seq, int32_t* table, int32_t max_blocks,
                                  int32_t* num_blocks) {
  if (!valid_seq(pool, seq) || !num_blocks || max_blocks < 0 || (max_blocks > 0 && !table))
    return PA_ERR_INVALID_ARG;
  const pa_block_pool::Seq& s = pool->seqs[(size_t)seq];
  *num_blocks = (int32_t)s.blocks.size();
  if ((int32_t)s.blocks.size() > max_blocks) return PA_ERR_WORKSPACE;
  for (size_t i = 0; i < s.blocks.size(); ++i) table[i] = s.blocks[i];
  return PA_OK;
}

// Shared prefixes in a decode batch, from the block tables on the host: runs
// of consecutive sequences whose tables start with the same blocks (forks of
// one prompt).  A group's prefix is the whole blocks every member shares,
// ending before any member's last token (the block a new token is written to
// is private after copy-on-write).  A run shorter than two members, or
// sharing fewer than min_prefix_blocks blocks, is a group of one with no
// prefix.
extern "C" int pa_shared_prefix_groups(const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                                       int32_t max_blocks_per_seq, int32_t block_size, int32_t min_prefix_blocks,
                                       int32_t* group_start, int32_t* prefix_lens, int32_t* seq_prefix_lens,
                                       int32_t* num_groups, int32_t* max_group_size, int32_t* max_prefix_len) {
  if (!block_tables || !context_lens || !group_start || !prefix_lens || !seq_prefix_lens || !num_groups ||
      !max_group_size || !max_prefix_len || num_seqs <= 0 || max_blocks_per_seq <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  const int32_t need = min_prefix_blocks > 1 ? min_prefix_blocks : 1;
  auto cap = [&](int32_t b) -> int32_t {  // whole blocks before sequence b's last token
    const int32_t L = context_lens[b];
    const int32_t c = L > 0 ? (L - 1) / block_size : 0;
    return c < max_blocks_per_seq ? c : max_blocks_per_seq;
  };
  auto lcp = [&](int32_t a, int32_t b, int32_t limit) {
    const int32_t* ta = block_tables + (size_t)a * max_blocks_per_seq;
    const int32_t* tb = block_tables + (size_t)b * max_blocks_per_seq;
    int32_t k = 0;
    while (k < limit && ta[k] == tb[k]) ++k;
    return k;
  };
  int32_t g = 0, gmax = 0, pmax = 0;
  for (int32_t i = 0; i < num_seqs;) {
    int32_t common = cap(i), j = i + 1;
    while (j < num_seqs) {
      const int32_t c = lcp(i, j, std::min(common, cap(j)));
      if (c < need) break;
      common = c;
      ++j;
    }
    if (j - i < 2) common = 0;
    group_start[g] = i;
    prefix_lens[g] = common * block_size;
    for (int32_t b = i; b < j; ++b) seq_prefix_lens[b] = common * block_size;
    gmax = std::max(gmax, j - i);
    pmax = std::max(pmax, common * block_size);
    ++g;
    i = j;
  }
  group_start[g] = num_seqs;
  *num_groups = g;
  *max_group_size = gmax;
  *max_prefix_len = pmax;
  return PA_OK;
}
