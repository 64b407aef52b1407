"""Seeded synthetic decode workloads shaped like the pages' examples.

This module only builds inputs: sequence lengths, block tables (through a
small reference-counted block allocator) and N(0,1) tensors.  It holds none of
the arithmetic of the paged write or of attention, so both the HIP path and
the CPU oracle may be fed from it.

Five workloads are defined (sizes in the docstring of each builder):

* ``tiny_f32``         - 4 sequences of lengths 1/7/16/33, fp32, 4/2 heads, D 64
* ``qwen1p5b_bf16``    - 64 sequences, lognormal lengths (mean ~480), 12/2, D 128
* ``llama_gqa4k_bf16`` - 256 sequences x 4096 tokens, 32/8, D 128
* ``opt13b_mha_f16``   - 200 sequences, prompt U[100,2000] + output U[20,1500], 40/40
* ``shared_prefix_bf16`` - 64 prompts x 6 forked samples, 450 tokens, 32/8

Block tables are built by allocating blocks in a plain sequence of logical
ids and then relabelling every id through a seeded permutation of the whole
pool, so a table's physical ids are scattered and unrelated to each other.
"""

from __future__ import annotations

import math
import random
from collections import deque
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}

# --------------------------------------------------------------------------
# Block allocation (input construction only)
# --------------------------------------------------------------------------


class BlockPool:
    """The physical blocks of one pool, for building inputs.

    Blocks not in use wait in line, first in first out; a block in use
    carries the number of sequences holding it.  The behaviour is the
    handbook's pool ("分页 KV Cache", sections "实现" and "块表与 slot
    mapping"): a request for more blocks than are waiting gets None and
    changes nothing, blocks are handed out from the front of the line, and a
    block whose last holder lets go rejoins the line at the back.  A fork
    takes one more hold on every block it shares (``retain``).
    """

    def __init__(self, num_blocks: int, order=None):
        self.num_blocks = int(num_blocks)
        initial = range(self.num_blocks) if order is None else order
        self._waiting = deque(int(x) for x in initial)
        self._holds = {}  # block id -> sequences holding it (absent when free)

    def free_count(self) -> int:
        """Blocks waiting to be handed out."""
        return len(self._waiting)

    def holds(self, block) -> int:
        """Sequences holding ``block`` (0 when it is free)."""
        return self._holds.get(int(block), 0)

    def held(self) -> dict:
        """Every block in use and its hold count."""
        return dict(self._holds)

    def allocate(self, n: int):
        n = int(n)
        if n > len(self._waiting):
            return None
        out = []
        while len(out) < n:
            block = self._waiting.popleft()
            self._holds[block] = 1
            out.append(block)
        return out

    def retain(self, blocks) -> None:
        for block in blocks:
            self._holds[block] += 1

    def free(self, blocks) -> None:
        for block in blocks:
            remaining = self._holds.pop(block) - 1
            if remaining > 0:
                self._holds[block] = remaining
            else:
                self._waiting.append(block)


@dataclass
class SeqBlocks:
    """One sequence's block list and token count, grown token-run by run."""

    block_size: int
    blocks: list = field(default_factory=list)
    length: int = 0

    def fork(self, pool: BlockPool) -> "SeqBlocks":
        """A second sequence sharing every block (parallel sampling)."""
        pool.retain(self.blocks)
        return SeqBlocks(self.block_size, list(self.blocks), self.length)

    def append(self, n: int, pool: BlockPool, copies: list) -> None:
        """Append n tokens: open a new block when the last one is full, and
        copy a shared, partly filled last block before writing into it
        (copy-on-write).  Each copy is recorded as (src, dst, rows)."""
        while n > 0:
            used = self.length % self.block_size
            if used == 0:
                got = pool.allocate(1)
                if got is None:
                    raise MemoryError("block pool exhausted")
                self.blocks.append(got[0])
            elif pool.holds(self.blocks[-1]) > 1:
                got = pool.allocate(1)
                if got is None:
                    raise MemoryError("block pool exhausted")
                old = self.blocks[-1]
                copies.append((old, got[0], used))
                pool.free([old])
                self.blocks[-1] = got[0]
            take = min(n, self.block_size - used)
            self.length += take
            n -= take


# --------------------------------------------------------------------------
# Workload structure (integers only)
# --------------------------------------------------------------------------


@dataclass
class Workload:
    name: str
    dtype: str
    num_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray  # int32 [B], includes this step's token
    block_tables: np.ndarray  # int32 [B, max_blocks_per_seq]
    scale: float  # float32 value 1/sqrt(head_dim)
    pad_block: int  # an unowned block id filling unused table entries
    unowned_blocks: np.ndarray  # int64 ids no sequence references
    cow_copies: list  # (src, dst, rows) prefix copies made by copy-on-write
    description: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max())

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]

    def kv_read_bytes(self) -> int:
        """K and V bytes of every valid context token (each read once)."""
        return int(self.context_lens.astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * self.elem_bytes * 2

    def aux_bytes(self) -> dict:
        """Bytes a decode step moves besides the valid K/V rows: the query
        and output rows, the block-table entries in use, and the unused rows
        of each sequence's last block (a kernel that reads whole blocks
        fetches them)."""
        lens = self.context_lens.astype(np.int64)
        row = self.num_kv_heads * self.head_dim * self.elem_bytes * 2  # K + V row of one token
        used_blocks = (lens + self.block_size - 1) // self.block_size
        qo = self.num_seqs * self.num_heads * self.head_dim * self.elem_bytes
        return {"query": int(qo), "out": int(qo), "block_table_entries": int(used_blocks.sum()) * 4,
                "tail_slots": int((used_blocks * self.block_size - lens).sum()) * row}

    def kv_unique_read_bytes(self) -> int:
        """K and V bytes of the distinct pool rows the batch reads: a block
        shared by several sequences counts once, with the rows its longest
        user reads."""
        rows = {}
        for b in range(self.num_seqs):
            L = int(self.context_lens[b])
            for j in range((L + self.block_size - 1) // self.block_size):
                blk = int(self.block_tables[b, j])
                rows[blk] = max(rows.get(blk, 0), min(self.block_size, L - j * self.block_size))
        return sum(rows.values()) * self.num_kv_heads * self.head_dim * self.elem_bytes * 2


def _scale(head_dim: int) -> float:
    return float(np.float32(1.0 / math.sqrt(head_dim)))


def _finish(name, dtype, heads, kv_heads, head_dim, bs, seqs, used, num_blocks, perm_ids,
            lens, copies, extra_cols, description):
    """Relabel logical ids 0..used-1 to physical ids perm_ids[k]; pad tables."""
    perm_ids = np.asarray(perm_ids, dtype=np.int64)
    assert len(set(perm_ids[:used].tolist())) == used
    owned = set(int(x) for x in perm_ids[:used])
    unowned = np.array(sorted(set(range(num_blocks)) - owned), dtype=np.int64)
    assert unowned.size > 0, "pool needs at least one unowned block"
    pad = int(unowned[0])
    width = max(len(s.blocks) for s in seqs) + int(extra_cols)
    tables = np.full((len(seqs), width), pad, dtype=np.int32)
    for i, s in enumerate(seqs):
        tables[i, : len(s.blocks)] = perm_ids[np.asarray(s.blocks, dtype=np.int64)]
    cow = [(int(perm_ids[a]), int(perm_ids[b]), int(r)) for a, b, r in copies]
    return Workload(name, dtype, heads, kv_heads, head_dim, bs, int(num_blocks),
                    np.asarray(lens, dtype=np.int32), tables, _scale(head_dim), pad, unowned,
                    cow, description)


def _alloc_plain(lens, bs):
    """Allocate each sequence's full context in sequence order (logical ids)."""
    pool = BlockPool(sum(int(n) for n in lens) + 1)  # ample: a block holds >= 1 token
    seqs, copies = [], []
    for n in lens:
        s = SeqBlocks(bs)
        s.append(int(n), pool, copies)
        seqs.append(s)
    used = pool.num_blocks - pool.free_count()
    return seqs, used, copies


def tiny_f32(seed: int = 0, extra_cols: int = 0) -> Workload:
    """4 sequences with contexts 1, 7, 16, 33; block 16; 64-block pool whose
    free order is a seeded permutation; 4 query / 2 KV heads; D 64; fp32;
    scale 1/8.  New tokens land at positions 0, 6, 15 (last slot of a block)
    and 32 (first slot of a new block)."""
    lens = [1, 7, 16, 33]
    bs, nb = 16, 64
    perm = np.random.default_rng(seed).permutation(nb)
    seqs, used, copies = _alloc_plain(lens, bs)
    return _finish("tiny_f32", "f32", 4, 2, 64, bs, seqs, used, nb, perm, lens, copies,
                   extra_cols, "4 seqs L={1,7,16,33}, H 4 / Hkv 2, D 64, fp32, NB 64")


def lognormal_lengths(n: int, mean: float, sigma: float, lo: int, hi: int, seed: int):
    """Lengths ~ lognormal with the given mean, rounded and clipped."""
    mu = math.log(mean) - sigma * sigma / 2.0
    raw = np.random.default_rng(seed).lognormal(mu, sigma, n)
    return np.clip(np.rint(raw), lo, hi).astype(np.int64)


def qwen1p5b_bf16(seed: int = 0, extra_cols: int = 0) -> Workload:
    """Qwen2.5-1.5B-shaped layer: 64 sequences, lengths lognormal (sigma 0.8,
    mean 480) clipped to [16, 2048]; 12 query / 2 KV heads; D 128; bf16; pool =
    used blocks + 10%, physical ids shuffled."""
    lens = lognormal_lengths(64, 480.0, 0.8, 16, 2048, seed)
    bs = 16
    seqs, used, copies = _alloc_plain(lens, bs)
    nb = math.ceil(1.1 * used)
    perm = np.random.default_rng(seed + 1).permutation(nb)
    return _finish("qwen1p5b_bf16", "bf16", 12, 2, 128, bs, seqs, used, nb, perm, lens, copies,
                   extra_cols, "64 seqs lognormal(mean 480, sigma 0.8) in [16,2048], H 12 / Hkv 2, D 128, bf16")


def llama_gqa4k_bf16(seed: int = 0, extra_cols: int = 0, num_seqs: int = 256,
                     context: int = 4096, block_size: int = 16) -> Workload:
    """Llama-style GQA layer: 256 sequences of exactly 4096 tokens (256
    blocks each); 32 query / 8 KV heads; D 128; bf16; the 65536 used blocks
    are a random sample of a 72090-block pool, in random order.  Another
    block_size keeps the bytes and scales the block counts."""
    lens = [context] * num_seqs
    bs = int(block_size)
    seqs, used, copies = _alloc_plain(lens, bs)
    nb = max(math.ceil(1.1 * used), used + 1)
    perm = np.random.default_rng(seed).permutation(nb)
    name = "llama_gqa4k_bf16" if bs == 16 else f"llama_gqa4k_bf16_bs{bs}"
    return _finish(name, "bf16", 32, 8, 128, bs, seqs, used, nb, perm, lens, copies,
                   extra_cols, f"{num_seqs} seqs x {context} tokens, H 32 / Hkv 8, D 128, bf16, NB {nb}")


def opt13b_lengths(seed: int = 0):
    """Prompt U[100,2000] + output U[20,1500] for 200 requests, drawn with
    Python's random module exactly as the handbook's utilisation estimate."""
    rnd = random.Random(seed)
    reqs = [(rnd.randint(100, 2000), rnd.randint(20, 1500)) for _ in range(200)]
    return [p + o for p, o in reqs]


def opt13b_mha_f16(seed: int = 0, extra_cols: int = 0) -> Workload:
    """OPT-13B-shaped MHA layer: 200 sequences of prompt+output length from
    the handbook's seed-0 generator; 40 query / 40 KV heads; D 128; fp16; pool =
    used blocks + 10%, physical ids shuffled."""
    lens = opt13b_lengths(seed)
    bs = 16
    seqs, used, copies = _alloc_plain(lens, bs)
    nb = math.ceil(1.1 * used)
    perm = np.random.default_rng(seed + 1).permutation(nb)
    return _finish("opt13b_mha_f16", "f16", 40, 40, 128, bs, seqs, used, nb, perm, lens, copies,
                   extra_cols, "200 seqs prompt U[100,2000] + output U[20,1500], H 40 / Hkv 40, D 128, fp16")


def shared_prefix_bf16(seed: int = 0, extra_cols: int = 0, prompts: int = 64, samples: int = 6,
                       prompt_len: int = 300, gen_len: int = 150, name: str = "shared_prefix_bf16") -> Workload:
    """Parallel sampling: 64 prompts of 300 tokens, each forked into 6
    samples that generate 150 tokens; the prompt's blocks are shared by
    reference count and a sample copies the shared, partly filled last prompt
    block before its first write (copy-on-write).  One decode step at length
    450 over the 384 sequences (sample-major within each prompt); 32/8 heads,
    D 128, bf16; pool = used blocks + 10%, physical ids shuffled.

    Engine-like order: prefill every prompt, fork, then generate round-robin
    over all sequences; the decode step's token is the last generated one."""
    bs = 16
    total = prompt_len + gen_len
    pool = BlockPool(prompts * samples * total + 1)  # ample: a block holds >= 1 token
    copies = []
    roots = []
    for _ in range(prompts):
        s = SeqBlocks(bs)
        s.append(prompt_len, pool, copies)
        roots.append(s)
    seqs = []
    for r in roots:
        group = [r] + [r.fork(pool) for _ in range(samples - 1)]
        # the root becomes the last sample: the others copy before it writes
        seqs.extend(group[1:] + [group[0]])
    for _ in range(gen_len):
        for s in seqs:
            s.append(1, pool, copies)
    used = len(set(b for s in seqs for b in s.blocks))
    nb = math.ceil(1.1 * used)
    perm = np.random.default_rng(seed).permutation(nb)
    # make the referenced logical ids dense before relabelling
    live = sorted(set(b for s in seqs for b in s.blocks))
    relabel = {b: i for i, b in enumerate(live)}
    for s in seqs:
        s.blocks = [relabel[b] for b in s.blocks]
    copies = [(relabel[a], relabel[b], r) for a, b, r in copies if a in relabel and b in relabel]
    lens = [total] * len(seqs)
    return _finish(name, "bf16", 32, 8, 128, bs, seqs, len(live), nb, perm, lens,
                   copies, extra_cols,
                   f"{prompts} prompts x {samples} samples, {prompt_len}+{gen_len} tokens, H 32 / Hkv 8, D 128, bf16")


def custom(lens, num_heads: int, num_kv_heads: int, head_dim: int, dtype: str, seed: int = 0,
           extra_cols: int = 0, slack: float = 0.1, name: str = "custom", block_size: int = 16) -> Workload:
    """Any batch of context lengths with shuffled physical ids (edge cases)."""
    bs = int(block_size)
    seqs, used, copies = _alloc_plain(lens, bs)
    nb = max(math.ceil((1.0 + slack) * used), used + 1)
    perm = np.random.default_rng(seed).permutation(nb)
    return _finish(name, dtype, num_heads, num_kv_heads, head_dim, bs, seqs, used, nb, perm, lens, copies,
                   extra_cols, f"custom {len(lens)} seqs, H {num_heads} / Hkv {num_kv_heads}, D {head_dim}, {dtype}")


def shared_prefix_long_bf16(seed: int = 0, extra_cols: int = 0) -> Workload:
    """Parallel sampling with long prompts: 32 prompts of 3600 tokens, 8
    samples each, one decode step after 48 generated tokens (256 sequences at
    length 3648; 225 shared prompt blocks per group); otherwise as
    shared_prefix_bf16."""
    return shared_prefix_bf16(seed, extra_cols, prompts=32, samples=8, prompt_len=3600, gen_len=48,
                              name="shared_prefix_long_bf16")


BUILDERS = {
    "tiny_f32": tiny_f32,
    "qwen1p5b_bf16": qwen1p5b_bf16,
    "llama_gqa4k_bf16": llama_gqa4k_bf16,
    "opt13b_mha_f16": opt13b_mha_f16,
    "shared_prefix_bf16": shared_prefix_bf16,
    "shared_prefix_long_bf16": shared_prefix_long_bf16,
}


def make_workload(name: str, seed: int = 0, **kw) -> Workload:
    return BUILDERS[name](seed=seed, **kw)


# --------------------------------------------------------------------------
# Several new tokens per sequence (varlen prefill, chunked prefill)
# --------------------------------------------------------------------------

@dataclass
class PrefillBatch:
    """A batch whose sequence b brings query_lens[b] new tokens: the last
    query_lens[b] positions of its context of workload.context_lens[b] tokens
    (the context after this step, as in the decode workloads)."""
    workload: Workload
    query_lens: np.ndarray  # int32 [B], 1 <= n_b <= L_b
    description: str = ""

    @property
    def name(self) -> str:
        return self.workload.name

    @property
    def num_tokens(self) -> int:
        return int(self.query_lens.sum())

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max())

    @property
    def query_start_loc(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.query_lens.astype(np.int64))]).astype(np.int32)

    def attention_flops(self) -> int:
        """QK and PV multiply-adds of every visible (query row, key) pair,
        2 flops each: new token i of sequence b sees L_b - n_b + i + 1 keys."""
        w = self.workload
        pairs = 0
        for L, n in zip(w.context_lens.astype(np.int64), self.query_lens.astype(np.int64)):
            pairs += n * (L - n) + n * (n + 1) // 2
        return int(pairs) * w.num_heads * w.head_dim * 4

    def kv_read_bytes(self) -> int:
        return self.workload.kv_read_bytes()


def prefill_batch(lens, query_lens, num_heads: int, num_kv_heads: int, head_dim: int, dtype: str,
                  seed: int = 0, name: str = "prefill", extra_cols: int = 0, block_size: int = 16) -> PrefillBatch:
    q = np.asarray(query_lens, dtype=np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    assert q.shape == lens.shape and (q >= 1).all() and (q <= lens).all()
    w = custom(lens.tolist(), num_heads, num_kv_heads, head_dim, dtype, seed=seed, extra_cols=extra_cols,
               name=name, block_size=block_size)
    return PrefillBatch(w, q, f"{len(lens)} seqs, {int(q.sum())} new tokens, contexts {lens.min()}..{lens.max()}")


def chunked_prefill_llama_bf16(seed: int = 0, num_seqs: int = 16, context: int = 4096,
                               chunk: int = 512, block_size: int = 16) -> PrefillBatch:
    """Chunked prefill of the Llama-style GQA layer: 16 sequences each add a
    512-token chunk on top of 3584 cached tokens (context 4096); 32 query /
    8 KV heads; D 128; bf16; physical ids shuffled in a pool with 10% slack."""
    pb = prefill_batch([context] * num_seqs, [chunk] * num_seqs, 32, 8, 128, "bf16", seed=seed,
                       name="chunked_prefill_llama_bf16" + ("" if block_size == 16 else f"_bs{block_size}"),
                       block_size=block_size)
    pb.description = (f"{num_seqs} seqs x {chunk}-token chunks on {context - chunk} cached tokens, "
                      f"H 32 / Hkv 8, D 128, bf16")
    return pb


def mixed_varlen_bf16(seed: int = 0) -> PrefillBatch:
    """A mixed batch: whole prompts (n = L), chunks on cached context, and
    decode steps (n = 1), with ragged lengths over block boundaries; 12 query
    / 2 KV heads (group of 6), D 128, bf16."""
    rng = np.random.default_rng(seed)
    lens = [1, 16, 17, 33, 200, 500, 1000, 1500, 64, 300, 2049, 7]
    qls = [1, 16, 5, 33, 1, 129, 64, 1, 64, 300, 700, 7]
    order = rng.permutation(len(lens))
    pb = prefill_batch([lens[i] for i in order], [qls[i] for i in order], 12, 2, 128, "bf16", seed=seed,
                       name="mixed_varlen_bf16")
    pb.description = "12 seqs mixing whole prompts, chunks and decode steps, H 12 / Hkv 2, D 128, bf16"
    return pb


def handbook_verification_batch():
    """The handbook's paged-attention verification run ("分页 KV Cache",
    section "分页注意力"): three requests at different stages - one decode
    token on a 37-token context, a whole 5-token prompt, the last 8 tokens of a
    20-token chunked prefill - with 8 query / 2 KV heads, head_dim 64, fp32,
    block size 4, in a 32-block pool whose blocks are handed out one per
    request in turn, so the requests' blocks interleave.

    Returns (tables, seq_lens, query_lens, ks, vs, qs): ks[i] / vs[i] are the
    request's whole-context K/V [L_i, 2, 64] and qs[i] its new tokens' queries
    [n_i, 8, 64], float32 tensors on the CPU drawn from torch's CPU generator
    seeded with 0 in the page's order (all K, then all V, then all queries)."""
    import torch

    num_heads, num_kv_heads, head_dim, block_size = 8, 2, 64, 4
    seq_lens, query_lens = [37, 5, 20], [1, 5, 8]
    pool = BlockPool(32)
    tables = [[] for _ in seq_lens]
    while True:
        short = [i for i, L in enumerate(seq_lens) if len(tables[i]) * block_size < L]
        if not short:
            break
        for i in short:
            tables[i] += pool.allocate(1)
    gen = torch.Generator().manual_seed(0)
    ks = [torch.randn(L, num_kv_heads, head_dim, generator=gen) for L in seq_lens]
    vs = [torch.randn(L, num_kv_heads, head_dim, generator=gen) for L in seq_lens]
    qs = [torch.randn(n, num_heads, head_dim, generator=gen) for n in query_lens]
    return tables, seq_lens, query_lens, ks, vs, qs


def multi_token_llama_f32(seed: int = 0, num_seqs: int = 256, context: int = 4096, new_tokens: int = 4,
                          block_size: int = 16) -> PrefillBatch:
    """Several new tokens per sequence on the Llama-style GQA layer in fp32: 256
    sequences of 4096 tokens each add 4 tokens (a verification step of
    speculative decoding, or a short chunk); 32 query / 8 KV heads, D 128, fp32
    (8.6 GB of K/V); physical ids shuffled in a pool with 10% slack.  Each
    (sequence, KV head) has 4 x 4 = 16 (token, query head) columns."""
    pb = prefill_batch([context] * num_seqs, [new_tokens] * num_seqs, 32, 8, 128, "f32", seed=seed,
                       name="multi_token_llama_f32", block_size=block_size)
    pb.description = (f"{num_seqs} seqs x {new_tokens} new tokens on {context - new_tokens} cached tokens, "
                      f"H 32 / Hkv 8, D 128, fp32")
    return pb


PREFILL_BUILDERS = {
    "chunked_prefill_llama_bf16": chunked_prefill_llama_bf16,
    "mixed_varlen_bf16": mixed_varlen_bf16,
    "multi_token_llama_f32": multi_token_llama_f32,
}


# --------------------------------------------------------------------------
# Copy-on-write block copies
# --------------------------------------------------------------------------

@dataclass
class CopyBatch:
    """Whole-block copies inside a pool: dst[i] <- src[i] (distinct dst ids,
    none of them a src id)."""
    name: str
    dtype: str
    num_blocks: int
    block_size: int
    num_kv_heads: int
    head_dim: int
    src: np.ndarray  # int64 [P]
    dst: np.ndarray  # int64 [P]
    description: str = ""

    @property
    def block_bytes(self) -> int:
        return self.block_size * self.num_kv_heads * self.head_dim * ELEM_BYTES[self.dtype]

    def copy_bytes(self) -> int:
        """Bytes read plus bytes written, K and V pools."""
        return int(self.src.shape[0]) * self.block_bytes * 2 * 2


def copy_batch(num_blocks, block_size, num_kv_heads, head_dim, dtype, num_pairs, seed=0, name="copy"):
    ids = np.random.default_rng(seed).permutation(num_blocks)
    assert 2 * num_pairs <= num_blocks
    return CopyBatch(name, dtype, num_blocks, block_size, num_kv_heads, head_dim,
                     ids[:num_pairs].astype(np.int64), ids[num_pairs:2 * num_pairs].astype(np.int64),
                     f"{num_pairs} block copies in a {num_blocks}-block pool, H_kv {num_kv_heads}, D {head_dim}, "
                     f"{dtype}")


def cow_copy_llama_bf16(seed: int = 0, num_pairs: int = 8192) -> CopyBatch:
    """8192 copy-on-write block copies in the Llama-style layer's pool
    (72090 blocks of 16 tokens x 8 KV heads x 128 dims, bf16: 32 KiB per
    block and pool), sources and destinations random and disjoint."""
    cb = copy_batch(72090, 16, 8, 128, "bf16", num_pairs, seed=seed, name="cow_copy_llama_bf16")
    return cb


def swap_llama_bf16(seed: int = 0, num_pairs: int = 2048) -> CopyBatch:
    """Swap-out of 2048 random blocks of the Llama-style layer's pool (a
    preempted batch's 2048 x 16 tokens, 128 MiB of K and V) into a host pool
    of 2048 blocks, in order; the swap-in reverses the pairs."""
    ids = np.random.default_rng(seed).permutation(72090)[:num_pairs].astype(np.int64)
    return CopyBatch("swap_llama_bf16", "bf16", 72090, 16, 8, 128, ids, np.arange(num_pairs, dtype=np.int64),
                     f"{num_pairs} blocks of a 72090-block pool to a {num_pairs}-block pinned host pool and back, "
                     "H_kv 8, D 128, bf16")


COPY_BUILDERS = {"cow_copy_llama_bf16": cow_copy_llama_bf16}
SWAP_BUILDERS = {"swap_llama_bf16": swap_llama_bf16}


# --------------------------------------------------------------------------
# Tensors (torch, on any device)
# --------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def _randn(shape, dtype, gen, device, chunk=1 << 27):
    """N(0,1) drawn in float32 from ``gen`` and rounded to ``dtype``,
    generated in chunks so large pools need no float32 copy of the whole."""
    import torch
    td = torch_dtype(dtype)
    out = torch.empty(shape, dtype=td, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for start in range(0, n, chunk):
        stop = min(n, start + chunk)
        flat[start:stop] = torch.randn(stop - start, generator=gen, device=device,
                                       dtype=torch.float32).to(td)
    return out


def make_tensors(w: Workload, seed: int = 0, device="cpu"):
    """q [B,H,D], new key/value rows [B,H_kv,D] and the K/V pools
    [NB,BS,H_kv,D], all N(0,1) in the workload dtype from one seeded
    generator on ``device``.  Copy-on-write copies are replayed on the pools,
    so a copied block starts with the rows of the block it was copied from."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    b, h, hkv, d = w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim
    q = _randn((b, h, d), w.dtype, gen, device)
    key = _randn((b, hkv, d), w.dtype, gen, device)
    value = _randn((b, hkv, d), w.dtype, gen, device)
    pshape = (w.num_blocks, w.block_size, hkv, d)
    k_pool = _randn(pshape, w.dtype, gen, device)
    v_pool = _randn(pshape, w.dtype, gen, device)
    for src, dst, rows in w.cow_copies:
        k_pool[dst, :rows] = k_pool[src, :rows]
        v_pool[dst, :rows] = v_pool[src, :rows]
    return {"query": q, "key": key, "value": value, "k_pool": k_pool, "v_pool": v_pool}


def make_prefill_tensors(pb: PrefillBatch, seed: int = 0, device="cpu"):
    """q [T,H,D] and the new tokens' key/value rows [T,H_kv,D] (T = all new
    tokens, packed by sequence), the K/V pools [NB,BS,H_kv,D] and
    query_start_loc, all N(0,1) in the workload dtype from one seeded
    generator on ``device``."""
    import torch
    w = pb.workload
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    t, h, hkv, d = pb.num_tokens, w.num_heads, w.num_kv_heads, w.head_dim
    q = _randn((t, h, d), w.dtype, gen, device)
    key = _randn((t, hkv, d), w.dtype, gen, device)
    value = _randn((t, hkv, d), w.dtype, gen, device)
    pshape = (w.num_blocks, w.block_size, hkv, d)
    k_pool = _randn(pshape, w.dtype, gen, device)
    v_pool = _randn(pshape, w.dtype, gen, device)
    for src, dst, rows in w.cow_copies:
        k_pool[dst, :rows] = k_pool[src, :rows]
        v_pool[dst, :rows] = v_pool[src, :rows]
    qsl = torch.from_numpy(pb.query_start_loc).to(device)
    return {"query": q, "key": key, "value": value, "k_pool": k_pool, "v_pool": v_pool, "query_start_loc": qsl}


def raw_numpy(t):
    """A torch tensor's storage as numpy: float32/float16 as such, bfloat16 as
    uint16 bit patterns."""
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
