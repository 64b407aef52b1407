"""Oracle: the paged KV write and paged attention as plain float64 definitions.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.

Storage conventions (raw, as the device holds them):
  * "f32"  -> numpy float32
  * "f16"  -> numpy float16
  * "bf16" -> numpy uint16 holding bfloat16 bit patterns

A KV pool is ``[num_blocks, block_size, num_kv_heads, head_dim]`` in one of
those storage types, one pool for K and one for V (HB, section "实现"
(implementation), the KV-storage bullet and the PagedKVCache class).

Paging changes where K/V live, not what attention computes (HB, section
"分页注意力" (paged attention): the kernel addresses K/V through the block
table yet the mathematics is that of contiguous attention).  So the attention
oracle below is the ordinary scaled-dot-product softmax attention evaluated on
the K/V rows gathered through each block table, in float64.
"""

import math

import numpy as np


def widen(x, dtype):
    """Decode raw storage to float64.

    bf16 is the upper half of an IEEE binary32: shifting the 16 stored bits
    left by 16 gives the float32 with the same value exactly.
    """
    x = np.asarray(x)
    if dtype == "bf16":
        assert x.dtype == np.uint16, x.dtype
        return (np.ascontiguousarray(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "f16":
        assert x.dtype == np.float16, x.dtype
        return x.astype(np.float64)
    if dtype == "f32":
        assert x.dtype == np.float32, x.dtype
        return x.astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# O1 / O2: addressing and block counts
# --------------------------------------------------------------------------

def slot_for(block_table, pos, block_size):
    """Physical slot of logical token position ``pos``.

    The token sits in logical block ``pos // block_size`` at offset
    ``pos % block_size``; the block table turns the logical block into a
    physical block, and the slot is physical_block * block_size + offset.
    HB, section "块表与 slot mapping" (block table and slot mapping); MV,
    section "block_table：逻辑位置到物理槽位的翻译" (translation formula).
    """
    pos = int(pos)
    block_size = int(block_size)
    return int(block_table[pos // block_size]) * block_size + pos % block_size


def slot_mapping(block_tables, seq_lens, block_size, query_lens=None):
    """Slots of every new token of one step, requests concatenated in order.

    Request ``i`` brings ``query_lens[i]`` new tokens (one each for decode),
    and they are the last tokens of its context of total length
    ``seq_lens[i]``, i.e. positions seq_len - n .. seq_len - 1 (HB, section
    "分页注意力": seq_lens is the context length after this step, and the
    paged_attention docstring places the new tokens at the end).
    """
    slots = []
    for i, (table, seq_len) in enumerate(zip(block_tables, seq_lens)):
        n = 1 if query_lens is None else int(query_lens[i])
        for pos in range(int(seq_len) - n, int(seq_len)):
            slots.append(slot_for(table, pos, block_size))
    return np.asarray(slots, dtype=np.int64)


def num_blocks(tokens, block_size):
    """Blocks a request of ``tokens`` tokens occupies: ceil(T / B).

    AQ, section "PagedAttention 核心" (NumBlocks formula); KC, section
    "分页怎样减少预留浪费" (the T=4100 example).
    """
    tokens = int(tokens)
    block_size = int(block_size)
    return (tokens + block_size - 1) // block_size


def tail_slots(tokens, block_size):
    """Unused slots in the last block: ceil(T/B)*B - T, at most B - 1.

    KC, section "分页怎样减少预留浪费"; AQ, section "PagedAttention 核心"
    (at most B-1 wasted positions).
    """
    return num_blocks(tokens, block_size) * int(block_size) - int(tokens)


# --------------------------------------------------------------------------
# O3 / O4: the pool write and the block-table gather
# --------------------------------------------------------------------------

def reshape_and_cache(pool, rows, slots):
    """Write row ``i`` of ``rows`` ([N, H_kv, D]) into slot ``slots[i]``.

    The pool ``[NB, BS, H_kv, D]`` is seen as a flat array of NB*BS slots, each
    holding one token's ``[H_kv, D]`` values, and each new token's row is
    copied, bit for bit, to its slot (HB, section "实现", PagedKVCache.write).
    Works in place on ``pool`` and returns it.  Rows are applied in index
    order; slots are expected to be distinct.
    """
    nb, bs, hkv, d = pool.shape
    assert rows.dtype == pool.dtype and rows.shape[1:] == (hkv, d)
    flat = pool.reshape(nb * bs, hkv, d)
    assert np.shares_memory(flat, pool)
    for i, s in enumerate(slots):
        flat[int(s)] = rows[i]
    return pool


def copy_blocks(pool, src_blocks, dst_blocks):
    """Copy-on-write at block granularity: block ``dst_blocks[i]`` of the pool
    becomes a bit copy of block ``src_blocks[i]``, for every i in order
    ("KV cache: capacity derivation, paging and reclamation", section on
    shared prefixes and reference counts: the fork that writes into a shared,
    partly filled block first gets its own copy).  Works in place on ``pool``
    ``[NB, BS, H_kv, D]`` and returns it.
    """
    assert len(src_blocks) == len(dst_blocks)
    for s, d in zip(src_blocks, dst_blocks):
        pool[int(d)] = pool[int(s)].copy()
    return pool


def swap_blocks(dst_pool, src_pool, src_blocks, dst_blocks):
    """Swap-out / swap-in of whole blocks between two pools of one block
    shape (handbook "分页 KV Cache", section on scheduling when memory runs
    short: a preempted sequence's blocks move to host memory and back):
    ``dst_pool[dst_blocks[i]] = src_pool[src_blocks[i]]`` bit for bit, in
    order.  Works in place on ``dst_pool`` and returns it."""
    assert dst_pool.shape[1:] == src_pool.shape[1:] and dst_pool.dtype == src_pool.dtype
    assert len(src_blocks) == len(dst_blocks)
    for s, d in zip(src_blocks, dst_blocks):
        dst_pool[int(d)] = src_pool[int(s)]
    return dst_pool


def gather(pool, block_table, seq_len):
    """The first ``seq_len`` tokens of one sequence, ``[seq_len, H_kv, D]``.

    Take the sequence's first ceil(seq_len / BS) physical blocks in logical
    order, lay their slots end to end and keep the first seq_len rows (HB,
    section "实现", PagedKVCache.gather).
    """
    bs = pool.shape[1]
    used = [int(b) for b in block_table[: num_blocks(seq_len, bs)]]
    blocks = [pool[b] for b in used]  # each [BS, H_kv, D]
    return np.concatenate(blocks, axis=0)[: int(seq_len)]


# --------------------------------------------------------------------------
# O5: paged attention (definition), O6: second formulation, brute force
# --------------------------------------------------------------------------

def paged_attention(q, k_pool, v_pool, block_tables, seq_lens, query_start_loc, scale, dtype):
    """Variable-length causal attention reading K/V through block tables.

    q: ``[N, H, D]`` raw storage; request ``i`` owns q rows
    ``query_start_loc[i] : query_start_loc[i+1]``, which are the last tokens
    of its context of length ``seq_lens[i]`` (HB, section "分页注意力", the
    inputs table and the paged_attention reference).

    For each request, each of its query tokens at position p and each query
    head h:
      * KV head g = h // (H / H_kv): every KV head serves a contiguous group
        of query heads (grouped-query attention, the KV heads repeated
        group-wise in HB's reference);
      * s_t = scale * <q_h, K_t,g> for the visible positions t <= p (causal);
      * o = sum_t exp(s_t - max s) V_t,g / sum_t exp(s_t - max s).
    The scale travels as a float32 through the C interface, so its float32
    value is used.  Everything is float64 from the raw inputs: the page's
    reference casts probabilities back to the input precision before the
    value product, an extra rounding the oracle does not make.
    Returns float64 ``[N, H, D]``.
    """
    qf = widen(q, dtype)
    n_tok, n_heads, head_dim = qf.shape
    n_kv = k_pool.shape[2]
    assert n_heads % n_kv == 0
    rep = n_heads // n_kv
    scale64 = float(np.float32(scale))
    out = np.zeros((n_tok, n_heads, head_dim), dtype=np.float64)
    for i, (table, seq_len) in enumerate(zip(block_tables, seq_lens)):
        start, end = int(query_start_loc[i]), int(query_start_loc[i + 1])
        n_new = end - start
        seq_len = int(seq_len)
        k = widen(gather(k_pool, table, seq_len), dtype)  # [L, H_kv, D]
        v = widen(gather(v_pool, table, seq_len), dtype)
        for j in range(n_new):
            visible = seq_len - n_new + j + 1  # positions 0 .. pos
            for h in range(n_heads):
                g = h // rep
                s = (k[:visible, g, :] @ qf[start + j, h, :]) * scale64
                w = np.exp(s - s.max())
                out[start + j, h, :] = (w @ v[:visible, g, :]) / w.sum()
    return out


def decode_attention(q, k_pool, v_pool, block_tables, context_lens, scale, dtype):
    """Decode step: one query token per sequence, the last of its context.

    The causal mask of a single final-position query keeps every position,
    so this is paged_attention with query_start_loc = 0, 1, ..., B.
    q: ``[B, H, D]`` raw.  Returns float64 ``[B, H, D]``.
    """
    qsl = list(range(len(context_lens) + 1))
    return paged_attention(q, k_pool, v_pool, block_tables, context_lens, qsl, scale, dtype)


def contiguous_attention(q, k, v, scale, dtype):
    """Second formulation, on unpaged per-sequence K/V ``[L, H_kv, D]``.

    Vectorised: KV heads are expanded to the query heads by repetition
    (each KV head repeated H/H_kv times in place, as HB's reference does),
    scores for all heads and query rows come from one contraction, the causal
    mask puts the n query rows at the last n positions, then a stable softmax
    and a second contraction.  q: ``[n, H, D]`` raw.  Returns float64
    ``[n, H, D]``.
    """
    qf, kf, vf = widen(q, dtype), widen(k, dtype), widen(v, dtype)
    n, n_heads, _ = qf.shape
    seq_len, n_kv, _ = kf.shape
    rep = n_heads // n_kv
    kr = np.repeat(kf, rep, axis=1)  # [L, H, D]
    vr = np.repeat(vf, rep, axis=1)
    scores = np.einsum("nhd,lhd->hnl", qf, kr) * float(np.float32(scale))
    rows = np.arange(n)[:, None] + (seq_len - n)
    cols = np.arange(seq_len)[None, :]
    scores = np.where(cols <= rows, scores, -np.inf)
    scores = scores - scores.max(axis=-1, keepdims=True)
    p = np.exp(scores)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("hnl,lhd->nhd", p, vr)


def brute_force_decode(q, k, v, scale, dtype):
    """Scalar-loop decode attention for tiny inputs, with exact sums.

    q: ``[H, D]`` raw, k/v: ``[L, H_kv, D]`` raw.  Every dot product and
    weighted sum goes through math.fsum (correctly rounded), each softmax
    weight through math.exp.  Returns float64 ``[H, D]``.
    """
    qf, kf, vf = widen(q, dtype), widen(k, dtype), widen(v, dtype)
    n_heads, head_dim = qf.shape
    seq_len, n_kv, _ = kf.shape
    rep = n_heads // n_kv
    scale64 = float(np.float32(scale))
    out = np.zeros((n_heads, head_dim))
    for h in range(n_heads):
        g = h // rep
        s = [scale64 * math.fsum(float(qf[h, d]) * float(kf[t, g, d]) for d in range(head_dim))
             for t in range(seq_len)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        total = math.fsum(w)
        for d in range(head_dim):
            out[h, d] = math.fsum(w[t] * float(vf[t, g, d]) for t in range(seq_len)) / total
    return out
