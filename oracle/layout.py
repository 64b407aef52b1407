"""The fused K|V pool layout, for the oracle (TEST INFRASTRUCTURE ONLY; see
the package docstring for who may import it).

HB, section "源码对照": vLLM's FlashAttention backend keeps one KV tensor per
layer of shape [num_blocks, num_kv_heads, block_size, 2 * head_size], K and V
joined on the last axis, while the handbook's own pools are a K and a V
tensor of shape [num_blocks, block_size, num_kv_heads, head_dim] each; the
same section notes that backends differ in layout, so moving KV between them
means converting it.  Both hold the same rows: element (block p, head h,
token t, j) of the fused pool is K[p, t, h, j] for j < D and V[p, t, h, j - D]
for j >= D.  Raw arrays throughout (bf16 as uint16 bit patterns), so every
function here is an exact rearrangement.
"""

import numpy as np


def fuse_kv(k_pool, v_pool):
    """Split pools [NB, BS, H_kv, D] -> one fused pool [NB, H_kv, BS, 2D]."""
    k_pool, v_pool = np.asarray(k_pool), np.asarray(v_pool)
    if k_pool.shape != v_pool.shape or k_pool.dtype != v_pool.dtype:
        raise ValueError("K and V pools differ")
    d = k_pool.shape[3]
    out = np.empty(k_pool.shape[:1] + (k_pool.shape[2], k_pool.shape[1], 2 * d), dtype=k_pool.dtype)
    out[..., :d] = k_pool.transpose(0, 2, 1, 3)  # [p, t, h, :] -> [p, h, t, :]
    out[..., d:] = v_pool.transpose(0, 2, 1, 3)
    return out


def split_kv(kv_pool):
    """One fused pool [NB, H_kv, BS, 2D] -> split pools [NB, BS, H_kv, D]."""
    kv_pool = np.asarray(kv_pool)
    if kv_pool.shape[3] % 2:
        raise ValueError("the last axis of a fused pool is 2 * head_dim")
    d = kv_pool.shape[3] // 2
    k = np.ascontiguousarray(kv_pool[..., :d].transpose(0, 2, 1, 3))
    v = np.ascontiguousarray(kv_pool[..., d:].transpose(0, 2, 1, 3))
    return k, v


def reshape_and_cache_fused(kv_pool, key, value, slots):
    """HB "实现" PagedKVCache.write, into the fused pool: token i's K and V
    rows of head h go to block slot // BS, head h, row slot % BS, first and
    second half.  Slots applied in index order."""
    block_size = kv_pool.shape[2]
    d = kv_pool.shape[3] // 2
    for i, s in enumerate(slots):
        s = int(s)
        p, t = s // block_size, s % block_size
        for h in range(kv_pool.shape[1]):
            kv_pool[p, h, t, :d] = key[i, h]
            kv_pool[p, h, t, d:] = value[i, h]


def convert_blocks(dst, src, src_blocks, dst_blocks, dst_fused, src_fused):
    """Block dst_blocks[i] of ``dst`` = block src_blocks[i] of ``src``; each
    is a fused pool (``*_fused``) or a (k_pool, v_pool) pair.  Pairs applied
    in order; ids outside either pool skip their pair."""
    def rows(pool, fused, p):  # logical [BS, H_kv, 2D] rows of block p
        if fused:
            return pool[p].transpose(1, 0, 2)
        return np.concatenate([pool[0][p], pool[1][p]], axis=-1)

    n_src = src.shape[0] if src_fused else src[0].shape[0]
    n_dst = dst.shape[0] if dst_fused else dst[0].shape[0]
    for s, d in zip(src_blocks, dst_blocks):
        s, d = int(s), int(d)
        if not (0 <= s < n_src and 0 <= d < n_dst):
            continue
        r = rows(src, src_fused, s).copy()
        half = r.shape[-1] // 2
        if dst_fused:
            dst[d] = r.transpose(1, 0, 2)
        else:
            dst[0][d] = r[..., :half]
            dst[1][d] = r[..., half:]
