"""The oracle's fused K|V layout (oracle/layout.py) pinned without a GPU: a
hand-worked example of the shape statement, exact round trips, and the
direct write into the fused pool against the split write rearranged."""

import json
from pathlib import Path

import numpy as np
import pytest

import oracle as O

GOLDEN = Path(__file__).resolve().parent / "golden"


def rand_pools(rng, nb, bs, hkv, d):
    k = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d), dtype=np.uint16)
    return k, v


def test_hand_worked_example():
    g = json.loads((GOLDEN / "fused_layout.json").read_text())
    k, v = np.array(g["k"], np.int32), np.array(g["v"], np.int32)
    fused = O.fuse_kv(k, v)
    np.testing.assert_array_equal(fused, np.array(g["fused"], np.int32))
    # a head's rows of one block are contiguous, K row then V row per token
    np.testing.assert_array_equal(np.ascontiguousarray(fused).reshape(-1), g["fused_memory_order"])
    k2, v2 = O.split_kv(fused)
    np.testing.assert_array_equal(k2, k)
    np.testing.assert_array_equal(v2, v)


@pytest.mark.parametrize("shape", [(3, 16, 8, 128), (5, 1, 2, 64), (2, 32, 1, 64), (4, 4, 40, 128)])
def test_round_trip_is_exact(shape):
    rng = np.random.default_rng(sum(shape))
    k, v = rand_pools(rng, *shape)
    f = O.fuse_kv(k, v)
    assert f.shape == (shape[0], shape[2], shape[1], 2 * shape[3])
    k2, v2 = O.split_kv(f)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    # every element lands where the shape statement puts it
    p, t, h, j = (int(rng.integers(n)) for n in shape)
    assert f[p, h, t, j] == k[p, t, h, j] and f[p, h, t, shape[3] + j] == v[p, t, h, j]


@pytest.mark.parametrize("bs", [1, 4, 16])
def test_fused_write_matches_split_write(bs):
    rng = np.random.default_rng(bs)
    nb, hkv, d, n = 12, 4, 64, 20
    k, v = rand_pools(rng, nb, bs, hkv, d)
    fused = O.fuse_kv(k, v)
    key = rng.integers(0, 1 << 16, size=(n, hkv, d), dtype=np.uint16)
    val = rng.integers(0, 1 << 16, size=(n, hkv, d), dtype=np.uint16)
    slots = rng.choice(nb * bs, min(n, nb * bs), replace=False)
    key, val = key[:len(slots)], val[:len(slots)]
    O.reshape_and_cache(k, key, slots)
    O.reshape_and_cache(v, val, slots)
    O.reshape_and_cache_fused(fused, key, val, slots)
    np.testing.assert_array_equal(fused, O.fuse_kv(k, v))


def test_convert_blocks_moves_listed_blocks_only():
    rng = np.random.default_rng(7)
    nb, bs, hkv, d = 9, 16, 2, 64
    k, v = rand_pools(rng, nb, bs, hkv, d)
    dst = rng.integers(0, 1 << 16, size=(6, hkv, bs, 2 * d), dtype=np.uint16)
    before = dst.copy()
    src_ids, dst_ids = [4, 0, 8, 99], [1, 5, 2, 3]  # the last pair is out of range: skipped
    O.convert_blocks(dst, (k, v), src_ids, dst_ids, dst_fused=True, src_fused=False)
    ref = O.fuse_kv(k, v)
    for s, t in zip(src_ids[:3], dst_ids[:3]):
        np.testing.assert_array_equal(dst[t], ref[s])
    for t in (0, 3, 4):
        np.testing.assert_array_equal(dst[t], before[t])
    # and back into a split pair
    k2, v2 = np.zeros_like(k), np.zeros_like(v)
    O.convert_blocks((k2, v2), dst, [1, 5, 2], [4, 0, 8], dst_fused=False, src_fused=True)
    for p in (4, 0, 8):
        np.testing.assert_array_equal(k2[p], k[p])
        np.testing.assert_array_equal(v2[p], v[p])
    assert not k2[[1, 2, 3, 5, 6, 7]].any()


def test_attention_is_layout_free():
    # the same rows give the same decode result whichever layout held them
    rng = np.random.default_rng(3)
    nb, bs, hkv, d = 6, 4, 2, 64
    k = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    v = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    k2, v2 = O.split_kv(O.fuse_kv(k, v))
    q = rng.standard_normal((1, 4, d)).astype(np.float32)
    a = O.decode_attention(q, k, v, [[3, 0, 5]], [10], 0.125, "f32")
    b = O.decode_attention(q, k2, v2, [[3, 0, 5]], [10], 0.125, "f32")
    np.testing.assert_array_equal(a, b)
