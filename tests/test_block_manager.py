"""The library's host block pool (pa_block_pool_*, pa_seq_*) and the oracle's
block copy, without a GPU.

The native pool is pinned to the allocator behaviour the pages print (FIFO
free queue, round-robin tables, fork and copy-on-write snapshots, the
parallel-sampling table) and checked operation by operation against the
input builder's independent Python pool on random traces.
"""

import json
from pathlib import Path

import numpy as np
import pytest

import oracle as O
from paged_kv_cache_size_amd import binding as B
from paged_kv_cache_size_amd.workloads import BlockPool, SeqBlocks

GOLDEN = Path(__file__).resolve().parent / "golden"


def load(name):
    return json.loads((GOLDEN / name).read_text())


def refs(m):
    return {str(i): m.ref_count(i) for i in range(m.num_blocks) if m.ref_count(i) > 0}


# ------------------------------------------------------------------ pins from the pages

def test_fifo_doctest_from_page():
    d = load("allocator_examples.json")["fifo_doctest"]
    m = B.BlockManager(d["num_blocks"], 16)
    table = m.allocate(d["first_allocate"])
    assert (table, m.num_free()) == (d["first_table"], d["free_after_first"])
    m.allocate(d["second_allocate"])
    m.free(table)
    assert m.allocate(d["third_allocate"]) == d["third_table"]
    assert m.allocate(100) is None


def test_round_robin_tables_from_page():
    d = load("allocator_examples.json")["round_robin_tables"]
    m = B.BlockManager(d["num_blocks"], d["block_size"])
    seqs = [m.new_seq() for _ in d["seq_lens"]]
    left = list(d["seq_lens"])
    while any(x > 0 for x in left):  # one block per request in turn
        for i, s in enumerate(seqs):
            if left[i] > 0:
                take = min(left[i], d["block_size"])
                assert m.append(s, take) is None
                left[i] -= take
    assert [m.block_table(s) for s in seqs] == d["tables"]


def test_fork_copy_on_write_snapshots():
    d = load("allocator_examples.json")["fork_cow_snapshots"]
    m = B.BlockManager(16, d["block_size"])
    a = m.new_seq()
    assert m.append(a, d["a_tokens"]) is None
    b = m.fork(a)
    s = d["after_fork"]
    assert (m.block_table(a), m.block_table(b), refs(m)) == (s["a"], s["b"], s["refs"])
    cow = m.append(b, 1)
    s = d["after_b_appends_one"]
    assert (m.block_table(a), m.block_table(b), refs(m)) == (s["a"], s["b"], s["refs"])
    assert cow == (1, 2)  # B copies A's half-full second block before writing
    m.release(a)
    assert refs(m) == d["after_release_a"]["refs"]
    m.release(b)
    assert len(refs(m)) == d["after_release_b"]["physical_blocks"]
    assert m.num_free() == 16


def test_parallel_sampling_block_table():
    d = load("allocator_examples.json")["parallel_sampling"]
    bs = d["block_size"]
    for row in d["rows"]:
        n = row["samples"]
        m = B.BlockManager(1000, bs)
        root = m.new_seq()
        m.append(root, d["prompt_len"])
        seqs = [m.fork(root) for _ in range(n - 1)] + [root]
        for _ in range(d["gen_len"]):
            for s in seqs:
                m.append(s, 1)
        shared = len({b for s in seqs for b in m.block_table(s)})
        assert (n * O.num_blocks(d["prompt_len"] + d["gen_len"], bs), shared) == (row["unshared_blocks"],
                                                                                  row["shared_blocks"])
        assert 1000 - m.num_free() == shared


# ------------------------------------------------------------------ all-or-nothing, errors

def test_exhaustion_changes_nothing():
    m = B.BlockManager(4, 4)
    a = m.new_seq()
    m.append(a, 6)  # 2 blocks
    b = m.fork(a)
    before = (m.block_table(a), m.block_table(b), refs(m), m.num_free(), m.length(b))
    with pytest.raises(B.PAError) as e:
        m.append(b, 11)  # needs a copy-on-write block and 3 more: 4 > 2 free
    assert e.value.status == B.PA_ERR_NO_BLOCKS
    assert (m.block_table(a), m.block_table(b), refs(m), m.num_free(), m.length(b)) == before
    assert m.append(b, 6) == (1, 2)  # 1 copy + 1 new block fits exactly
    assert m.num_free() == 0


def test_free_checks_before_changing_anything():
    m = B.BlockManager(4, 4)
    blocks = m.allocate(2)
    with pytest.raises(B.PAError):
        m.free([blocks[0], blocks[0]])  # listed twice, referenced once
    with pytest.raises(B.PAError):
        m.free([blocks[1], 7])
    assert [m.ref_count(b) for b in blocks] == [1, 1] and m.num_free() == 2
    m.free(blocks)
    assert m.num_free() == 4 and m.allocate(4) == [2, 3, 0, 1]  # freed blocks rejoin at the tail


def test_handles_and_arguments():
    m = B.BlockManager(8, 4, free_order=[7, 6, 5, 4, 3, 2, 1, 0])
    a = m.new_seq()
    m.append(a, 5)
    assert m.block_table(a) == [7, 6]
    m.release(a)
    with pytest.raises(B.PAError):
        m.release(a)  # released handles are invalid
    assert m.length(a) == -1
    assert m.new_seq() == a  # and reused
    with pytest.raises(B.PAError):
        B.BlockManager(0, 4)
    with pytest.raises(B.PAError):
        B.BlockManager(3, 4, free_order=[0, 0, 1])  # not a permutation
    lib = B.lib()
    assert lib.pa_block_pool_num_free(None) == -1
    assert lib.pa_seq_create(None, None) == B.PA_ERR_INVALID_ARG


# ------------------------------------------------------------------ against the Python pool

@pytest.mark.parametrize("seed", range(6))
def test_random_traces_match_the_python_pool(seed):
    rng = np.random.default_rng(seed)
    bs = int(rng.choice([1, 4, 16]))
    nb = 4000
    order = rng.permutation(nb)
    m = B.BlockManager(nb, bs, free_order=order)
    pool = BlockPool(nb, order=order)
    native, python = [], []  # parallel lists of live sequences
    for _ in range(400):
        op = rng.random()
        if op < 0.15 or not native:
            native.append(m.new_seq())
            python.append(SeqBlocks(bs))
        elif op < 0.3:
            i = int(rng.integers(len(native)))
            native.append(m.fork(native[i]))
            python.append(python[i].fork(pool))
        elif op < 0.42 and len(native) > 1:
            i = int(rng.integers(len(native)))
            m.release(native.pop(i))
            pool.free(python.pop(i).blocks)
        else:
            i = int(rng.integers(len(native)))
            n = int(rng.integers(0, 3 * bs + 2))
            copies = []
            cow = m.append(native[i], n)
            python[i].append(n, pool, copies)
            assert cow == (None if not copies else copies[0][:2])
        assert m.num_free() == pool.free_count()
    for s, p in zip(native, python):
        assert m.block_table(s) == p.blocks and m.length(s) == p.length
    assert all(m.ref_count(b) == pool.holds(b) for b in range(nb))


# ------------------------------------------------------------------ the oracle's block copy

def test_copy_on_write_keeps_both_views():
    # a fork writes into the shared half-full block: after copying that block
    # the parent still reads its own rows and the child reads the same prefix
    rng = np.random.default_rng(1)
    pool = BlockPool(16)
    copies = []
    parent = SeqBlocks(4)
    parent.append(6, pool, copies)
    child = parent.fork(pool)
    child.append(1, pool, copies)
    assert [c[:2] for c in copies] == [(1, 2)]
    kp = rng.standard_normal((16, 4, 2, 8)).astype(np.float32)
    snapshot = kp.copy()
    before = O.gather(kp, parent.blocks, 6).copy()
    O.copy_blocks(kp, [c[0] for c in copies], [c[1] for c in copies])
    np.testing.assert_array_equal(O.gather(kp, parent.blocks, 6), before)
    np.testing.assert_array_equal(O.gather(kp, child.blocks, 6), before)
    np.testing.assert_array_equal(kp[2], snapshot[1])  # the whole block, tail rows included
    others = [b for b in range(16) if b != 2]
    np.testing.assert_array_equal(kp[others], snapshot[others])


def test_swap_out_and_in_keeps_attention():
    # a preempted sequence's blocks go to a host pool and come back to other
    # device blocks: with the table renumbered, attention is unchanged, and
    # no other block of either pool moves
    rng = np.random.default_rng(2)
    dev_k = rng.standard_normal((12, 4, 2, 8)).astype(np.float32)
    dev_v = rng.standard_normal((12, 4, 2, 8)).astype(np.float32)
    host_k = np.zeros((5, 4, 2, 8), np.float32)
    host_v = np.zeros_like(host_k)
    table, L = [7, 2, 9], 11
    q = rng.standard_normal((1, 4, 8)).astype(np.float32)
    before = O.decode_attention(q, dev_k, dev_v, [table], [L], 0.35, "f32")
    snap_k, snap_v = dev_k.copy(), dev_v.copy()
    O.swap_blocks(host_k, dev_k, table, [4, 0, 3])
    O.swap_blocks(host_v, dev_v, table, [4, 0, 3])
    assert not host_k[[1, 2]].any()
    new_table = [5, 11, 0]
    O.swap_blocks(dev_k, host_k, [4, 0, 3], new_table)
    O.swap_blocks(dev_v, host_v, [4, 0, 3], new_table)
    after = O.decode_attention(q, dev_k, dev_v, [new_table], [L], 0.35, "f32")
    np.testing.assert_array_equal(before, after)
    others = [b for b in range(12) if b not in new_table]
    np.testing.assert_array_equal(dev_k[others], snap_k[others])
    np.testing.assert_array_equal(dev_v[others], snap_v[others])
