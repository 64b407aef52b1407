"""GPU parity on pools larger than 4 GiB, with sequences in blocks past it.

A pool's byte offsets pass 2^32 once a block id times the block's bytes does
(the handbook's pools are sized to fill what is left of HBM, so on a 288 GB
device any long-running server has such ids).  Each case builds a batch on a
small pool, copies that pool's blocks to scattered ids of a large one (most
past 4 GiB, a few below it, the pool's last block among them) and runs the
path on both: slots bit-exact against the oracle, the written rows
bit-exact, the attention outputs bitwise equal to the small pool's (block ids
do not enter the arithmetic) and within the tolerance of the float64 oracle.
Covered: the pool writer, decode (bf16 GQA, fp16 MHA, fp32), varlen prefill
(bf16, fp32), the shared-prefix decode, block copies, and conversion to the
fused layout with decode on it.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_size_amd import binding as PB
from paged_kv_cache_size_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
FOUR_GIB = 1 << 32


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


@pytest.fixture(autouse=True)
def _free_pools():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def block_bytes(w):
    return w.block_size * w.num_kv_heads * w.head_dim * w.elem_bytes


def large_ids(w, seed, spare=4096):
    """Ids in a pool just past 4 GiB for each of w's blocks: all but four at
    or past the first block that starts at 4 GiB, the pool's last block
    included.  Returns (ids, number of blocks of the large pool)."""
    first_high = -(-FOUR_GIB // block_bytes(w))
    nb_big = first_high + w.num_blocks + spare
    rng = np.random.default_rng(seed)
    n = w.num_blocks
    high = rng.choice(np.arange(first_high, nb_big - 1), size=n - 5, replace=False)
    low = rng.choice(np.arange(0, first_high), size=4, replace=False)
    ids = rng.permutation(np.concatenate([[nb_big - 1], high, low])).astype(np.int64)
    assert len(set(ids.tolist())) == n and (ids.astype(np.int64) * block_bytes(w) >= FOUR_GIB).sum() == n - 4
    return ids, nb_big


def to_large(w, t, seed):
    """The large pools holding w's blocks at ids[...], and w's tables relabeled."""
    ids, nb_big = large_ids(w, seed)
    shape = (nb_big,) + tuple(t["k_pool"].shape[1:])
    say(f"  large pool: {nb_big} blocks of {block_bytes(w)} B = {nb_big * block_bytes(w) / 2**30:.2f} GiB per pool")
    idx = torch.from_numpy(ids).to(DEV)
    big = {}
    for key in ("k_pool", "v_pool"):
        big[key] = torch.empty(shape, dtype=t["k_pool"].dtype, device=DEV)
        big[key][idx] = t[key]
    tables = ids[w.block_tables].astype(np.int32)
    return big, tables, idx


def decode_step(t, k_pool, v_pool, tables, w, partition_size):
    bt = torch.from_numpy(tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], k_pool, v_pool, slots)
    out = PB.pa_decode_attention(t["query"], k_pool, v_pool, bt, lens, w.scale, w.max_context_len,
                                 partition_size=partition_size)
    torch.cuda.synchronize()
    return slots, out


DECODE_CASES = [
    ("bf16", 32, 8, 128, [1, 17, 300, 1000, 2500, 4096, 33, 777]),
    ("f16", 40, 40, 128, [5, 250, 1890, 3500, 16, 1023]),
    ("f32", 8, 2, 64, [1, 7, 16, 33, 1500, 4100]),
]


@pytest.mark.parametrize("dtype,h,hkv,d,lens", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
@pytest.mark.parametrize("ps", [0, 512])
def test_decode_past_4gib(dtype, h, hkv, d, lens, ps):
    w = W.custom(lens, h, hkv, d, dtype, seed=5, name=f"large_{dtype}")
    say(f"decode past 4 GiB: {w.description}, ps={ps}")
    t = W.make_tensors(w, seed=5, device=DEV)
    big, tables, idx = to_large(w, t, seed=11)
    small = {k: v.clone() for k, v in t.items()}

    slots_big, out_big = decode_step(t, big["k_pool"], big["v_pool"], tables, w, ps)
    slots_small, out_small = decode_step(small, small["k_pool"], small["v_pool"], w.block_tables, w, ps)

    ref_slots = O.slot_mapping(tables, w.context_lens, w.block_size)
    assert np.array_equal(slots_big.cpu().numpy(), ref_slots)
    assert int(ref_slots.max()) * w.num_kv_heads * w.head_dim * w.elem_bytes >= FOUR_GIB
    # the oracle's pools: the seeded small pools with the oracle's own write
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    small_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    assert np.array_equal(slots_small.cpu().numpy(), small_slots)
    O.reshape_and_cache(kp, W.raw_numpy(t["key"]), small_slots)
    O.reshape_and_cache(vp, W.raw_numpy(t["value"]), small_slots)
    # the rows written past 4 GiB, and every other block moved there
    assert np.array_equal(W.raw_numpy(big["k_pool"][idx]).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(W.raw_numpy(big["v_pool"][idx]).view(np.uint8), vp.view(np.uint8))
    assert torch.equal(bits(out_big), bits(out_small))

    ref = O.decode_attention(W.raw_numpy(t["query"]), kp, vp, w.block_tables, w.context_lens, w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(out_big), w.dtype) - ref)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


PREFILL_CASES = [
    ("bf16", 32, 8, 128, [700, 2100, 1500, 100], [700, 37, 300, 1]),
    ("f32", 8, 2, 64, [300, 1200, 40], [300, 9, 4]),
]


@pytest.mark.parametrize("dtype,h,hkv,d,lens,qlens", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_past_4gib(dtype, h, hkv, d, lens, qlens):
    pb = W.prefill_batch(lens, qlens, h, hkv, d, dtype, seed=6, name=f"large_prefill_{dtype}")
    w = pb.workload
    say(f"prefill past 4 GiB: {pb.description}, {dtype}")
    t = W.make_prefill_tensors(pb, seed=6, device=DEV)
    big, tables, idx = to_large(w, t, seed=12)
    small = {k: v.clone() for k, v in t.items()}
    lens_d = torch.from_numpy(w.context_lens).to(DEV)
    outs = []
    for pools, tab in ((big, tables), (small, w.block_tables)):
        bt = torch.from_numpy(tab).to(DEV)
        slots = PB.pa_slot_mapping(bt, lens_d, w.block_size, query_start_loc=t["query_start_loc"],
                                   num_tokens=pb.num_tokens)
        PB.pa_reshape_and_cache(t["key"], t["value"], pools["k_pool"], pools["v_pool"], slots)
        outs.append(PB.pa_prefill_attention(t["query"], pools["k_pool"], pools["v_pool"], bt, lens_d,
                                            t["query_start_loc"], w.scale, pb.max_query_len, w.max_context_len))
    torch.cuda.synchronize()
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    small_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size, query_lens=pb.query_lens)
    O.reshape_and_cache(kp, W.raw_numpy(t["key"]), small_slots)
    O.reshape_and_cache(vp, W.raw_numpy(t["value"]), small_slots)
    assert np.array_equal(W.raw_numpy(big["k_pool"][idx]).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(W.raw_numpy(big["v_pool"][idx]).view(np.uint8), vp.view(np.uint8))
    assert torch.equal(bits(outs[0]), bits(outs[1]))

    ref = O.paged_attention(W.raw_numpy(t["query"]), kp, vp, w.block_tables, w.context_lens, pb.query_start_loc,
                            w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(outs[0]), w.dtype) - ref)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


def test_shared_prefix_past_4gib():
    w = W.shared_prefix_bf16(seed=7, prompts=6, samples=3, prompt_len=300, gen_len=40, name="large_shared")
    say(f"shared-prefix decode past 4 GiB: {w.num_seqs} seqs")
    t = W.make_tensors(w, seed=7, device=DEV)
    big, tables, _ = to_large(w, t, seed=13)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    outs = []
    for pools, tab in ((big, tables), (t, w.block_tables)):
        groups = PB.pa_shared_prefix_groups(tab, w.context_lens, w.block_size)
        assert groups.num_groups == 6
        bt = torch.from_numpy(tab).to(DEV)
        outs.append(PB.pa_decode_attention_shared_prefix(t["query"], pools["k_pool"], pools["v_pool"], bt, lens,
                                                         groups, w.scale, w.max_context_len))
    torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(outs[1]))
    ref = O.decode_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                             w.block_tables, w.context_lens, w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(outs[0]), w.dtype) - ref)))
    say(f"  max abs err {err:.3e} (tol 2e-2)")
    assert err <= TOL["bf16"]


def test_copy_and_fused_conversion_past_4gib():
    w = W.custom([4096, 2000, 333], 32, 8, 128, "bf16", seed=8, name="large_copy")
    t = W.make_tensors(w, seed=8, device=DEV)
    big, tables, idx = to_large(w, t, seed=14)
    nb_big = big["k_pool"].shape[0]
    first_high = -(-FOUR_GIB // block_bytes(w))
    rng = np.random.default_rng(15)
    used = set(int(x) for x in idx.cpu().numpy())
    free_high = np.array([i for i in range(first_high, nb_big) if i not in used], dtype=np.int64)
    src = rng.choice(idx.cpu().numpy(), size=64, replace=False)
    dst = rng.choice(free_high, size=64, replace=False)
    say(f"copy 64 blocks between ids past 4 GiB of a {nb_big}-block pool")
    PB.pa_copy_blocks(big["k_pool"], big["v_pool"], torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    s_d, d_d = torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV)
    for key in ("k_pool", "v_pool"):
        assert torch.equal(bits(big[key][d_d]), bits(big[key][s_d]))

    # the small split pool into a large fused pool at the same ids, then decode on it
    say("convert split -> fused past 4 GiB, decode on the fused pool")
    bs, hkv, d = w.block_size, w.num_kv_heads, w.head_dim
    del big
    torch.cuda.empty_cache()
    fused = torch.empty((nb_big, hkv, bs, 2 * d), dtype=t["k_pool"].dtype, device=DEV)
    small_ids = torch.arange(w.num_blocks, dtype=torch.int64, device=DEV)
    PB.pa_convert_blocks(fused, None, PB.PA_KV_FUSED, t["k_pool"], t["v_pool"], PB.PA_KV_SPLIT, small_ids, idx)
    bt_big = torch.from_numpy(tables).to(DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    got = PB.pa_decode_attention(t["query"], fused, None, bt_big, lens, w.scale, w.max_context_len,
                                 layout=PB.PA_KV_FUSED)
    want = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(want))
    fused_rows = W.raw_numpy(fused[idx])
    assert np.array_equal(fused_rows, O.fuse_kv(W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])))
