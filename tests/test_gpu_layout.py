"""GPU parity of the fused K|V pool layout [NB, H_kv, BS, 2D].

Fused pools given to the kernels are built on the host by the oracle
(``O.fuse_kv`` of the seeded split pools), except where the device
conversion itself is under test.  Checks:

  * pa_convert_blocks (split <-> fused, fused -> fused, to and from pinned
    host memory): bit-exact against ``O.convert_blocks`` over whole pools;
  * the pool write into a fused pool: bit-exact against
    ``O.reshape_and_cache_fused``;
  * decode and prefill attention on a fused pool: bitwise equal to the same
    call on the split pools (the kernels read the same rows in the same
    order), and within 1e-5 (fp32) / 2e-2 (bf16, fp16) of the float64 oracle.
"""

import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_size_amd import binding as PB
from paged_kv_cache_size_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
DEV = "cuda"
FUSED, SPLIT = PB.PA_KV_FUSED, PB.PA_KV_SPLIT


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def to_torch(raw, dtype, device=DEV):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(device)


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def ids(x):
    return torch.tensor(list(x), dtype=torch.int64, device=DEV)


# ------------------------------------------------------------------ conversion

@pytest.mark.parametrize("dtype,bs,hkv,d", [("bf16", 16, 8, 128), ("f32", 4, 2, 64), ("f16", 64, 3, 64),
                                            ("bf16", 1, 4, 128)])
def test_convert_round_trip(dtype, bs, hkv, d):
    say(f"convert {dtype} bs={bs} hkv={hkv} d={d}")
    rng = np.random.default_rng(bs * 7 + hkv)
    nb = 37
    gen = torch.Generator(device=DEV).manual_seed(5)
    kp = W._randn((nb, bs, hkv, d), dtype, gen, DEV)
    vp = W._randn((nb, bs, hkv, d), dtype, gen, DEV)
    k_raw, v_raw = W.raw_numpy(kp), W.raw_numpy(vp)

    # every block, identity ids
    fused = torch.full((nb, hkv, bs, 2 * d), float("nan"), dtype=kp.dtype, device=DEV)
    PB.pa_convert_blocks(fused, None, FUSED, kp, vp, SPLIT, ids(range(nb)), ids(range(nb)))
    torch.cuda.synchronize()
    assert np.array_equal(W.raw_numpy(fused), O.fuse_kv(k_raw, v_raw))

    # a subset into other places, one pair out of range (skipped)
    src = rng.choice(nb, 9, replace=False).tolist() + [nb + 3]
    dst = rng.choice(nb, 10, replace=False).tolist()
    k2 = W._randn((nb, bs, hkv, d), dtype, gen, DEV)
    v2 = W._randn((nb, bs, hkv, d), dtype, gen, DEV)
    ref = (W.raw_numpy(k2), W.raw_numpy(v2))
    PB.pa_convert_blocks(k2, v2, SPLIT, fused, None, FUSED, ids(src), ids(dst))
    torch.cuda.synchronize()
    O.convert_blocks(ref, O.fuse_kv(k_raw, v_raw), src, dst, dst_fused=False, src_fused=True)
    assert np.array_equal(W.raw_numpy(k2), ref[0]) and np.array_equal(W.raw_numpy(v2), ref[1])

    # same layout: copy-on-write inside one fused pool
    f_ref = W.raw_numpy(fused)
    PB.pa_convert_blocks(fused, None, FUSED, fused, None, FUSED, ids([3, 4]), ids([20, 21]))
    torch.cuda.synchronize()
    O.convert_blocks(f_ref, f_ref.copy(), [3, 4], [20, 21], dst_fused=True, src_fused=True)
    assert np.array_equal(W.raw_numpy(fused), f_ref)


def test_convert_to_and_from_pinned_host():
    # a fused pool swapped out to pinned host memory and back into other blocks
    say("convert fused <-> pinned host fused")
    nb, bs, hkv, d = 64, 16, 8, 128
    gen = torch.Generator(device=DEV).manual_seed(9)
    kp = W._randn((nb, bs, hkv, d), "bf16", gen, DEV)
    vp = W._randn((nb, bs, hkv, d), "bf16", gen, DEV)
    fused = to_torch(O.fuse_kv(W.raw_numpy(kp), W.raw_numpy(vp)), "bf16")
    host = torch.zeros((8, hkv, bs, 2 * d), dtype=torch.bfloat16, pin_memory=True)
    out_ids, host_ids = [5, 17, 40], [7, 0, 3]
    PB.pa_convert_blocks(host, None, FUSED, fused, None, FUSED, ids(out_ids), ids(host_ids))
    torch.cuda.synchronize()
    for s, h in zip(out_ids, host_ids):
        assert torch.equal(bits(host[h]), bits(fused[s].cpu()))
    # back in, into a split pool pair (a layout change on the way)
    k2, v2 = torch.zeros_like(kp), torch.zeros_like(vp)
    PB.pa_convert_blocks(k2, v2, SPLIT, host, None, FUSED, ids(host_ids), ids([1, 2, 3]))
    torch.cuda.synchronize()
    for s, t in zip(out_ids, [1, 2, 3]):
        assert torch.equal(bits(k2[t]), bits(kp[s])) and torch.equal(bits(v2[t]), bits(vp[s]))


# ------------------------------------------------------------------ pool write

@pytest.mark.parametrize("dtype,bs", [("bf16", 16), ("f32", 16), ("f16", 1), ("bf16", 32)])
def test_fused_write(dtype, bs):
    w = W.custom([1, 5, 16, 17, 40, 100], 8, 2, 64, dtype, seed=bs, block_size=bs)
    say(f"fused write {w.name} {dtype} bs={bs}")
    t = W.make_tensors(w, 3, DEV)
    fused_raw = O.fuse_kv(W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]))
    fused = to_torch(fused_raw, dtype)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], fused, None, slots, layout=FUSED)
    torch.cuda.synchronize()
    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    O.reshape_and_cache_fused(fused_raw, W.raw_numpy(t["key"]), W.raw_numpy(t["value"]), ref_slots)
    assert np.array_equal(W.raw_numpy(fused).view(np.uint8), fused_raw.view(np.uint8))


# ------------------------------------------------------------------ decode and prefill

LENS = [1, 5, 16, 17, 100, 700, 1300, 33]


@pytest.mark.parametrize("dtype,d,bs", [("bf16", 128, 16), ("f16", 64, 16), ("f32", 128, 16), ("f32", 64, 16),
                                        ("bf16", 128, 1), ("bf16", 128, 4), ("f16", 128, 32), ("bf16", 64, 256)])
@pytest.mark.parametrize("ps", [0, 256])
def test_fused_decode_matches_split(dtype, d, bs, ps):
    w = W.custom(LENS, 8, 2, d, dtype, seed=bs + d, extra_cols=1, block_size=bs)
    ps = max(ps, bs) if ps else 0
    say(f"fused decode {dtype} d={d} bs={bs} ps={ps}")
    t = W.make_tensors(w, 1, DEV)
    kr, vr = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    fused = to_torch(O.fuse_kv(kr, vr), dtype)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    split_out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len,
                                       partition_size=ps)
    fused_out = PB.pa_decode_attention(t["query"], fused, None, bt, lens, w.scale, w.max_context_len,
                                       partition_size=ps, layout=FUSED)
    torch.cuda.synchronize()
    assert torch.equal(bits(split_out), bits(fused_out))
    ref = O.decode_attention(W.raw_numpy(t["query"]), kr, vr, w.block_tables, w.context_lens, w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(fused_out), w.dtype) - ref)))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[dtype], err


def test_fused_decode_llama_full_size():
    # the Llama-layer batch converted on the device: every output bitwise equal
    # to the split-layout decode, sampled sequences against the oracle
    w = W.make_workload("llama_gqa4k_bf16")
    say(f"{w.name} fused, full size")
    t = W.make_tensors(w, 0, DEV)
    fused = torch.empty((w.num_blocks, w.num_kv_heads, w.block_size, 2 * w.head_dim), dtype=torch.bfloat16,
                        device=DEV)
    PB.pa_convert_blocks(fused, None, FUSED, t["k_pool"], t["v_pool"], SPLIT, ids(range(w.num_blocks)),
                         ids(range(w.num_blocks)))
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    ps = PB.pa_decode_partition_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                                     w.block_size, torch.bfloat16, context_lens=w.context_lens)
    split_out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len,
                                       partition_size=ps)
    fused_out = PB.pa_decode_attention(t["query"], fused, None, bt, lens, w.scale, w.max_context_len,
                                       partition_size=ps, layout=FUSED)
    torch.cuda.synchronize()
    assert torch.equal(bits(split_out), bits(fused_out))
    for b in (0, 97, 255):
        nb = O.num_blocks(int(w.context_lens[b]), w.block_size)
        blk = torch.from_numpy(w.block_tables[b, :nb].astype(np.int64)).to(DEV)
        kf, vf = O.split_kv(W.raw_numpy(fused[blk]))
        ref = O.decode_attention(W.raw_numpy(t["query"][b:b + 1]), kf, vf, [list(range(nb))],
                                 [int(w.context_lens[b])], w.scale, w.dtype)
        err = float(np.max(np.abs(O.widen(W.raw_numpy(fused_out[b:b + 1]), w.dtype) - ref)))
        assert err <= TOL["bf16"], (b, err)


@pytest.mark.parametrize("ps", [0, 64])
def test_fused_prefill_matches_split(ps):
    pb = W.mixed_varlen_bf16(seed=2)
    w = pb.workload
    say(f"fused prefill {pb.name} ps={ps}")
    t = W.make_prefill_tensors(pb, 0, DEV)
    kr, vr = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    fused = to_torch(O.fuse_kv(kr, vr), "bf16")
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    args = (bt, lens, t["query_start_loc"], w.scale, pb.max_query_len, w.max_context_len)
    split_out = PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], *args, partition_size=ps)
    fused_out = PB.pa_prefill_attention(t["query"], fused, None, *args, partition_size=ps, layout=FUSED)
    torch.cuda.synchronize()
    assert torch.equal(bits(split_out), bits(fused_out))
    ref = O.paged_attention(W.raw_numpy(t["query"]), kr, vr, w.block_tables, w.context_lens, pb.query_start_loc,
                            w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(fused_out), w.dtype) - ref)))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("bs,d", [(16, 128), (4, 64), (64, 128)])
def test_fused_prefill_f32_matches_split(bs, d):
    # the fp32 column tile over a fused pool: the same rows in the same order
    # as over the split pools (bitwise), at pool blocks of 16, 4 and 64 tokens
    pb = W.prefill_batch([1, 7, 100, 700, 1500], [1, 7, 64, 300, 520], 8, 2, d, "f32", seed=bs + d,
                         extra_cols=1, block_size=bs)
    w = pb.workload
    say(f"fused fp32 prefill bs={bs} d={d}")
    t = W.make_prefill_tensors(pb, 0, DEV)
    kr, vr = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    fused = to_torch(O.fuse_kv(kr, vr), "f32")
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    args = (bt, lens, t["query_start_loc"], w.scale, pb.max_query_len, w.max_context_len)
    split_out = PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], *args)
    fused_out = PB.pa_prefill_attention(t["query"], fused, None, *args, layout=FUSED)
    torch.cuda.synchronize()
    assert torch.equal(bits(split_out), bits(fused_out))
    ref = O.paged_attention(W.raw_numpy(t["query"]), kr, vr, w.block_tables, w.context_lens, pb.query_start_loc,
                            w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(fused_out), w.dtype) - ref)))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL["f32"], err


# ------------------------------------------------------------------ shared-prefix decode

@pytest.mark.parametrize("bs", [16, 4, 32])
def test_shared_prefix_decode_fused_equals_split(bs):
    # the cascade over a fused pool reads the same rows in the same order as
    # over the split pools: bitwise equal outputs, within 2e-2 of the oracle;
    # block 16 takes the one-launch form, 4 and 32 the three passes
    from test_gpu_shared_prefix import forked_batch
    rng = np.random.default_rng(bs + 40)
    prompts = [int(x) for x in rng.integers(2 * bs, 300, 24)]
    forks = [int(x) for x in rng.integers(1, 9, 24)]
    gens = [[int(x) for x in rng.integers(1, 50, f)] for f in forks]
    w = forked_batch(prompts, forks, gens, 32, 8, 128, "bf16", seed=bs, bs=bs)
    say(f"shared prefix fused vs split bs={bs} B={w.num_seqs}")
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, bs)
    t = W.make_tensors(w, 2, DEV)
    fused = to_torch(O.fuse_kv(W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])), w.dtype)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    split_out = PB.pa_decode_attention_shared_prefix(t["query"], t["k_pool"], t["v_pool"], bt, lens, g, w.scale,
                                                     w.max_context_len)
    fused_out = PB.pa_decode_attention_shared_prefix(t["query"], fused, None, bt, lens, g, w.scale,
                                                     w.max_context_len, layout=FUSED)
    torch.cuda.synchronize()
    assert torch.equal(bits(split_out), bits(fused_out))
    ref = O.decode_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                             w.block_tables, w.context_lens, w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(fused_out), w.dtype) - ref)))
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[w.dtype]
