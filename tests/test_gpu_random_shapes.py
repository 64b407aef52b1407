"""Seeded random-shape parity sweep of the whole path against the float64 oracle.

Each case draws its own shape from a seeded generator: batch size, KV heads
and query heads per KV head (1 to 16), head size, dtype, pool block size (a
power of two from 1 to 256), ragged context lengths from 1 to a few thousand,
new tokens per sequence (prefill), an explicit partition size or the
library's choice, NaN in every slot the step must not read, and the pool
layout.  It then runs slot mapping, the pool write and attention on the
device and compares with the oracle on the same inputs: slots and pools
bit-exact, attention max-abs error <= 1e-5 (fp32) / 2e-2 (bf16, fp16)
against the unrounded float64 result, and the fused K|V layout bitwise equal
to the split one.  The generator's seed is the case id, printed before the
case runs.
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
BLOCK_SIZES = [1, 2, 4, 8, 16, 32, 64, 128, 256]


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def to_torch(raw, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(raw)).to(DEV)


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def draw_shape(rng, max_len):
    """Heads, head size, dtype, block size and ragged lengths of one case."""
    hkv = int(rng.choice([1, 2, 3, 4, 8]))
    group = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    d = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["f32", "f16", "bf16"]))
    bs = int(rng.choice(BLOCK_SIZES))
    b = int(rng.integers(1, 13))
    # log-uniform lengths: many short contexts, a few long ones
    lens = np.exp(rng.uniform(0.0, np.log(max_len), size=b)).astype(np.int64) + 1
    return hkv * group, hkv, d, dtype, bs, [int(x) for x in lens]


def draw_partition(rng, bs, max_len):
    """0 (the library's choice) or a size the entry points accept: a multiple
    of max(16, block_size) of at most 256 blocks (1024 under 16 tokens),
    drawn so that it often splits the longest context."""
    if rng.random() < 0.3:
        return 0
    unit = max(16, bs)
    cap = (1024 if bs < 16 else 256) * bs // unit
    top = max(1, min(cap, -(-max_len // unit) + 1))
    return unit * int(rng.integers(1, top + 1))


def poison_decode(w, t):
    ids = torch.from_numpy(w.unowned_blocks).to(DEV)
    for key in ("k_pool", "v_pool"):
        t[key][ids] = float("nan")
    slots = []
    for b in range(w.num_seqs):
        L = int(w.context_lens[b])
        for p in range(L - 1, O.num_blocks(L, w.block_size) * w.block_size):
            slots.append(O.slot_for(w.block_tables[b], p, w.block_size))
    s = torch.tensor(slots, device=DEV)
    for key in ("k_pool", "v_pool"):
        t[key].view(-1, w.num_kv_heads, w.head_dim)[s] = float("nan")


def poison_prefill(pb, t):
    w = pb.workload
    ids = torch.from_numpy(w.unowned_blocks).to(DEV)
    for key in ("k_pool", "v_pool"):
        t[key][ids] = float("nan")
    slots = []
    for b in range(w.num_seqs):
        L, n = int(w.context_lens[b]), int(pb.query_lens[b])
        for p in range(L - n, O.num_blocks(L, w.block_size) * w.block_size):
            slots.append(O.slot_for(w.block_tables[b], p, w.block_size))
    s = torch.tensor(slots, device=DEV)
    for key in ("k_pool", "v_pool"):
        t[key].view(-1, w.num_kv_heads, w.head_dim)[s] = float("nan")


def check_pools(w, t, kp, vp, key, val, ref_slots):
    O.reshape_and_cache(kp, key, ref_slots)
    O.reshape_and_cache(vp, val, ref_slots)
    assert np.array_equal(W.raw_numpy(t["k_pool"]).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(W.raw_numpy(t["v_pool"]).view(np.uint8), vp.view(np.uint8))


def check_attention(got_t, ref, dtype):
    got = O.widen(W.raw_numpy(got_t), dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("case", range(96))
def test_random_decode(case):
    rng = np.random.default_rng(1000 + case)
    h, hkv, d, dtype, bs, lens = draw_shape(rng, 4000)
    ps = draw_partition(rng, bs, max(lens))
    poisoned, fused = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    say(f"decode case {case}: B={len(lens)} H={h}/{hkv} D={d} {dtype} bs={bs} ps={ps} "
        f"poison={poisoned} fused={fused} lens={lens}")
    w = W.custom(lens, h, hkv, d, dtype, seed=case, extra_cols=int(rng.integers(0, 3)), name=f"random{case}",
                 block_size=bs)
    t = W.make_tensors(w, case, DEV)
    if poisoned:
        poison_decode(w, t)
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    q, key, val = W.raw_numpy(t["query"]), W.raw_numpy(t["key"]), W.raw_numpy(t["value"])

    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, cl, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, cl, w.scale, w.max_context_len,
                                 partition_size=ps)
    torch.cuda.synchronize()

    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    check_pools(w, t, kp, vp, key, val, ref_slots)
    check_attention(out, O.decode_attention(q, kp, vp, w.block_tables, w.context_lens, w.scale, w.dtype), dtype)

    if fused:
        pool = to_torch(O.fuse_kv(kp, vp), dtype)
        fout = PB.pa_decode_attention(t["query"], pool, None, bt, cl, w.scale, w.max_context_len,
                                      partition_size=ps, layout=PB.PA_KV_FUSED)
        torch.cuda.synchronize()
        assert torch.equal(bits(fout), bits(out))


@pytest.mark.parametrize("case", range(64))
def test_random_prefill(case):
    rng = np.random.default_rng(2000 + case)
    h, hkv, d, dtype, bs, lens = draw_shape(rng, 2500)
    # new tokens: a decode step, a short chunk, or most of the context
    qlens = []
    for L in lens:
        kind = rng.integers(0, 3)
        n = 1 if kind == 0 else int(rng.integers(1, min(L, 40) + 1)) if kind == 1 else int(rng.integers(1, L + 1))
        qlens.append(n)
    ps = draw_partition(rng, bs, max(lens))
    poisoned, fused = bool(rng.random() < 0.5), bool(rng.random() < 0.5)
    say(f"prefill case {case}: B={len(lens)} H={h}/{hkv} D={d} {dtype} bs={bs} ps={ps} "
        f"poison={poisoned} fused={fused} lens={lens} qlens={qlens}")
    pb = W.prefill_batch(lens, qlens, h, hkv, d, dtype, seed=case, name=f"random{case}",
                         extra_cols=int(rng.integers(0, 3)), block_size=bs)
    w = pb.workload
    t = W.make_prefill_tensors(pb, case, DEV)
    if poisoned:
        poison_prefill(pb, t)
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    q, key, val = W.raw_numpy(t["query"]), W.raw_numpy(t["key"]), W.raw_numpy(t["value"])

    bt = torch.from_numpy(w.block_tables).to(DEV)
    cl = torch.from_numpy(w.context_lens).to(DEV)
    qsl = t["query_start_loc"]
    slots = PB.pa_slot_mapping(bt, cl, w.block_size, query_start_loc=qsl, num_tokens=pb.num_tokens)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    out = PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], bt, cl, qsl, w.scale, pb.max_query_len,
                                  w.max_context_len, partition_size=ps)
    torch.cuda.synchronize()

    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size, query_lens=pb.query_lens)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    check_pools(w, t, kp, vp, key, val, ref_slots)
    ref = O.paged_attention(q, kp, vp, w.block_tables, w.context_lens, pb.query_start_loc, w.scale, w.dtype)
    check_attention(out, ref, dtype)

    if fused:
        pool = to_torch(O.fuse_kv(kp, vp), dtype)
        fout = PB.pa_prefill_attention(t["query"], pool, None, bt, cl, qsl, w.scale, pb.max_query_len,
                                       w.max_context_len, partition_size=ps, layout=PB.PA_KV_FUSED)
        torch.cuda.synchronize()
        assert torch.equal(bits(fout), bits(out))
