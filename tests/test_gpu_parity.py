"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Every case runs the whole decode hot path on the device - slot mapping, the
pool write, paged attention (and the split-context merge when the context is
partitioned) - and compares with the oracle on the same seeded inputs:

  * slots and the written pools: bit-exact, over the whole pool;
  * attention: max-abs error <= 1e-5 (fp32) / 2e-2 (bf16, fp16) against the
    unrounded float64 oracle.

The two full-size workloads (256 x 4096 GQA bf16, the 200-sequence OPT-13B
MHA fp16 batch) are checked on every sequence and every pool byte, both at
the partition size a scheduler launches with and through the plain
pa_decode_attention entry point.
"""

import ctypes
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_size_amd import binding as PB
from paged_kv_cache_size_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "f16": 2e-2, "bf16": 2e-2}
DEV = "cuda"


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def poison(w, t):
    """NaN into every slot no context position before this step owns: unowned
    blocks (the table padding included) and the last block's slots from the
    new token's position on."""
    ids = torch.from_numpy(w.unowned_blocks).to(DEV)
    for key in ("k_pool", "v_pool"):
        t[key][ids] = float("nan")
    slots = []
    for b in range(w.num_seqs):
        L = int(w.context_lens[b])
        for p in range(max(L - 1, 0), O.num_blocks(L, w.block_size) * w.block_size):
            slots.append(O.slot_for(w.block_tables[b], p, w.block_size))
    if slots:
        s = torch.tensor(slots, device=DEV)
        for key in ("k_pool", "v_pool"):
            t[key].view(-1, w.num_kv_heads, w.head_dim)[s] = float("nan")


def gpu_step(w, t, partition_size=0):
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale,
                                 max(w.max_context_len, 1), partition_size=partition_size)
    torch.cuda.synchronize()
    return slots, out


def check_whole(w, seed=0, partition_size=0, poisoned=False):
    """Whole-batch parity; returns the GPU output."""
    say(f"{w.name} seed={seed} ps={partition_size} poison={poisoned} B={w.num_seqs} "
        f"H={w.num_heads}/{w.num_kv_heads} D={w.head_dim} {w.dtype}")
    t = W.make_tensors(w, seed, DEV)
    if poisoned:
        poison(w, t)
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    q, key, val = W.raw_numpy(t["query"]), W.raw_numpy(t["key"]), W.raw_numpy(t["value"])
    slots, out = gpu_step(w, t, partition_size)

    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    O.reshape_and_cache(kp, key, ref_slots)
    O.reshape_and_cache(vp, val, ref_slots)
    assert np.array_equal(W.raw_numpy(t["k_pool"]).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(W.raw_numpy(t["v_pool"]).view(np.uint8), vp.view(np.uint8))

    ref = O.decode_attention(q, kp, vp, w.block_tables, w.context_lens, w.scale, w.dtype)
    got = O.widen(W.raw_numpy(out), w.dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3e} (tol {TOL[w.dtype]})")
    assert err <= TOL[w.dtype], err
    return out, t


# ------------------------------------------------------------------ the five workloads

def test_tiny_fp32_full():
    w = W.make_workload("tiny_f32")
    out, t = check_whole(w)
    # context of one token: the output is that token's value row, exactly
    rep = w.num_heads // w.num_kv_heads
    for h in range(w.num_heads):
        assert torch.equal(out[0, h], t["value"][0, h // rep])


def test_qwen1p5b_bf16_full():
    check_whole(W.make_workload("qwen1p5b_bf16"))


def test_shared_prefix_bf16_full():
    check_whole(W.make_workload("shared_prefix_bf16"))


def oracle_decode(q, kp, vp, tables, lens, scale, dtype, workers=8):
    """O.decode_attention over every sequence, the batch cut into contiguous
    runs of sequences evaluated side by side in threads (NumPy releases the
    interpreter lock in its array loops); each run is one plain oracle call."""
    n = len(lens)
    cuts = np.linspace(0, n, min(workers, n) + 1).astype(int)
    runs = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    with ThreadPoolExecutor(len(runs)) as ex:
        parts = list(ex.map(lambda r: O.decode_attention(q[r[0]:r[1]], kp, vp, tables[r[0]:r[1]],
                                                         lens[r[0]:r[1]], scale, dtype), runs))
    return np.concatenate(parts, axis=0)


_FULL = {}


def full_size_reference(name):
    """The oracle's slots, pools after the write and attention output for the
    whole seeded batch of a full-size workload, computed once per process:
    the tensors come from the same generator on the device, are copied to the
    host before any library call, and go through the oracle only."""
    if name not in _FULL:
        w = W.make_workload(name)
        t = W.make_tensors(w, 0, DEV)
        kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
        q, key, val = W.raw_numpy(t["query"]), W.raw_numpy(t["key"]), W.raw_numpy(t["value"])
        del t
        torch.cuda.empty_cache()
        slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
        O.reshape_and_cache(kp, key, slots)
        O.reshape_and_cache(vp, val, slots)
        ref = oracle_decode(q, kp, vp, w.block_tables, w.context_lens, w.scale, w.dtype)
        _FULL.clear()  # one workload's pools on the host at a time
        _FULL[name] = (w, slots, kp, vp, ref)
    return _FULL[name]


def check_full_size(name, partition_size=None):
    """Full-size batch: every sequence's output against the oracle, element by
    element, and both pools after the write byte for byte.

    partition_size None: attention through the plain C entry point
    pa_decode_attention itself (its own blind partition choice, workspace
    sized by pa_decode_workspace_bytes); otherwise pa_decode_attention_ex with
    that size."""
    w, ref_slots, kp, vp, ref = full_size_reference(name)
    how = "pa_decode_attention (plain entry)" if partition_size is None else f"ps={partition_size}"
    say(f"{name} full size, every sequence, {how}")
    t = W.make_tensors(w, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    if partition_size is None:
        lib = PB.lib()
        q = t["query"]
        B, H, D = q.shape
        code = PB.pa_dtype(q)
        need = int(lib.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size))
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
        out = torch.empty_like(q)
        ptr = lambda x: ctypes.c_void_p(x.data_ptr())  # noqa: E731
        rc = lib.pa_decode_attention(ptr(out), ptr(q), ptr(t["k_pool"]), ptr(t["v_pool"]), ptr(bt), ptr(lens), B, H,
                                     w.num_kv_heads, D, w.block_size, w.max_blocks_per_seq, w.max_context_len,
                                     w.scale, code, ptr(ws), need, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert rc == PB.PA_OK, PB.pa_status_string(rc)
    else:
        out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len,
                                     partition_size=partition_size)
    torch.cuda.synchronize()
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    for pool, ref_pool in (("k_pool", kp), ("v_pool", vp)):
        assert np.array_equal(W.raw_numpy(t[pool]).view(np.uint8), ref_pool.view(np.uint8)), pool
    got = O.widen(W.raw_numpy(out), w.dtype)
    err_seq = np.abs(got - ref).reshape(w.num_seqs, -1).max(axis=1)
    worst = int(np.argmax(err_seq))
    say(f"  {w.num_seqs} sequences: max abs err {err_seq[worst]:.3e} (sequence {worst}), "
        f"median {float(np.median(err_seq)):.3e}")
    assert (err_seq <= TOL[w.dtype]).all(), (np.flatnonzero(err_seq > TOL[w.dtype])[:10], float(err_seq[worst]))


def bench_partition_size(w):
    """The size bench.py launches with: the policy given the host-side lengths."""
    ps = PB.pa_decode_partition_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                                     w.block_size, W.torch_dtype(w.dtype), context_lens=w.context_lens)
    assert ps % w.block_size == 0 and w.block_size <= ps <= 256 * w.block_size
    return ps


def test_llama_gqa4k_bf16_full_size_every_sequence():
    w = W.make_workload("llama_gqa4k_bf16")
    check_full_size("llama_gqa4k_bf16", bench_partition_size(w))


def test_llama_gqa4k_bf16_full_size_plain_entry_point():
    check_full_size("llama_gqa4k_bf16", None)


def test_opt13b_mha_f16_full_size_every_sequence():
    w = W.make_workload("opt13b_mha_f16")
    check_full_size("opt13b_mha_f16", bench_partition_size(w))


def test_opt13b_mha_f16_full_size_plain_entry_point():
    check_full_size("opt13b_mha_f16", None)


# ------------------------------------------------------------------ splits, poison, edges

@pytest.mark.parametrize("ps", [16, 48, 128, 1024])
def test_partition_sizes_tiny(ps):
    check_whole(W.make_workload("tiny_f32", extra_cols=2), partition_size=ps)


@pytest.mark.parametrize("ps", [16, 64, 256, 1024])
def test_partition_sizes_qwen(ps):
    check_whole(W.make_workload("qwen1p5b_bf16"), partition_size=ps)


@pytest.mark.parametrize("ps", [128, 512, 1024, 2048, 4096, 0])
def test_partition_sizes_llama_subset(ps):
    check_whole(W.make_workload("llama_gqa4k_bf16", num_seqs=8), partition_size=ps)


@pytest.mark.parametrize("name", ["tiny_f32", "qwen1p5b_bf16", "shared_prefix_bf16"])
def test_poisoned_unowned_and_tail_slots(name):
    check_whole(W.make_workload(name, extra_cols=3), poisoned=True)


EDGE_LENS = [1, 2, 15, 16, 17, 31, 32, 33, 127, 128, 129, 255, 256, 257, 1023, 1024, 1025, 1500]


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("f16", 64), ("f16", 128), ("bf16", 64),
                                     ("bf16", 128)])
@pytest.mark.parametrize("ps", [0, 16, 256])
def test_edge_lengths_all_dtypes(dtype, d, ps):
    w = W.custom(EDGE_LENS, 8, 2, d, dtype, seed=5, extra_cols=1)
    check_whole(w, seed=5, partition_size=ps, poisoned=True)


@pytest.mark.parametrize("h,hkv", [(4, 4), (8, 4), (12, 4), (16, 4), (10, 2), (12, 2), (14, 2), (16, 2),
                                   (32, 2), (32, 1), (9, 1), (22, 2), (64, 1), (128, 8), (64, 64)])
def test_head_groupings(h, hkv):
    w = W.custom([1, 40, 300, 777], h, hkv, 128, "bf16", seed=h * 100 + hkv)
    check_whole(w, seed=3, partition_size=128)
    check_whole(w, seed=3, partition_size=0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_very_long_contexts(dtype):
    # contexts far beyond one partition's 256 blocks: up to 128K tokens, an odd
    # length one past a power of two, a single token; the policy's partition
    # given the lengths, the blind one, and a fixed 4096
    lens = [131072, 65537, 1, 4097] if dtype == "bf16" else [70001, 16385, 1]
    w = W.custom(lens, 32, 8, 128, dtype, seed=11, extra_cols=1)
    for ps in (bench_partition_size(w), 0, 4096):
        check_whole(w, seed=3, partition_size=ps)


def test_split_kv_agrees_with_one_partition():
    # fp32 (the tile computes scores, probabilities and P.V in float32): the
    # split-context merge changes only the summation order, so every
    # partition size agrees with the single-partition result to a few float32
    # ulps of the sums.  (The 16-bit tiles round probabilities to the input
    # dtype relative to each partition's own running max, so there the
    # partitions differ by that rounding and the oracle tolerance applies.)
    w = W.custom([1, 16, 17, 300, 1000, 2047], 8, 2, 128, "f32", seed=4)
    t = W.make_tensors(w, 2, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    run = lambda ps: PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale,  # noqa: E731
                                            w.max_context_len, partition_size=ps)
    one = run(2048)
    for ps in (16, 128, 512, 1024):
        diff = (run(ps) - one).abs()
        assert float(diff.max()) <= 4e-6 * max(1.0, float(one.abs().max())), ps


def test_zero_length_context_gives_zeros():
    w = W.custom([0, 5, 0, 20], 4, 2, 64, "f32", seed=2)
    t = W.make_tensors(w, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    for ps in (16, 0):
        out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, 20,
                                     partition_size=ps)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out[0]) == 0 and torch.count_nonzero(out[2]) == 0
        ref = O.decode_attention(W.raw_numpy(t["query"])[[1, 3]], W.raw_numpy(t["k_pool"]),
                                 W.raw_numpy(t["v_pool"]), w.block_tables[[1, 3]], [5, 20], w.scale, "f32")
        assert np.max(np.abs(out[[1, 3]].cpu().numpy() - ref)) <= 1e-5


@pytest.mark.parametrize("name", ["tiny_f32", "qwen1p5b_bf16"])
def test_empty_batch_changes_nothing(name):
    # no sequence: slot mapping, the pool write, decode and prefill all return
    # empty results and leave the pools bitwise untouched
    w = W.make_workload(name)
    say(f"empty batch on the pools of {name}")
    t = W.make_tensors(w, 0, DEV)
    kp0, vp0 = t["k_pool"].clone(), t["v_pool"].clone()
    H, D = t["query"].shape[1:]
    bt = torch.empty((0, w.block_tables.shape[1]), dtype=torch.int32, device=DEV)
    lens = torch.empty(0, dtype=torch.int32, device=DEV)
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"][:0], t["value"][:0], t["k_pool"], t["v_pool"], slots)
    q = t["query"][:0]
    out = PB.pa_decode_attention(q, t["k_pool"], t["v_pool"], bt, lens, w.scale)
    out16 = PB.pa_decode_attention(q, t["k_pool"], t["v_pool"], bt, lens, w.scale, 64, partition_size=16)
    qsl = torch.zeros(1, dtype=torch.int32, device=DEV)
    pre = PB.pa_prefill_attention(q, t["k_pool"], t["v_pool"], bt, lens, qsl, w.scale, 0, 64)
    torch.cuda.synchronize()
    assert slots.shape == (0,) and out.shape == (0, H, D) and out16.shape == (0, H, D) and pre.shape == (0, H, D)
    assert torch.equal(bits(t["k_pool"]), bits(kp0)) and torch.equal(bits(t["v_pool"]), bits(vp0))


# ------------------------------------------------------------------ properties

def test_block_permutation_gives_bitwise_identical_output():
    w = W.make_workload("qwen1p5b_bf16")
    t = W.make_tensors(w, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    base = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len)
    perm = torch.from_numpy(np.random.default_rng(9).permutation(w.num_blocks)).to(DEV)
    kp2, vp2 = torch.empty_like(t["k_pool"]), torch.empty_like(t["v_pool"])
    kp2[perm], vp2[perm] = t["k_pool"], t["v_pool"]
    bt2 = perm[bt.long()].to(torch.int32)
    again = PB.pa_decode_attention(t["query"], kp2, vp2, bt2, lens, w.scale, w.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(bits(base), bits(again))


def test_run_to_run_bitwise_determinism():
    w = W.make_workload("llama_gqa4k_bf16", num_seqs=16)
    t = W.make_tensors(w, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    outs = [PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, 4096,
                                   partition_size=ps) for ps in (256, 256, 0, 0)]
    torch.cuda.synchronize()
    assert torch.equal(bits(outs[0]), bits(outs[1])) and torch.equal(bits(outs[2]), bits(outs[3]))
    # different splits agree to float32 rounding
    assert (outs[0].float() - outs[2].float()).abs().max().item() < 1e-2


def test_varlen_slot_mapping_matches_oracle():
    w = W.custom([5, 37, 20, 64, 1], 8, 2, 64, "f32", seed=4)
    qlens = [2, 7, 20, 16, 1]
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    got = PB.pa_slot_mapping(bt, lens, w.block_size, query_start_loc=torch.from_numpy(qsl).to(DEV),
                             num_tokens=int(qsl[-1]))
    ref = O.slot_mapping(w.block_tables, w.context_lens, w.block_size, query_lens=qlens)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_reshape_skips_out_of_range_slots():
    w = W.custom([3, 9], 4, 2, 64, "bf16", seed=6)
    t = W.make_tensors(w, 0, DEV)
    before = t["k_pool"].clone()
    nslots = w.num_blocks * w.block_size
    slots = torch.tensor([-1, nslots], dtype=torch.int64, device=DEV)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    torch.cuda.synchronize()
    assert torch.equal(bits(before), bits(t["k_pool"]))


# ------------------------------------------------------------------ pool block sizes

BS_LENS = [1, 5, 16, 17, 100, 700, 1300, 33]


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 64, 128, 256])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64), ("f32", 64), ("f32", 128)])
def test_block_sizes(bs, dtype, d):
    # blocks smaller than the 16-token MFMA step are gathered row by row,
    # larger ones are walked in 16-row windows; NaN in every unowned slot
    w = W.custom(BS_LENS, 8, 2, d, dtype, seed=bs, extra_cols=1, block_size=bs)
    check_whole(w, seed=bs, partition_size=0, poisoned=True)
    check_whole(w, seed=bs, partition_size=max(16, bs), poisoned=True)


@pytest.mark.parametrize("bs,ps", [(1, 1024), (2, 2048), (8, 8192), (1, 1008)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_blocks_long_partitions(bs, ps, dtype):
    # blocks under 16 tokens: the partition's table (up to 1024 entries) sits
    # in LDS, so partitions may hold 1024 blocks
    w = W.custom(BS_LENS + [3000, 8192], 8, 2, 128, dtype, seed=bs, extra_cols=1, block_size=bs)
    check_whole(w, seed=bs, partition_size=ps, poisoned=True)


@pytest.mark.parametrize("bs", [4, 64])
def test_block_sizes_full_partition_policy(bs):
    # the policy's choice given the lengths, as a scheduler would launch it
    w = W.custom([4096] * 8 + [37, 900], 32, 8, 128, "bf16", seed=3, block_size=bs)
    ps = PB.pa_decode_partition_size(w.num_seqs, w.num_heads, w.num_kv_heads, w.head_dim, w.max_context_len,
                                     w.block_size, torch.bfloat16, context_lens=w.context_lens)
    assert ps % max(16, bs) == 0 and ps <= 256 * bs
    check_whole(w, seed=1, partition_size=ps)
