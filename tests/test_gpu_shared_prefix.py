"""GPU parity of the shared-prefix (cascade) decode against the float64 oracle.

The cascade reads each group's shared prompt blocks once for all members,
each sequence's own blocks after the prefix, and merges the two softmax
partials; the oracle is the plain decode definition over each sequence's
whole context.  Tolerance 2e-2 (bf16, fp16); also compared with the library's
plain decode of the same batch.
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
TOL = 2e-2


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def run_cascade(w, t, groups):
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    casc = PB.pa_decode_attention_shared_prefix(t["query"], t["k_pool"], t["v_pool"], bt, lens, groups, w.scale,
                                                w.max_context_len)
    plain = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len)
    torch.cuda.synchronize()
    return casc, plain


def check(w, groups, seed=0, rows=None):
    say(f"{w.name} groups={groups.num_groups} max_group={groups.max_group_size} prefix<= {groups.max_prefix_len} "
        f"B={w.num_seqs} H={w.num_heads}/{w.num_kv_heads} D={w.head_dim} {w.dtype}")
    t = W.make_tensors(w, seed, DEV)
    casc, plain = run_cascade(w, t, groups)
    sel = list(range(w.num_seqs)) if rows is None else rows
    ref = O.decode_attention(W.raw_numpy(t["query"])[sel], W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                             w.block_tables[sel], w.context_lens[sel], w.scale, w.dtype)
    got = O.widen(W.raw_numpy(casc), w.dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got[sel] - ref)))
    diff = float((casc.float() - plain.float()).abs().max())
    say(f"  max abs err {err:.3e}, vs plain decode {diff:.3e}")
    assert err <= TOL and diff <= TOL
    return casc


def test_parallel_sampling_workload():
    w = W.make_workload("shared_prefix_bf16")
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
    assert g.num_groups == 64
    check(w, g, rows=list(range(0, 384, 7)))


def forked_batch(prompts, forks, gens, h, hkv, d, dtype, seed, bs=16):
    """Prompts forked into samples that each generate some tokens, built with
    the library's block pool (copy-on-write pairs replayed by the tensor
    builder, which copies the prompt rows)."""
    rng = np.random.default_rng(seed)
    need = sum(-(-p // bs) + f * (-(-max(gl) // bs) + 1) for p, f, gl in zip(prompts, forks, gens)) + 64
    nb = max(4096 * max(1, 16 // bs), need)  # room for every token at any block size
    m = PB.BlockManager(nb, bs, free_order=rng.permutation(nb))
    seqs, copies = [], []
    for p, f, gl in zip(prompts, forks, gens):
        root = m.new_seq()
        m.append(root, p)
        members = [m.fork(root) for _ in range(f - 1)] + [root]
        for s, extra in zip(members, gl):
            c = m.append(s, extra)
            if c is not None:
                copies.append((c[0], c[1], p % bs))
        seqs += members
    tables = [m.block_table(s) for s in seqs]
    lens = np.array([m.length(s) for s in seqs], np.int32)
    width = max(len(x) for x in tables) + 1
    used = {b for x in tables for b in x}
    pad = min(set(range(nb)) - used)
    bt = np.full((len(seqs), width), pad, np.int32)
    for i, x in enumerate(tables):
        bt[i, :len(x)] = x
    unowned = np.array(sorted(set(range(nb)) - used), np.int64)
    return W.Workload("forked", dtype, h, hkv, d, bs, nb, lens, bt, float(np.float32(1 / np.sqrt(d))), pad,
                      unowned, copies, "forked prompts")


@pytest.mark.parametrize("dtype,d,h,hkv", [("bf16", 128, 32, 8), ("f16", 64, 8, 2), ("bf16", 128, 12, 2),
                                           ("f16", 128, 40, 40)])
def test_mixed_groups(dtype, d, h, hkv):
    # groups of 1..7 members; prefixes from none to over 2 partitions of 1024
    # tokens; suffixes of 1 to 1300 tokens
    prompts = [37, 2100, 16, 600, 1, 333]
    forks = [3, 2, 4, 7, 1, 5]
    rng = np.random.default_rng(7)
    gens = [[int(x) for x in rng.integers(1, 1300 if i == 1 else 60, f)] for i, f in enumerate(forks)]
    w = forked_batch(prompts, forks, gens, h, hkv, d, dtype, seed=3)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, 16)
    assert g.max_prefix_len == 2096 and g.max_group_size == 7
    check(w, g, seed=1)


@pytest.mark.parametrize("bs", [1, 2, 4, 8, 32, 64, 256])
def test_mixed_groups_block_sizes(bs):
    # prefixes are whole pool blocks; the passes gather small blocks row by
    # row and walk large ones in 16-row windows
    prompts = [37, 2100, 16, 600, 1, 333]
    forks = [3, 2, 4, 7, 1, 5]
    rng = np.random.default_rng(bs)
    gens = [[int(x) for x in rng.integers(1, 1300 if i == 1 else 60, f)] for i, f in enumerate(forks)]
    w = forked_batch(prompts, forks, gens, 32, 8, 128, "bf16", seed=bs, bs=bs)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, bs)
    assert g.max_group_size == 7 and g.max_prefix_len % bs == 0 and g.max_prefix_len >= 2100 // bs * bs - bs
    check(w, g, seed=2)


@pytest.mark.parametrize("bs", [1, 4, 16, 64])
def test_many_wide_groups_block_sizes(bs):
    # 64 groups of 6 with 32/8 heads: 24 (member, head) columns per KV head
    # and 512 workgroups, so the prefix pass runs the cooperative tile, with
    # small blocks gathered row by row and large ones walked in windows
    rng = np.random.default_rng(bs + 100)
    prompts = [int(x) for x in rng.integers(max(20, 2 * bs), 200 + 2 * bs, 64)]  # at least one whole block
    forks = [6] * 64
    gens = [[int(x) for x in rng.integers(1, 40, 6)] for _ in range(64)]
    w = forked_batch(prompts, forks, gens, 32, 8, 128, "bf16", seed=bs, bs=bs)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, bs)
    assert g.num_groups == 64 and g.max_group_size == 6
    check(w, g, seed=3)


@pytest.mark.parametrize("bs,dtype,d", [(4, "bf16", 128), (32, "f16", 64)])
def test_wide_group_prefix_pass(bs, dtype, d):
    # a group of 70 samples with 32/8 heads: 280 (member, head) columns per
    # KV head, so the prefix pass (block sizes other than 16 take the passes)
    # runs the cooperative tile over several column groups with its partials
    # in slots
    rng = np.random.default_rng(bs + 300)
    prompts, forks = [300, 90], [70, 3]
    gens = [[int(x) for x in rng.integers(1, 50, f)] for f in forks]
    w = forked_batch(prompts, forks, gens, 32, 8, d, dtype, seed=bs, bs=bs)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, bs)
    assert g.max_group_size == 70
    check(w, g, seed=4)


def test_no_shared_prefix_degenerates_to_plain_decode():
    w = W.make_workload("qwen1p5b_bf16")
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
    assert g.max_prefix_len == 0
    check(w, g)


@pytest.mark.parametrize("h,hkv", [(8, 4), (32, 4), (16, 1), (64, 2), (32, 8)])
def test_group_sizes_and_head_groupings(h, hkv):
    # query heads per KV head 2, 8, 16, 32 (two head chunks) and 4: one to
    # eight members share the 16 columns of a wave, and a group of 16 samples
    # spans several member sets; members of one group end at different lengths
    rng = np.random.default_rng(h + hkv)
    prompts = [300, 77, 1000, 16]
    forks = [16, 5, 3, 9]
    gens = [[int(x) for x in rng.integers(1, 90, f)] for f in forks]
    w = forked_batch(prompts, forks, gens, h, hkv, 128, "bf16", seed=h * 3 + hkv)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, 16)
    assert g.num_groups == 4 and g.max_group_size == 16
    check(w, g, seed=4)


def test_many_small_groups():
    # 300 prompts forked in two: more (group, KV head, member set) units than
    # the machine holds two waves of, so each unit runs on one wave
    rng = np.random.default_rng(11)
    prompts = [int(x) for x in rng.integers(17, 400, 300)]
    forks = [2] * 300
    gens = [[int(x) for x in rng.integers(1, 30, 2)] for _ in range(300)]
    w = forked_batch(prompts, forks, gens, 32, 8, 128, "bf16", seed=11)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, 16)
    assert g.num_groups == 300
    check(w, g, seed=5, rows=list(range(0, 600, 5)))


@pytest.mark.parametrize("prompts,samples,d,dtype", [(40, 3, 128, "bf16"), (160, 3, 128, "bf16"), (48, 6, 128, "bf16"),
                                                     (40, 3, 64, "f16"), (160, 3, 64, "bf16"), (48, 6, 64, "f16")])
def test_merge_across_wave_counts(prompts, samples, d, dtype):
    # 32/8 heads, one (group, KV head) unit per member set: 320 units run four
    # waves per set, 1280 two, and 48 x 6 (two sets of 3) four again with a
    # shared prefix of 1-7 blocks; every wave's partial state is merged in LDS
    # by the waves together, each storing a quarter or a half of every row's
    # dims (8 or 4 bytes per lane at head_dim 64)
    rng = np.random.default_rng(prompts + samples)
    plens = [int(x) for x in rng.integers(17, 120, prompts)]
    gens = [[int(x) for x in rng.integers(1, 40, samples)] for _ in range(prompts)]
    w = forked_batch(plens, [samples] * prompts, gens, 32, 8, d, dtype, seed=prompts)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, 16)
    assert g.num_groups == prompts
    check(w, g, seed=3)


def test_long_shared_prompts():
    # 32 prompts of 3600 tokens, 8 samples each: the set's 237 steps are split
    # over four waves whose partial softmax states are merged in LDS
    w = W.make_workload("shared_prefix_long_bf16")
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
    assert g.num_groups == 32
    check(w, g, rows=list(range(0, 256, 9)))
