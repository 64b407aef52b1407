"""Shared-prefix groups found on the host, and the cascade decode's host-side
argument checks (no GPU)."""

import ctypes

import numpy as np
import pytest

from paged_kv_cache_size_amd import binding as B
from paged_kv_cache_size_amd import workloads as W


def test_groups_of_the_parallel_sampling_workload():
    # 64 prompts of 300 tokens, 6 samples each: the 18 whole prompt blocks are
    # shared, the 12-token tail was copied on write by 5 of the 6
    w = W.make_workload("shared_prefix_bf16")
    g = B.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
    assert (g.num_groups, g.max_group_size, g.max_prefix_len) == (64, 6, 288)
    assert g.group_start.tolist() == list(range(0, 385, 6))
    assert (g.prefix_lens == 288).all() and (g.seq_prefix_lens == 288).all()


def test_no_sharing_gives_singletons():
    w = W.make_workload("qwen1p5b_bf16")
    g = B.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
    assert g.num_groups == w.num_seqs and g.max_group_size == 1 and g.max_prefix_len == 0
    assert (g.prefix_lens == 0).all()


def test_hand_built_tables():
    bt = np.array([[1, 2, 3], [1, 2, 4], [1, 5, 6], [7, 8, 9], [7, 8, 10]], np.int32)
    lens = np.array([40, 40, 40, 40, 33], np.int32)  # whole blocks before the last token: 2
    g = B.pa_shared_prefix_groups(bt, lens, 16)
    assert g.group_start.tolist() == [0, 3, 5] and g.prefix_lens.tolist() == [16, 32]
    assert g.seq_prefix_lens.tolist() == [16, 16, 16, 32, 32]
    g = B.pa_shared_prefix_groups(bt, lens, 16, min_prefix_blocks=2)
    assert g.group_start.tolist() == [0, 2, 3, 5] and g.prefix_lens.tolist() == [32, 0, 32]
    # the last token's block is never part of a prefix, even when shared
    g = B.pa_shared_prefix_groups(bt[:2], np.array([17, 17], np.int32), 16)
    assert g.prefix_lens.tolist() == [16]
    g = B.pa_shared_prefix_groups(bt[:2], np.array([16, 16], np.int32), 16)
    assert g.prefix_lens.tolist() == [0, 0]


FAKE = ctypes.c_void_p(0x1000)


def cascade(**kw):
    a = dict(out=FAKE, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, gs=FAKE, pl=FAKE, spl=FAKE, B=12, G=2, gmax=6,
             H=8, Hkv=2, D=128, bs=16, mb=8, maxlen=128, maxpre=64, scale=0.088, dtype=B.PA_BF16, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return B.lib().pa_decode_attention_shared_prefix(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["lens"], a["gs"], a["pl"], a["spl"], a["B"], a["G"], a["gmax"],
        a["H"], a["Hkv"], a["D"], a["bs"], a["mb"], a["maxlen"], a["maxpre"], a["scale"], a["dtype"], a["ws"],
        a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(gs=None), B.PA_ERR_INVALID_ARG),
    (dict(spl=None), B.PA_ERR_INVALID_ARG),
    (dict(G=0), B.PA_ERR_INVALID_ARG),
    (dict(G=13), B.PA_ERR_INVALID_ARG),
    (dict(gmax=0), B.PA_ERR_INVALID_ARG),
    (dict(maxpre=24), B.PA_ERR_INVALID_ARG),      # not whole blocks
    (dict(maxpre=144), B.PA_ERR_INVALID_ARG),     # longer than any context
    (dict(dtype=B.PA_F32), B.PA_ERR_UNSUPPORTED),
    (dict(D=96), B.PA_ERR_UNSUPPORTED),
    (dict(bs=24, mb=6, maxpre=48), B.PA_ERR_UNSUPPORTED),  # block sizes are powers of two
    (dict(bs=32, mb=4, maxpre=48), B.PA_ERR_INVALID_ARG),  # the prefix is whole blocks
    (dict(ws=None), B.PA_ERR_WORKSPACE),
    (dict(wsb=100), B.PA_ERR_WORKSPACE),
])
def test_cascade_argument_checks(kw, status):
    assert cascade(**kw) == status


def test_cascade_workspace_size():
    # one prefix partition and one suffix partition of 1024 tokens: 2 slots
    assert B.lib().pa_shared_prefix_workspace_bytes(12, 8, 128, 128, 64) == 12 * 8 * 2 * 130 * 4
    assert B.lib().pa_shared_prefix_workspace_bytes(12, 8, 128, 3000, 2048) == 12 * 8 * (2 + 3) * 130 * 4
    assert B.lib().pa_shared_prefix_workspace_bytes(12, 8, 128, 128, 256) == 0  # prefix longer than context
