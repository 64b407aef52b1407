"""pa_decode_attention_noalloc: the decode entry point without a workspace
argument (its split-context partials live in the library's static per-GPU
buffer) against pa_decode_attention_ex with a workspace PyTorch allocates, on
the same inputs and partition size, and both against the float64 oracle.

Two calls in a row on one GPU, the second with a smaller batch, so the second
runs over the buffer the first left filled."""

import ctypes
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


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def noalloc(q, kp, vp, bt, lens, w, partition_size):
    B, H, D = q.shape
    out = torch.empty_like(q)
    rc = PB.lib().pa_decode_attention_noalloc(
        ptr(out), ptr(q), ptr(kp), ptr(vp), ptr(bt), ptr(lens), B, H, w.num_kv_heads, D, w.block_size,
        w.max_blocks_per_seq, w.max_context_len, w.scale, PB.pa_dtype(q), int(partition_size),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc, out


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def one_call(w, partition_size, seed):
    say(f"noalloc {w.description} ps={partition_size}")
    t = W.make_tensors(w, seed, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    if partition_size:
        need = PB.pa_decode_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim, w.max_context_len, w.block_size,
                                            partition_size)
        assert need > 0  # the context is split: the static buffer is used
    rc, got = noalloc(t["query"], t["k_pool"], t["v_pool"], bt, lens, w, partition_size)
    assert rc == PB.PA_OK, PB.pa_status_string(rc)
    ref_gpu = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len,
                                     partition_size=partition_size)
    torch.cuda.synchronize()
    # same kernels, same partition size: the same bits
    assert torch.equal(bits(got), bits(ref_gpu))
    ref = O.decode_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                             w.block_tables, w.context_lens, w.scale, w.dtype)
    err = float(np.max(np.abs(O.widen(W.raw_numpy(got), w.dtype) - ref)))
    say(f"  bitwise equal to the workspace entry point; max abs err vs oracle {err:.3e}")
    assert err <= TOL[w.dtype], err


def test_noalloc_two_calls_second_smaller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    big = W.make_workload("llama_gqa4k_bf16", num_seqs=24)                # 24 x 4096, 8 partitions of 512
    small = W.custom([1, 17, 300, 1000, 2047], 12, 2, 128, "bf16", seed=3)  # fewer, shorter contexts
    one_call(big, 512, seed=1)
    one_call(small, 256, seed=2)
    one_call(W.custom([5, 37, 20], 8, 2, 64, "f32", seed=4), 16, seed=5)
    one_call(small, 0, seed=6)  # the library's own partition choice


def test_noalloc_refuses_partials_beyond_the_buffer():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # 4096 sequences x 64 heads x 256 partitions of 16 tokens: about 35 GB of
    # partials against the 64 MiB buffer; refused before anything is enqueued
    w = W.custom([1], 64, 8, 128, "bf16", seed=0)
    t = W.make_tensors(w, 0, DEV)
    B = 4096
    q = torch.zeros((B, 64, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((B, 256), dtype=torch.int32, device=DEV)
    lens = torch.ones(B, dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    rc = PB.lib().pa_decode_attention_noalloc(ptr(out), ptr(q), ptr(t["k_pool"]), ptr(t["v_pool"]), ptr(bt),
                                              ptr(lens), B, 64, 8, 128, 16, 256, 4096, w.scale, PB.PA_BF16, 16,
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == PB.PA_ERR_WORKSPACE
