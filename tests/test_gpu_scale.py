"""Scales other than 1/sqrt(head_dim): negative, zero and large.

The pages fix the scale at head_dim ** -0.5, but the library takes any finite
float, so every tile must honour it: a negative scale turns the largest raw
score into the smallest scaled one (the tiles keep their running max on
scaled scores), a zero scale makes the softmax uniform over the visible keys
(a masked key must not become -inf * 0 = NaN), and a large one makes the
running max move often.  Decode (MFMA and VALU tiles), prefill (per-wave and
cooperative tiles, split and unsplit, fp32 rows) and the shared-prefix cascade
are compared with the float64 oracle at the same scale.
"""

import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_size_amd import binding as PB
from paged_kv_cache_size_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOLS = {"bf16": 2e-2, "f16": 2e-2, "f32": 1e-5}
SCALES = [-0.08838834764831845, 0.0, 0.5]


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def with_scale(w, scale):
    return dataclasses.replace(w, scale=float(np.float32(scale)))


def check(got, ref, dtype):
    got = O.widen(W.raw_numpy(got), dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got - ref)))
    say(f"  max abs err {err:.3e} (tol {TOLS[dtype]})")
    assert err <= TOLS[dtype], err


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("name,ps", [("qwen1p5b_bf16", 0), ("qwen1p5b_bf16", 64), ("tiny_f32", 16)])
def test_decode_scales(name, ps, scale):
    w = with_scale(W.make_workload(name), scale)
    say(f"decode {name} ps={ps} scale={w.scale}")
    t = W.make_tensors(w, 3, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len,
                                 partition_size=ps)
    torch.cuda.synchronize()
    ref = O.decode_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                             w.block_tables, w.context_lens, w.scale, w.dtype)
    check(out, ref, w.dtype)


LENS = [1, 7, 16, 33, 100, 260, 700]


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("dtype,qlens,ps", [
    # columns per KV head = new tokens x 4 query heads; the widest sequence
    # picks the tile: per-wave (<= 16), cooperative 2x1 (<= 32), 2x2 (<= 64), 4x2
    ("bf16", [1, 2, 1, 3, 1, 2, 4], 0),
    ("bf16", [1, 7, 5, 8, 1, 2, 6], 0),
    ("bf16", [1, 7, 5, 16, 9, 2, 12], 0),
    ("bf16", [1, 7, 5, 33, 50, 17, 300], 0),
    ("bf16", [1, 7, 5, 33, 50, 17, 300], 64),  # split and merged
    ("f16", [1, 7, 5, 33, 50, 17, 300], 0),
    ("f32", [1, 7, 5, 33, 50, 17, 300], 0),   # fp32 rows
])
def test_prefill_scales(dtype, qlens, ps, scale):
    pb = W.prefill_batch(LENS, qlens, 8, 2, 128, dtype, seed=5)
    pb = dataclasses.replace(pb, workload=with_scale(pb.workload, scale))
    w = pb.workload
    say(f"prefill {dtype} qlens={qlens} ps={ps} scale={w.scale}")
    t = W.make_prefill_tensors(pb, 4, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    out = PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, t["query_start_loc"], w.scale,
                                  pb.max_query_len, w.max_context_len, partition_size=ps)
    torch.cuda.synchronize()
    ref = O.paged_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                            w.block_tables, w.context_lens, pb.query_start_loc, w.scale, w.dtype)
    check(out, ref, w.dtype)


@pytest.mark.parametrize("scale", SCALES)
def test_cascade_scales(scale):
    w = with_scale(W.make_workload("shared_prefix_bf16"), scale)
    say(f"cascade shared_prefix_bf16 scale={w.scale}")
    t = W.make_tensors(w, 6, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    g = PB.pa_shared_prefix_groups(w.block_tables, w.context_lens, w.block_size)
    out = PB.pa_decode_attention_shared_prefix(t["query"], t["k_pool"], t["v_pool"], bt, lens, g, w.scale,
                                               w.max_context_len)
    torch.cuda.synchronize()
    ref = O.decode_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                             w.block_tables, w.context_lens, w.scale, w.dtype)
    check(out, ref, w.dtype)
