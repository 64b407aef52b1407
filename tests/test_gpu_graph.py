"""The hot path captured in a HIP graph.

The library's calls only enqueue kernels on the caller's stream (no memset,
no allocation, no synchronisation when the partition size is given), so a
whole step can be captured once and replayed.  Each test captures a step,
then replays it several times with eager work and synchronisation between
the replays (the output is cleared and the workspace overwritten), and checks
every replay bitwise against the eager step, and the eager step against the
float64 oracle.
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


def capture(step):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, out, ws, eager):
    for i in range(4):
        out.zero_()
        if ws is not None:
            ws.fill_(0x7F)  # stale partials from another "call"
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i}"


@pytest.mark.parametrize("name", ["qwen1p5b_bf16", "shared_prefix_bf16"])
def test_decode_step_graph(name):
    w = W.make_workload(name)
    say(f"graph decode step {name}")
    t = W.make_tensors(w, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    B, H, D = t["query"].shape
    ps = PB.pa_decode_partition_size(B, H, w.num_kv_heads, D, w.max_context_len, w.block_size, torch.bfloat16,
                                     context_lens=w.context_lens)
    ws = torch.empty(max(1, PB.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size, ps)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(t["query"])
    slots = torch.empty(B, dtype=torch.int64, device=DEV)
    kp_raw, vp_raw = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])

    def step():
        PB.pa_slot_mapping(bt, lens, w.block_size, out=slots)
        PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
        PB.pa_decode_partitions(t["query"], t["k_pool"], t["v_pool"], bt, lens, w.scale, w.max_context_len, ps,
                                workspace=ws, out=out)
        PB.pa_decode_combine(out, lens, w.max_context_len, ps, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    O.reshape_and_cache(kp_raw, W.raw_numpy(t["key"]), ref_slots)
    O.reshape_and_cache(vp_raw, W.raw_numpy(t["value"]), ref_slots)
    ref = O.decode_attention(W.raw_numpy(t["query"]), kp_raw, vp_raw, w.block_tables, w.context_lens, w.scale,
                             w.dtype)
    assert float(np.max(np.abs(O.widen(W.raw_numpy(eager), w.dtype) - ref))) <= TOL
    g = capture(step)
    replay_and_check(g, out, ws, eager)


@pytest.mark.parametrize("name", ["qwen1p5b_bf16", "shared_prefix_bf16"])
def test_one_call_decode_step_graph(name):
    """pa_decode_step (slots and new rows in one launch, then attention)
    captured whole: every replay bitwise equal to the eager step, which
    matches the oracle, and the slots and pools left as the oracle writes
    them (rewriting the same rows is idempotent)."""
    w = W.make_workload(name)
    say(f"graph one-call decode step {name}")
    t = W.make_tensors(w, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    B, H, D = t["query"].shape
    ps = PB.pa_decode_partition_size(B, H, w.num_kv_heads, D, w.max_context_len, w.block_size, torch.bfloat16,
                                     context_lens=w.context_lens)
    ws = torch.empty(max(1, PB.pa_decode_workspace_bytes(B, H, D, w.max_context_len, w.block_size, ps)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(t["query"])
    slots = torch.empty(B, dtype=torch.int64, device=DEV)
    kp_raw, vp_raw = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])

    def step():
        PB.pa_decode_step(t["query"], t["key"], t["value"], t["k_pool"], t["v_pool"], bt, lens, w.scale,
                          w.max_context_len, out=out, workspace=ws, slot_out=slots, partition_size=ps)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    O.reshape_and_cache(kp_raw, W.raw_numpy(t["key"]), ref_slots)
    O.reshape_and_cache(vp_raw, W.raw_numpy(t["value"]), ref_slots)
    ref = O.decode_attention(W.raw_numpy(t["query"]), kp_raw, vp_raw, w.block_tables, w.context_lens, w.scale,
                             w.dtype)
    assert float(np.max(np.abs(O.widen(W.raw_numpy(eager), w.dtype) - ref))) <= TOL
    g = capture(step)
    slots.fill_(-5)
    replay_and_check(g, out, ws, eager)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    assert np.array_equal(W.raw_numpy(t["k_pool"]).view(np.uint8), kp_raw.view(np.uint8))
    assert np.array_equal(W.raw_numpy(t["v_pool"]).view(np.uint8), vp_raw.view(np.uint8))


def test_prefill_step_graph():
    pb = W.mixed_varlen_bf16(seed=1)
    w = pb.workload
    say("graph prefill step mixed_varlen_bf16")
    t = W.make_prefill_tensors(pb, 0, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    T, H, D = t["query"].shape
    ps = 256
    ws = torch.empty(max(1, PB.pa_prefill_workspace_bytes(T, H, D, w.max_context_len, w.block_size, ps)),
                     dtype=torch.uint8, device=DEV)
    out = torch.empty_like(t["query"])
    slots = torch.empty(T, dtype=torch.int64, device=DEV)

    def step():
        PB.pa_slot_mapping(bt, lens, w.block_size, query_start_loc=t["query_start_loc"], num_tokens=T, out=slots)
        PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
        PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], bt, lens, t["query_start_loc"], w.scale,
                                pb.max_query_len, w.max_context_len, out=out, workspace=ws, partition_size=ps)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = O.paged_attention(W.raw_numpy(t["query"]), W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"]),
                            w.block_tables, w.context_lens, pb.query_start_loc, w.scale, w.dtype)
    assert float(np.max(np.abs(O.widen(W.raw_numpy(eager), w.dtype) - ref))) <= TOL
    g = capture(step)
    replay_and_check(g, out, ws, eager)
