"""Calls from several host threads on several streams at once.

The library keeps only per-device caches (compute-unit count, resident
workgroups per kernel) behind a lock and otherwise no state, so concurrent
calls on different streams must give exactly the results of the same calls
made one after another.  Four threads, each with its own stream (default
priority), run the whole decode step with the automatic partition choice (the
cached device queries are exercised) on different workloads; every output is
compared bitwise with the sequential run.
"""

import sys
import threading

import pytest
import torch

from paged_kv_cache_size_amd import binding as PB
from paged_kv_cache_size_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def prepare(name, seed):
    w = W.make_workload(name) if name != "custom" else W.custom([1, 700, 33, 4096, 130], 16, 4, 64, "f16",
                                                                 seed=seed)
    t = W.make_tensors(w, seed, DEV)
    bt = torch.from_numpy(w.block_tables).to(DEV)
    lens = torch.from_numpy(w.context_lens).to(DEV)
    return w, t, bt, lens


def step(w, t, bt, lens):
    # a fresh copy of the pools: the write must not see another thread's rows
    kp, vp = t["k_pool"].clone(), t["v_pool"].clone()
    slots = PB.pa_slot_mapping(bt, lens, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], kp, vp, slots)
    return PB.pa_decode_attention(t["query"], kp, vp, bt, lens, w.scale, w.max_context_len)


def test_threads_on_streams_match_sequential():
    names = ["qwen1p5b_bf16", "tiny_f32", "shared_prefix_bf16", "custom"]
    print(f"[gpu-case] concurrent decode on {names}", file=sys.stderr, flush=True)
    cases = [prepare(n, i) for i, n in enumerate(names)]
    torch.cuda.synchronize()
    expect = [step(*c) for c in cases]
    torch.cuda.synchronize()

    results, errors = [None] * len(cases), []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(s):
                outs = [step(*cases[i]) for _ in range(3)]
            s.synchronize()
            results[i] = outs
        except Exception as e:  # reported below, on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, outs in enumerate(results):
        ref = expect[i].view(torch.int32) if expect[i].dtype == torch.float32 else expect[i].view(torch.int16)
        for o in outs:
            got = o.view(torch.int32) if o.dtype == torch.float32 else o.view(torch.int16)
            assert torch.equal(got, ref), names[i]
