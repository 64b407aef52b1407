"""GPU parity on batches whose launches pass 65,535 workgroups.

Many short sequences (a decode step of 70,000 sequences, a prefill step of
40,000 sequences bringing 4 tokens each) put one workgroup per (sequence, KV
head unit) on the grid's first axis, beyond the 65,535 that the second and
third axes allow.  Checked: the slots and the written pools bit-exact
against the oracle; every output row bitwise equal to the same sequences
launched in chunks of at most 2,000 (the same partition size, so the same
arithmetic); sampled sequences within the tolerance of the float64 oracle.
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
TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def sample(n, step):
    return sorted(set([0, 1, n - 1] + list(range(7, n, step))))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_70000_sequences(dtype):
    B = 70_000
    lens = np.random.default_rng(21).integers(1, 49, B)
    w = W.custom(lens.tolist(), 4, 1, 64, dtype, seed=21, name=f"many_seqs_{dtype}")
    say(f"decode of {B} sequences (one workgroup each), contexts 1..48, H 4/1, D 64, {dtype}")
    t = W.make_tensors(w, seed=21, device=DEV)
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    bt = torch.from_numpy(w.block_tables).to(DEV)
    ln = torch.from_numpy(w.context_lens).to(DEV)
    slots = PB.pa_slot_mapping(bt, ln, w.block_size)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    ps = 64  # one partition per sequence
    out = PB.pa_decode_attention(t["query"], t["k_pool"], t["v_pool"], bt, ln, w.scale, w.max_context_len,
                                 partition_size=ps)
    torch.cuda.synchronize()

    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    O.reshape_and_cache(kp, W.raw_numpy(t["key"]), ref_slots)
    O.reshape_and_cache(vp, W.raw_numpy(t["value"]), ref_slots)
    assert np.array_equal(W.raw_numpy(t["k_pool"]).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(W.raw_numpy(t["v_pool"]).view(np.uint8), vp.view(np.uint8))

    for c0 in range(0, B, 2000):
        c1 = min(B, c0 + 2000)
        part = PB.pa_decode_attention(t["query"][c0:c1].contiguous(), t["k_pool"], t["v_pool"],
                                      bt[c0:c1].contiguous(), ln[c0:c1].contiguous(), w.scale,
                                      int(lens[c0:c1].max()), partition_size=ps)
        assert torch.equal(bits(part), bits(out[c0:c1])), c0

    sel = sample(B, 97)
    ref = O.decode_attention(W.raw_numpy(t["query"])[sel], kp, vp, w.block_tables[sel], w.context_lens[sel],
                             w.scale, w.dtype)
    got = O.widen(W.raw_numpy(out), w.dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got[sel] - ref)))
    say(f"  {len(sel)} sampled sequences: max abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_40000_sequences(dtype):
    B, n_new = 40_000, 4
    lens = np.random.default_rng(22).integers(n_new, 65, B)
    pb = W.prefill_batch(lens.tolist(), [n_new] * B, 8, 2, 64, dtype, seed=22, name=f"many_prefill_{dtype}")
    w = pb.workload
    say(f"prefill of {B} sequences x {n_new} new tokens ({pb.num_tokens} rows), contexts {n_new}..64, "
        f"H 8/2, D 64, {dtype}")
    t = W.make_prefill_tensors(pb, seed=22, device=DEV)
    kp, vp = W.raw_numpy(t["k_pool"]), W.raw_numpy(t["v_pool"])
    bt = torch.from_numpy(w.block_tables).to(DEV)
    ln = torch.from_numpy(w.context_lens).to(DEV)
    qsl = t["query_start_loc"]
    slots = PB.pa_slot_mapping(bt, ln, w.block_size, query_start_loc=qsl, num_tokens=pb.num_tokens)
    PB.pa_reshape_and_cache(t["key"], t["value"], t["k_pool"], t["v_pool"], slots)
    ps = 64
    out = PB.pa_prefill_attention(t["query"], t["k_pool"], t["v_pool"], bt, ln, qsl, w.scale, n_new,
                                  w.max_context_len, partition_size=ps)
    torch.cuda.synchronize()

    ref_slots = O.slot_mapping(w.block_tables, w.context_lens, w.block_size, query_lens=pb.query_lens)
    assert np.array_equal(slots.cpu().numpy(), ref_slots)
    O.reshape_and_cache(kp, W.raw_numpy(t["key"]), ref_slots)
    O.reshape_and_cache(vp, W.raw_numpy(t["value"]), ref_slots)
    assert np.array_equal(W.raw_numpy(t["k_pool"]).view(np.uint8), kp.view(np.uint8))
    assert np.array_equal(W.raw_numpy(t["v_pool"]).view(np.uint8), vp.view(np.uint8))

    qsl_h = pb.query_start_loc.astype(np.int64)
    for c0 in range(0, B, 2000):
        c1 = min(B, c0 + 2000)
        r0, r1 = int(qsl_h[c0]), int(qsl_h[c1])
        sub_qsl = torch.from_numpy((qsl_h[c0:c1 + 1] - r0).astype(np.int32)).to(DEV)
        part = PB.pa_prefill_attention(t["query"][r0:r1].contiguous(), t["k_pool"], t["v_pool"],
                                       bt[c0:c1].contiguous(), ln[c0:c1].contiguous(), sub_qsl, w.scale, n_new,
                                       int(lens[c0:c1].max()), partition_size=ps)
        assert torch.equal(bits(part), bits(out[r0:r1])), c0

    sel = sample(B, 211)
    rows = np.concatenate([np.arange(qsl_h[b], qsl_h[b + 1]) for b in sel])
    sel_qsl = np.concatenate([[0], np.cumsum([int(pb.query_lens[b]) for b in sel])])
    ref = O.paged_attention(W.raw_numpy(t["query"])[rows], kp, vp, w.block_tables[sel], w.context_lens[sel],
                            sel_qsl, w.scale, w.dtype)
    got = O.widen(W.raw_numpy(out), w.dtype)
    assert np.isfinite(got).all()
    err = float(np.max(np.abs(got[rows] - ref)))
    say(f"  {len(sel)} sampled sequences: max abs err {err:.3e} (tol {TOL[dtype]})")
    assert err <= TOL[dtype]
