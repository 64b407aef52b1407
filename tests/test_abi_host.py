"""The C ABI without a GPU: symbols, argument checks, workspace sizing.

Every call here fails host-side validation (or is a pure size query), so no
HIP call is reached.
"""

import ctypes
import re
from pathlib import Path

import pytest

from paged_kv_cache_size_amd import binding as B

HEADER = Path(__file__).resolve().parents[1] / "include" / "pa.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(pa_\w+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(B.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for s, key in [(0, "PA_OK"), (1, "INVALID_ARG"), (2, "UNSUPPORTED"), (3, "WORKSPACE"), (4, "HIP")]:
        assert key in B.pa_status_string(s)
    assert "unknown" in B.pa_status_string(99)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def decode(**kw):
    args = dict(out=FAKE, query=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, B=4, H=8, Hkv=2, D=128, bs=16,
                mb=8, maxlen=128, scale=0.088, dtype=B.PA_BF16, ws=None, wsb=0, ps=16)
    args.update(kw)
    a = args
    return B.lib().pa_decode_attention_ex(a["out"], a["query"], a["k"], a["v"], a["bt"], a["lens"], a["B"], a["H"],
                                          a["Hkv"], a["D"], a["bs"], a["mb"], a["maxlen"], a["scale"], a["dtype"],
                                          a["ws"], a["wsb"], a["ps"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), B.PA_ERR_INVALID_ARG),
    (dict(query=None), B.PA_ERR_INVALID_ARG),
    (dict(k=None), B.PA_ERR_INVALID_ARG),
    (dict(bt=None), B.PA_ERR_INVALID_ARG),
    (dict(lens=None), B.PA_ERR_INVALID_ARG),
    (dict(B=-1), B.PA_ERR_INVALID_ARG),
    (dict(H=-1), B.PA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), B.PA_ERR_INVALID_ARG),
    (dict(maxlen=129), B.PA_ERR_INVALID_ARG),     # > mb * bs
    (dict(maxlen=0), B.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.PA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), B.PA_ERR_INVALID_ARG),
    (dict(dtype=7), B.PA_ERR_UNSUPPORTED),
    (dict(D=96), B.PA_ERR_UNSUPPORTED),
    (dict(bs=24, mb=6), B.PA_ERR_UNSUPPORTED),    # not a power of two
    (dict(bs=512, mb=1), B.PA_ERR_UNSUPPORTED),
    (dict(dtype=B.PA_F32, bs=512, mb=1), B.PA_ERR_UNSUPPORTED),
    (dict(dtype=B.PA_F32, bs=32, mb=4), B.PA_ERR_INVALID_ARG),  # fp32 too: partitions hold whole blocks
    (dict(bs=32, mb=4, ps=16), B.PA_ERR_INVALID_ARG),  # partitions hold whole blocks
    (dict(bs=4, mb=32, ps=8), B.PA_ERR_INVALID_ARG),   # and whole 16-token steps
    (dict(bs=1, mb=2048, maxlen=2048, ps=1040), B.PA_ERR_INVALID_ARG),  # small blocks: above 1024 blocks
    (dict(bs=32, mb=129, maxlen=4128, ps=8224), B.PA_ERR_INVALID_ARG),  # above 256 blocks
    (dict(ps=24), B.PA_ERR_INVALID_ARG),          # not a multiple of the block size
    (dict(ps=4112, maxlen=128), B.PA_ERR_INVALID_ARG),  # above 256 blocks
    (dict(ps=-16), B.PA_ERR_INVALID_ARG),
    (dict(ps=16), B.PA_ERR_WORKSPACE),            # 8 partitions need a workspace
    (dict(ps=16, ws=FAKE, wsb=100), B.PA_ERR_WORKSPACE),
])
def test_decode_argument_checks(kw, status):
    assert decode(**kw) == status


def test_empty_batches_enqueue_nothing():
    # no sequence (decode) or no new token (prefill) is a valid call that
    # touches no pointer, null ones included
    lib = B.lib()
    nul = dict(out=None, query=None, k=None, v=FAKE, bt=None, lens=None)
    assert decode(B=0, ps=0, **nul) == B.PA_OK
    assert decode(B=0, ps=16, **nul) == B.PA_OK
    assert lib.pa_decode_partitions(None, None, None, None, None, None, 0, 8, 2, 128, 16, 8, 128, 0.088,
                                    B.PA_BF16, None, 0, 16, None) == B.PA_OK
    assert lib.pa_decode_combine(None, None, 0, 8, 128, 128, 16, B.PA_BF16, None, 0, None) == B.PA_OK
    assert lib.pa_slot_mapping(None, None, None, None, 0, 8, 16, 0, None) == B.PA_OK
    assert prefill(T=0, B=0, out=None, query=None, k=None, bt=None, lens=None, qsl=None) == B.PA_OK
    assert lib.pa_decode_attention_shared_prefix(None, None, None, None, None, None, None, None, None, 0, 0, 0, 8,
                                                 2, 128, 16, 8, 128, 0, 0.088, B.PA_BF16, None, 0,
                                                 None) == B.PA_OK
    # sizes are still checked where the call has work
    assert lib.pa_slot_mapping(None, None, None, None, 0, 8, 16, 5, None) == B.PA_ERR_INVALID_ARG
    assert decode(B=-1, **nul) == B.PA_ERR_INVALID_ARG


def test_workspace_sizes():
    lib = B.lib()
    # explicit partition: B*H*P*(D+2)*4 bytes, none for a single partition
    assert lib.pa_decode_workspace_bytes_ex(4, 8, 128, 128, 16, 16) == 4 * 8 * 8 * 130 * 4
    assert lib.pa_decode_workspace_bytes_ex(4, 8, 128, 128, 16, 128) == 0
    assert lib.pa_decode_workspace_bytes_ex(4, 8, 128, 128, 16, 24) == 0  # invalid
    # automatic: sized for partitions of at least 128 tokens
    assert lib.pa_decode_workspace_bytes(256, 32, 128, 4096, 16) == 256 * 32 * 32 * 130 * 4
    assert lib.pa_decode_workspace_bytes(4, 4, 64, 33, 16) == 0
    assert lib.pa_decode_workspace_bytes(0, 4, 64, 33, 16) == 0
    assert lib.pa_decode_workspace_bytes_ex(4, 8, 128, 128, 16, 16) == B.pa_decode_workspace_bytes(4, 8, 128, 128, 16, 16)
    assert decode(ps=16, ws=FAKE, wsb=4 * 8 * 8 * 130 * 4 - 1) == B.PA_ERR_WORKSPACE


def prefill(**kw):
    args = dict(out=FAKE, query=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, qsl=FAKE, B=4, T=40, mq=16, H=8, Hkv=2,
                D=128, bs=16, mb=8, maxlen=128, scale=0.088, dtype=B.PA_BF16, ws=None, wsb=0, ps=128)
    args.update(kw)
    a = args
    return B.lib().pa_prefill_attention(a["out"], a["query"], a["k"], a["v"], a["bt"], a["lens"], a["qsl"], a["B"],
                                        a["T"], a["mq"], a["H"], a["Hkv"], a["D"], a["bs"], a["mb"], a["maxlen"],
                                        a["scale"], a["dtype"], a["ws"], a["wsb"], a["ps"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(qsl=None), B.PA_ERR_INVALID_ARG),
    (dict(out=None), B.PA_ERR_INVALID_ARG),
    (dict(T=-1), B.PA_ERR_INVALID_ARG),
    (dict(mq=0), B.PA_ERR_INVALID_ARG),
    (dict(mq=41), B.PA_ERR_INVALID_ARG),          # longer than all rows
    (dict(mq=40, maxlen=32, mb=2), B.PA_ERR_INVALID_ARG),  # more new tokens than context
    (dict(H=6, Hkv=4), B.PA_ERR_INVALID_ARG),
    (dict(maxlen=129), B.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), B.PA_ERR_INVALID_ARG),
    (dict(dtype=B.PA_F32, bs=32, mb=4, ps=16), B.PA_ERR_INVALID_ARG),  # fp32 rows: whole blocks per partition
    (dict(dtype=B.PA_F32, bs=512, mb=1), B.PA_ERR_UNSUPPORTED),
    (dict(dtype=B.PA_F32, ps=16), B.PA_ERR_WORKSPACE),  # fp32 is accepted: 8 partitions need a workspace
    (dict(dtype=B.PA_F32, ps=24), B.PA_ERR_INVALID_ARG),
    (dict(D=96), B.PA_ERR_UNSUPPORTED),
    (dict(bs=24, mb=6), B.PA_ERR_UNSUPPORTED),    # block sizes are powers of two
    (dict(bs=512, mb=1), B.PA_ERR_UNSUPPORTED),
    (dict(bs=32, mb=4, ps=16), B.PA_ERR_INVALID_ARG),  # partitions hold whole blocks
    (dict(bs=4, mb=32, ps=8), B.PA_ERR_INVALID_ARG),   # and whole 16-token steps
    (dict(bs=1, mb=2048, maxlen=2048, ps=1040), B.PA_ERR_INVALID_ARG),  # small blocks: at most 1024
    (dict(bs=32, mb=129, maxlen=4128, ps=8224), B.PA_ERR_INVALID_ARG),  # at most 256 blocks
    (dict(ps=24), B.PA_ERR_INVALID_ARG),
    (dict(ps=4112), B.PA_ERR_INVALID_ARG),
    (dict(ps=16), B.PA_ERR_WORKSPACE),            # 8 partitions need a workspace
    (dict(ps=16, ws=FAKE, wsb=40 * 8 * 8 * 130 * 4 - 1), B.PA_ERR_WORKSPACE),
])
def test_prefill_argument_checks(kw, status):
    assert prefill(**kw) == status


def test_shared_prefix_block_sizes():
    # block sizes are powers of two (the passes split keys at 1024 tokens,
    # which every supported block size holds in one partition)
    lib = B.lib()
    f = lib.pa_decode_attention_shared_prefix
    for bs in (24, 512):
        mb = -(-4096 // bs)
        assert f(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 2, 8, 2, 128, bs, mb, 4096, 0,
                 0.088, B.PA_BF16, FAKE, 1 << 30, None) == B.PA_ERR_UNSUPPORTED


def test_prefill_workspace_sizes():
    lib = B.lib()
    # explicit partition: T*H*P*(D+2)*4 bytes, none for a single partition
    assert lib.pa_prefill_workspace_bytes(40, 8, 128, 128, 16, 16) == 40 * 8 * 8 * 130 * 4
    assert lib.pa_prefill_workspace_bytes(40, 8, 128, 128, 16, 128) == 0
    assert lib.pa_prefill_workspace_bytes(40, 8, 128, 128, 16, 24) == 0
    assert lib.pa_prefill_workspace_bytes(40, 8, 128, 128, 4, 8) == 0  # not whole 16-token steps
    assert lib.pa_prefill_workspace_bytes(40, 8, 128, 128, 4, 16) == 40 * 8 * 8 * 130 * 4
    # automatic: at most one partition per 128 tokens, partials within 256 MiB
    assert lib.pa_prefill_workspace_bytes(40, 8, 128, 4096, 16, 0) == 40 * 8 * 32 * 130 * 4
    assert lib.pa_prefill_workspace_bytes(8192, 32, 128, 4096, 16, 0) == 0  # one split alone exceeds the cap
    assert 0 < lib.pa_prefill_workspace_bytes(512, 32, 128, 4096, 16, 0) <= 256 << 20
    # a context beyond one 256-block slice always needs partitions
    assert lib.pa_prefill_workspace_bytes(1 << 20, 32, 128, 8192, 16, 0) == (1 << 20) * 32 * 2 * 130 * 4


def test_reshape_argument_checks():
    lib = B.lib()
    f = lib.pa_reshape_and_cache
    ok = (FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 64, 16, 10, B.PA_F32, None)
    def call(**kw):
        a = list(ok)
        names = ["key", "value", "kp", "vp", "slots", "n", "hkv", "d", "bs", "nb", "dtype", "stream"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)
    assert call(key=None) == B.PA_ERR_INVALID_ARG
    assert call(slots=None) == B.PA_ERR_INVALID_ARG
    assert call(kp=None) == B.PA_ERR_INVALID_ARG
    assert call(n=-1) == B.PA_ERR_INVALID_ARG
    assert call(hkv=0) == B.PA_ERR_INVALID_ARG
    assert call(nb=0) == B.PA_ERR_INVALID_ARG
    assert call(dtype=9) == B.PA_ERR_UNSUPPORTED
    assert call(n=0, key=None, value=None, slots=None) == B.PA_OK  # nothing to write


def test_slot_mapping_argument_checks():
    f = B.lib().pa_slot_mapping
    assert f(None, FAKE, FAKE, None, 4, 8, 16, 4, None) == B.PA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, None, 4, 8, 16, 5, None) == B.PA_ERR_INVALID_ARG  # decode needs num_tokens == num_seqs
    assert f(FAKE, FAKE, FAKE, None, -1, 8, 16, -1, None) == B.PA_ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 4, 8, 0, 9, None) == B.PA_ERR_INVALID_ARG


def test_stream_read_argument_checks():
    f = B.lib().pa_stream_read
    assert f(None, 1024, FAKE, 0, None) == B.PA_ERR_INVALID_ARG
    assert f(FAKE, 1024, None, 0, None) == B.PA_ERR_INVALID_ARG
    assert f(FAKE, 0, FAKE, 0, None) == B.PA_ERR_INVALID_ARG
    assert f(FAKE, 1000, FAKE, 1, None) == B.PA_ERR_INVALID_ARG  # not a whole number of 16-byte vectors
    assert f(ctypes.c_void_p(0x1008), 1024, FAKE, 0, None) == B.PA_ERR_INVALID_ARG  # misaligned


def decode_layout(layout, **kw):
    a = dict(out=FAKE, query=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, B=4, H=8, Hkv=2, D=128, bs=16,
             mb=8, maxlen=128, scale=0.088, dtype=B.PA_BF16, ws=None, wsb=0, ps=128)
    a.update(kw)
    return B.lib().pa_decode_attention_layout(a["out"], a["query"], a["k"], a["v"], a["bt"], a["lens"], a["B"],
                                              a["H"], a["Hkv"], a["D"], a["bs"], a["mb"], a["maxlen"], a["scale"],
                                              a["dtype"], a["ws"], a["wsb"], a["ps"], layout, None)


def test_layout_argument_checks():
    # the fused pool is one pointer: a V pool alongside it is an error, and
    # the split layout still needs both
    assert decode_layout(B.PA_KV_FUSED) == B.PA_ERR_INVALID_ARG
    assert decode_layout(B.PA_KV_SPLIT, v=None) == B.PA_ERR_INVALID_ARG
    assert decode_layout(2, v=None) == B.PA_ERR_INVALID_ARG
    assert decode_layout(B.PA_KV_FUSED, v=None, dtype=7) == B.PA_ERR_UNSUPPORTED
    assert decode_layout(B.PA_KV_FUSED, v=None, k=None) == B.PA_ERR_INVALID_ARG
    assert decode_layout(B.PA_KV_FUSED, v=None, ps=16) == B.PA_ERR_WORKSPACE  # checks reached the plan
    # a block over 2 GiB cannot be addressed with 32-bit offsets
    assert decode_layout(B.PA_KV_FUSED, v=None, Hkv=1 << 20, H=1 << 20, bs=256, mb=1, maxlen=256,
                         ps=256) == B.PA_ERR_INVALID_ARG
    lib = B.lib()
    rs = lib.pa_reshape_and_cache_layout
    assert rs(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 2, 64, 16, 10, B.PA_BF16, B.PA_KV_FUSED, None) == B.PA_ERR_INVALID_ARG
    assert rs(FAKE, FAKE, FAKE, None, FAKE, 4, 2, 64, 16, 10, B.PA_BF16, B.PA_KV_SPLIT, None) == B.PA_ERR_INVALID_ARG
    assert rs(FAKE, FAKE, FAKE, None, FAKE, 0, 2, 64, 16, 10, B.PA_BF16, B.PA_KV_FUSED, None) == B.PA_OK
    assert lib.pa_reshape_and_cache(FAKE, FAKE, FAKE, None, FAKE, 0, 2, 64, 16, 10, B.PA_BF16,
                                    None) == B.PA_ERR_INVALID_ARG
    cv = lib.pa_convert_blocks
    ok = [FAKE, None, B.PA_KV_FUSED, 10, FAKE, FAKE, B.PA_KV_SPLIT, 10, FAKE, FAKE, 3, 16, 2, 64, B.PA_BF16, None]

    def conv(**kw):
        a = list(ok)
        names = ["dk", "dv", "dl", "dn", "sk", "sv", "sl", "sn", "src", "dst", "n", "bs", "hkv", "d", "dt", "st"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return cv(*a)
    assert conv(n=0) == B.PA_OK
    assert conv(dv=FAKE) == B.PA_ERR_INVALID_ARG        # fused destination with a V pool
    assert conv(sv=None) == B.PA_ERR_INVALID_ARG        # split source without one
    assert conv(dl=5) == B.PA_ERR_INVALID_ARG
    assert conv(src=None) == B.PA_ERR_INVALID_ARG
    assert conv(n=-1) == B.PA_ERR_INVALID_ARG
    assert conv(dn=0) == B.PA_ERR_INVALID_ARG
    assert conv(dt=9) == B.PA_ERR_UNSUPPORTED
    pf = lib.pa_prefill_attention_layout
    assert pf(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 8, 4, 8, 2, 128, 16, 8, 128, 0.088, B.PA_BF16, None, 0, 0,
              B.PA_KV_FUSED, None) == B.PA_ERR_INVALID_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_LIB", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        B.lib()


def noalloc(**kw):
    args = dict(out=FAKE, query=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, B=4, H=8, Hkv=2, D=128, bs=16,
                mb=8, maxlen=128, scale=0.088, dtype=B.PA_BF16, ps=16)
    args.update(kw)
    a = args
    return B.lib().pa_decode_attention_noalloc(a["out"], a["query"], a["k"], a["v"], a["bt"], a["lens"], a["B"],
                                               a["H"], a["Hkv"], a["D"], a["bs"], a["mb"], a["maxlen"], a["scale"],
                                               a["dtype"], a["ps"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), B.PA_ERR_INVALID_ARG),
    (dict(v=None), B.PA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), B.PA_ERR_INVALID_ARG),
    (dict(maxlen=129), B.PA_ERR_INVALID_ARG),
    (dict(ps=24), B.PA_ERR_INVALID_ARG),
    (dict(D=96), B.PA_ERR_UNSUPPORTED),
    # 4096 x 64 heads x 256 partitions of partials: far beyond the static buffer
    (dict(B=4096, H=64, Hkv=8, mb=256, maxlen=4096, ps=16), B.PA_ERR_WORKSPACE),
])
def test_noalloc_argument_checks(kw, status):
    # every case fails on the host, before the buffer's address is looked up
    assert noalloc(**kw) == status


def test_noalloc_scratch_limit_is_the_header_constant():
    text = HEADER.read_text()
    m = re.search(r"#define PA_DECODE_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    limit = int(m.group(1)) << int(m.group(2))
    # the largest batch whose partials fit the static buffer, by the workspace
    # query; one sequence more is refused on the host as WORKSPACE
    per_seq = B.lib().pa_decode_workspace_bytes_ex(1, 64, 128, 4096, 16, 16)
    fit = limit // per_seq
    assert B.lib().pa_decode_workspace_bytes_ex(fit, 64, 128, 4096, 16, 16) <= limit
    assert B.lib().pa_decode_workspace_bytes_ex(fit + 1, 64, 128, 4096, 16, 16) > limit
    assert noalloc(B=fit + 1, H=64, Hkv=8, mb=256, maxlen=4096, ps=16) == B.PA_ERR_WORKSPACE


def test_oversized_grid_is_an_argument_error():
    # 2^25 new tokens of 8 KV heads x 128 bf16 dims: one workgroup of 128
    # threads per token row is 2^32 work-items in the grid's x dimension, one
    # more than the dispatch can count; refused on the host, nothing launched
    n = 1 << 25
    rc = B.lib().pa_reshape_and_cache(FAKE, FAKE, FAKE, FAKE, FAKE, n, 8, 128, 16, 1 << 22, B.PA_BF16, None)
    assert rc == B.PA_ERR_INVALID_ARG


def write_new(**kw):
    args = dict(key=FAKE, value=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, slots=None, B=4, Hkv=2, D=128, bs=16,
                mb=8, nb=64, dtype=B.PA_BF16, layout=B.PA_KV_SPLIT)
    args.update(kw)
    a = args
    return B.lib().pa_write_new_tokens(a["key"], a["value"], a["k"], a["v"], a["bt"], a["lens"], a["slots"], a["B"],
                                       a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"], a["dtype"], a["layout"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(key=None), B.PA_ERR_INVALID_ARG),
    (dict(value=None), B.PA_ERR_INVALID_ARG),
    (dict(k=None), B.PA_ERR_INVALID_ARG),
    (dict(v=None), B.PA_ERR_INVALID_ARG),
    (dict(bt=None), B.PA_ERR_INVALID_ARG),
    (dict(lens=None), B.PA_ERR_INVALID_ARG),
    (dict(B=-1), B.PA_ERR_INVALID_ARG),
    (dict(Hkv=0), B.PA_ERR_INVALID_ARG),
    (dict(D=0), B.PA_ERR_INVALID_ARG),
    (dict(bs=0), B.PA_ERR_INVALID_ARG),
    (dict(mb=0), B.PA_ERR_INVALID_ARG),
    (dict(nb=0), B.PA_ERR_INVALID_ARG),
    (dict(dtype=7), B.PA_ERR_UNSUPPORTED),
    (dict(layout=5), B.PA_ERR_INVALID_ARG),
    (dict(B=0, key=None, value=None, k=None, v=None, bt=None, lens=None), B.PA_OK),  # an empty batch
])
def test_write_new_tokens_argument_checks(kw, status):
    assert write_new(**kw) == status


def step(**kw):
    args = dict(out=FAKE, query=FAKE, key=FAKE, value=FAKE, k=FAKE, v=FAKE, bt=FAKE, lens=FAKE, slots=None, B=4, H=8,
                Hkv=2, D=128, bs=16, mb=8, nb=64, maxlen=128, scale=0.088, dtype=B.PA_BF16, ws=None, wsb=0, ps=16,
                layout=B.PA_KV_SPLIT)
    args.update(kw)
    a = args
    return B.lib().pa_decode_step(a["out"], a["query"], a["key"], a["value"], a["k"], a["v"], a["bt"], a["lens"],
                                  a["slots"], a["B"], a["H"], a["Hkv"], a["D"], a["bs"], a["mb"], a["nb"],
                                  a["maxlen"], a["scale"], a["dtype"], a["ws"], a["wsb"], a["ps"], a["layout"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(out=None), B.PA_ERR_INVALID_ARG),
    (dict(query=None), B.PA_ERR_INVALID_ARG),
    (dict(key=None), B.PA_ERR_INVALID_ARG),
    (dict(value=None), B.PA_ERR_INVALID_ARG),
    (dict(k=None), B.PA_ERR_INVALID_ARG),
    (dict(v=None), B.PA_ERR_INVALID_ARG),
    (dict(nb=0), B.PA_ERR_INVALID_ARG),
    (dict(H=6, Hkv=4), B.PA_ERR_INVALID_ARG),
    (dict(maxlen=129), B.PA_ERR_INVALID_ARG),           # beyond max_blocks_per_seq * block_size
    (dict(scale=float("nan")), B.PA_ERR_INVALID_ARG),
    (dict(D=96), B.PA_ERR_UNSUPPORTED),
    (dict(dtype=7), B.PA_ERR_UNSUPPORTED),
    (dict(layout=5), B.PA_ERR_INVALID_ARG),
    (dict(ps=24), B.PA_ERR_INVALID_ARG),                # not a whole number of 16-token steps
    (dict(ps=64, maxlen=128), B.PA_ERR_WORKSPACE),      # two partitions and no workspace
    (dict(ps=0, maxlen=128 * 8, mb=64), B.PA_ERR_WORKSPACE),  # the library's choice needs the documented bound
    (dict(B=0, out=None, query=None, key=None, value=None, k=None, v=None, bt=None, lens=None), B.PA_OK),
])
def test_decode_step_argument_checks(kw, status):
    """Every check runs before anything is enqueued (no HIP call is reached)."""
    assert step(**kw) == status
