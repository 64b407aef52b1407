"""The streaming-read measurement kernel reads every 16-byte vector of its
buffer: a buffer of zeros with the kernel's pattern word planted in one
vector makes exactly the thread that loads it store the pattern."""

import sys

import pytest
import torch

from paged_kv_cache_size_amd import binding as PB

pytestmark = pytest.mark.gpu

PATTERN = 0x5A17C0DE


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    PB.lib()


@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("n_vec", [1, 3, 2048, 4 * 512 * 16384 + 5])
def test_every_vector_is_read(n_vec, nontemporal):
    print(f"[gpu-case] stream read n_vec={n_vec} nt={nontemporal}", file=sys.stderr, flush=True)
    buf = torch.zeros(n_vec, 4, dtype=torch.int32, device="cuda")
    for pos in sorted({0, n_vec // 2, n_vec - 1}):
        buf.zero_()
        buf[pos, 1] = PATTERN
        sink = torch.zeros(1, dtype=torch.int32, device="cuda")
        PB.pa_stream_read(buf, sink, nontemporal=nontemporal)
        torch.cuda.synchronize()
        assert int(sink.item()) == PATTERN, pos
    buf.zero_()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    PB.pa_stream_read(buf, sink, nontemporal=nontemporal)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
