"""The read-stream probe (include/pagedattn_probe.h) reads exactly the bytes
it is asked to: the XOR of its per-thread accumulators equals the XOR, as
16-byte words, of every run gathered on the CPU from the same buffers."""
import numpy as np
import pytest
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import api
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pad.load_library()


def _xor_runs(buf: np.ndarray, pages, runs, page_stride, run_stride, run_bytes):
    acc = np.zeros(4, np.uint32)
    for pg in pages:
        for r in range(runs):
            o = int(pg) * page_stride + r * run_stride
            acc ^= np.bitwise_xor.reduce(buf[o:o + run_bytes].view(np.uint32).reshape(-1, 4), axis=0)
    return acc


@pytest.mark.parametrize("run_bytes,runs,two", [(4096, 8, True), (1152, 1, False), (8192, 2, True),
                                                (16, 3, False), (2048, 1, True)])
def test_read_probe_reads_the_requested_bytes(run_bytes, runs, two):
    say(f"read probe: run {run_bytes} B, {runs} runs per page, two bases {two}")
    rng = np.random.default_rng(run_bytes + runs)
    run_stride = run_bytes + 16 * int(rng.integers(0, 4))
    page_stride = runs * run_stride + 32
    npages_buf = 300
    size = npages_buf * page_stride + 64
    b0 = rng.integers(0, 2**32, size // 4, dtype=np.uint32).view(np.uint8)
    b1 = rng.integers(0, 2**32, size // 4, dtype=np.uint32).view(np.uint8)
    pages = rng.permutation(npages_buf)[:257].astype(np.int32)
    want = _xor_runs(b0, pages, runs, page_stride, run_stride, run_bytes)
    if two:
        want ^= _xor_runs(b1, pages, runs, page_stride, run_stride, run_bytes)
    g0 = torch.from_numpy(b0.copy()).to(DEV)
    g1 = torch.from_numpy(b1.copy()).to(DEV) if two else None
    sink = torch.full((7 * 1024,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    api.read_probe(sink, g0, torch.from_numpy(pages).to(DEV), runs, page_stride, run_stride, run_bytes,
                   base1=g1)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)
