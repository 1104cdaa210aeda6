"""Decode steps captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, never synchronises and reads every length,
split count and page id on the device, so one captured step serves any
inputs of the captured shapes. Each test captures a whole step (split
counts, page list, phase 1, phase 2) on one set of buffers, then replays it
several times with new query values and new lengths written in place,
eager torch work and synchronisations in between, and compares every
replay bit for bit with the same step run eagerly on a second set of
buffers (the kernels have no atomics: equal inputs give equal bits).
"""
import pytest
import torch

from paged_attention_decode_tables_amd import workloads
import paged_attention_decode_tables_amd as pad

pytestmark = pytest.mark.gpu
DEV = "cuda"


class Buffers:
    """Device inputs shared by both runs, and one set of outputs per run."""

    def __init__(self, w, *, max_splits=None, balanced=0, csr=False):
        self.w, self.g = w, w.to(DEV)
        self.balanced = balanced
        self.partition = 0 if balanced else w.partition_size
        R, H, Dv = w.num_seqs * w.num_group, w.num_heads, w.v_head_size
        if max_splits is not None:
            self.max_parts = max_splits
        elif balanced:
            self.max_parts = max(2, -(-w.max_seq_len // 256))
        else:
            self.max_parts = -(-w.max_seq_len // w.partition_size)
        self.max_splits = max_splits
        self.indptr = None
        if csr:
            cu = torch.zeros(w.num_seqs + 1, dtype=torch.int32)
            nblk = [(max(int(L), 0) + w.block_size - 1) // w.block_size for L in w.seq_lens]
            cu[1:] = torch.cumsum(torch.tensor(nblk, dtype=torch.int32), 0)
            self.indptr = cu.to(DEV)
            self.nflat = max(int(cu[-1]), 1)
        self.outs = []
        for _ in range(2):
            o = dict(tmp=torch.empty((R, H, self.max_parts, Dv), dtype=w.query.dtype, device=DEV),
                     ml=torch.empty((R, H, self.max_parts), device=DEV),
                     es=torch.empty((R, H, self.max_parts), device=DEV),
                     out=torch.empty((R, H, Dv), dtype=torch.float32, device=DEV),
                     ns=torch.empty(R, dtype=torch.int32, device=DEV) if max_splits is not None else None,
                     flat=torch.empty(self.nflat, dtype=torch.int32, device=DEV) if csr else None)
            self.outs.append(o)

    def step(self, k):
        """One decode step on output set k, on the current stream."""
        w, g, o = self.w, self.g, self.outs[k]
        if o["ns"] is not None:
            pad.num_kv_splits(o["ns"], g.seq_lens, w.num_group, w.num_heads, w.num_kv_heads,
                              self.max_splits, 256)
        bt = g.block_tables
        if o["flat"] is not None:
            pad.build_page_indices(o["flat"], g.block_tables, self.indptr)
            bt = o["flat"]
        pad.paged_attn_decode(o["tmp"], o["es"], o["ml"], g.query, g.key_cache, g.value_cache, bt,
                              g.seq_lens, w.scale, w.max_seq_len, partition_size=self.partition,
                              num_splits=o["ns"], kv_indptr=self.indptr, num_workers=self.balanced,
                              alibi_slopes=g.alibi_slopes, k_scale=w.k_scale, v_scale=w.v_scale,
                              num_group=w.num_group)
        pad.paged_attn_reduce(o["out"], o["tmp"], o["es"], o["ml"], g.seq_lens,
                              partition_size=self.partition, num_splits=o["ns"], num_group=w.num_group)


def _replays(b, new_lens):
    """Capture b.step(1); replay it once per entry of new_lens (None: the
    captured lengths) after writing new query values, and compare with the
    eager step b.step(0) on the same inputs."""
    pad.load_library()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture
        b.step(1)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.step(1)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(99)
    live = b.w.seq_lens.clone()
    for i, lens in enumerate(new_lens):
        q = torch.randn(b.g.query.shape, generator=gen).to(b.g.query.dtype)
        b.g.query.copy_(q.to(DEV))
        if lens is not None:
            live = torch.as_tensor(lens, dtype=torch.int32)
            b.g.seq_lens.copy_(live.to(DEV))
        # eager work between replays
        junk = torch.randn(1 << 20, device=DEV)
        junk.mul_(2.0).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        b.step(0)
        torch.cuda.synchronize()
        got, want = b.outs[1]["out"].cpu(), b.outs[0]["out"].cpu()
        assert torch.isfinite(want).all(), f"replay {i}: eager output not finite"
        assert torch.equal(got, want), f"replay {i}: max diff {(got - want).abs().max().item()}"
        for key in ("ml", "es"):
            assert torch.equal(b.outs[1][key].cpu(), b.outs[0][key].cpu()), f"replay {i}: {key}"
        if b.outs[0]["ns"] is not None:
            assert torch.equal(b.outs[1]["ns"].cpu(), b.outs[0]["ns"].cpu())
    del graph


def test_graph_grouped_heads_fixed_splits():
    """Matrix-core kernel, fixed 512-token splits, runs of splits."""
    w = workloads.custom(seed=11, seq_lens=[1700, 33, 1300, 512], num_heads=16, num_kv_heads=2,
                         head_size=128, block_size=16, dtype="bf16")
    _replays(Buffers(w), [None, [900, 1, 1700, 0], [1700, 1700, 64, 5]])


def test_graph_grouped_heads_split_counts():
    """Matrix-core persistent workers behind the split-count heuristic."""
    w = workloads.custom(seed=12, seq_lens=[3000, 70, 1200, 9, 2500], num_heads=32, num_kv_heads=8,
                         head_size=128, block_size=32, dtype="bf16")
    _replays(Buffers(w, max_splits=16), [None, [100, 3000, 7, 2900, 1]])


def test_graph_vector_kernel():
    """One-column MHA on the vector kernel."""
    w = workloads.custom(seed=13, seq_lens=[1000, 2000, 17], num_heads=4, num_kv_heads=4,
                         head_size=128, block_size=16, dtype="f16")
    _replays(Buffers(w), [None, [2000, 3, 1500]])


def test_graph_latent_rows_balanced():
    """Latent-row kernel, balanced splits over a CSR page list."""
    w = workloads.mla_custom(seed=14, seq_lens=[1500, 300, 900, 2048], num_heads=128)
    _replays(Buffers(w, balanced=8, csr=True), [None, [1500, 1, 900, 2000], [10, 300, 20, 2048]])
