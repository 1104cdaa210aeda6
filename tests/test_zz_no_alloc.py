"""paged_attn_decode_static (the entry point that allocates nothing: its
split partials live in the library's own device buffer) against
paged_attn_decode + paged_attn_reduce with caller workspaces, through the C
ABI. Each case makes two calls in a row, the second on a smaller input, so a
stale partial left in the shared buffer by the first call would show. The
results must be bit-identical (the same kernels run in the same launch
configuration) and within the oracle tolerance.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import workloads
from gpu_util import DEV, check_output, max_parts_for, say, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pad.load_library()


def _csr(w):
    g = w.to(DEV)
    cu = torch.zeros(w.num_seqs + 1, dtype=torch.int32)
    nblk = [(max(int(L), 0) + w.block_size - 1) // w.block_size for L in w.seq_lens]
    cu[1:] = torch.cumsum(torch.tensor(nblk, dtype=torch.int32), 0)
    indptr = cu.to(DEV)
    flat = torch.full((max(int(cu[-1]), 1),), -1, dtype=torch.int32, device=DEV)
    pad.build_page_indices(flat, g.block_tables, indptr)
    return flat, indptr


def _both(w, *, max_parts, partition_size=512, num_splits=None, csr=False, workers=0,
          out_dtype=torch.float32, tmp_dtype=torch.float32):
    """(static-scratch output, workspace-path output) on the same inputs."""
    g = w.to(DEV)
    bt, indptr = _csr(w) if csr else (g.block_tables, None)
    ns = None if num_splits is None else torch.as_tensor(num_splits, dtype=torch.int32, device=DEV)
    R = w.num_seqs * w.num_group
    kw = dict(partition_size=partition_size, num_splits=ns, kv_indptr=indptr, num_workers=workers,
              alibi_slopes=g.alibi_slopes, k_scale=w.k_scale, v_scale=w.v_scale,
              num_group=w.num_group)
    out_s = torch.full((R, w.num_heads, w.v_head_size), float("nan"), dtype=out_dtype, device=DEV)
    pad.paged_attn_decode_static(out_s, g.query, g.key_cache, g.value_cache, bt, g.seq_lens, w.scale,
                                 w.max_seq_len, max_num_parts=max_parts, tmp_dtype=tmp_dtype, **kw)
    tmp, ml, es = workspace(w, max_parts, tmp_dtype=tmp_dtype)
    pad.paged_attn_decode(tmp, es, ml, g.query, g.key_cache, g.value_cache, bt, g.seq_lens, w.scale,
                          w.max_seq_len, **kw)
    out_w = torch.full_like(out_s, float("nan"))
    pad.paged_attn_reduce(out_w, tmp, es, ml, g.seq_lens, partition_size=partition_size,
                          num_splits=ns, num_group=w.num_group)
    torch.cuda.synchronize()
    return out_s.cpu(), out_w.cpu()


def _check_pair(w, orc, out_s, out_w, tmp=None):
    assert torch.isfinite(out_s).all()
    assert torch.equal(out_s, out_w)
    check_output(w.expanded() if w.num_group > 1 else w, orc, out_s, tmp=tmp)


def test_static_fixed_splits_grouped_heads(orc):
    """Grouped-head matrix-core kernel, fixed 512-token splits: a long batch,
    then a short one (fewer rows, fewer splits) in the same buffer."""
    big = workloads.custom(seed=701, seq_lens=[5000, 1, 3000, 777, 4096, 12], num_heads=32,
                           num_kv_heads=4, head_size=128, block_size=16, dtype="bf16", poison=True)
    small = workloads.custom(seed=702, seq_lens=[700, 65], num_heads=32, num_kv_heads=4,
                             head_size=128, block_size=16, dtype="bf16", poison=True)
    for w in (big, small):
        say(f"static scratch: grouped heads, {w.num_seqs} seqs, max len {w.max_seq_len}")
        out_s, out_w = _both(w, max_parts=max_parts_for(w, 512))
        _check_pair(w, orc, out_s, out_w)


def test_static_split_counts_and_vector_kernel(orc):
    """Per-sequence split counts (persistent workers), then the vector
    kernel (fp32) on a smaller input, then query groups."""
    w1 = workloads.custom(seed=703, seq_lens=[9000, 33, 2500, 1, 6000], num_heads=16,
                          num_kv_heads=2, head_size=128, block_size=32, dtype="f16", poison=True)
    ns = np.array([9, 1, 3, 1, 7], np.int32)
    say("static scratch: split counts")
    out_s, out_w = _both(w1, max_parts=12, num_splits=ns)
    _check_pair(w1, orc, out_s, out_w)
    w2 = workloads.custom(seed=704, seq_lens=[300, 45], num_heads=4, num_kv_heads=2, head_size=64,
                          block_size=8, dtype="f32", poison=True)
    say("static scratch: vector kernel, fp32")
    out_s, out_w = _both(w2, max_parts=max_parts_for(w2, 64), partition_size=64)
    _check_pair(w2, orc, out_s, out_w)
    w3 = workloads.custom(seed=705, seq_lens=[1200, 9], num_heads=16, num_kv_heads=2,
                          head_size=128, block_size=16, dtype="bf16", num_group=2, poison=True)
    say("static scratch: query groups")
    out_s, out_w = _both(w3, max_parts=max_parts_for(w3, 512))
    _check_pair(w3, orc, out_s, out_w)


def test_static_latent_rows_balanced(orc):
    """The latent-row kernel with balanced splits, then a smaller batch with
    fixed splits and a bf16 output."""
    w1 = workloads.mla_custom(seed=706, seq_lens=[3000, 1, 1500, 640], num_heads=128, poison=True)
    say("static scratch: latent rows, balanced")
    out_s, out_w = _both(w1, max_parts=8, partition_size=0, csr=True, workers=16)
    _check_pair(w1, orc, out_s, out_w)
    w2 = workloads.mla_custom(seed=707, seq_lens=[200, 70], num_heads=128, poison=True)
    say("static scratch: latent rows, fixed, bf16 output")
    out_s, out_w = _both(w2, max_parts=1, csr=True, out_dtype=torch.bfloat16)
    assert torch.equal(out_s, out_w)
    check_output(w2, orc, out_s)


def test_static_16bit_partials(orc):
    """Split outputs in bf16 (then f16, on a smaller batch) in the library's
    buffer: bit-identical to the workspace path with the same element type."""
    for w, tdt, kw in (
            (workloads.mla_custom(seed=708, seq_lens=[2500, 3, 900], num_heads=128, poison=True),
             torch.bfloat16, dict(max_parts=8, partition_size=0, csr=True, workers=12)),
            (workloads.custom(seed=709, seq_lens=[1500, 7], num_heads=16, num_kv_heads=2, head_size=128,
                              block_size=16, dtype="f16", poison=True),
             torch.float16, dict(max_parts=3))):
        say(f"static scratch: {tdt} partials, {w.num_seqs} seqs")
        out_s, out_w = _both(w, tmp_dtype=tdt, **kw)
        assert torch.isfinite(out_s).all() and torch.equal(out_s, out_w)
        # bound: the 16-bit rounding of every stored value (at most |v| <= max|V|)
        bound = np.abs(w.value_cache.float().numpy()).max()
        check_output(w, orc, out_s, tmp=torch.full((w.num_seqs, w.num_heads, 1, 1), float(bound), dtype=tdt))


def test_static_rejects_oversized_partials():
    w = workloads.custom(seed=708, seq_lens=[64], num_heads=8, num_kv_heads=8, head_size=128,
                         block_size=16, dtype="bf16")
    g = w.to(DEV)
    out = torch.empty((1, 8, 128), device=DEV)
    # 1 x 8 x 1,000,000 x 130 x 4 bytes > 256 MiB
    with pytest.raises(pad.PagedAttnError, match="scratch buffer"):
        pad.paged_attn_decode_static(out, g.query, g.key_cache, g.value_cache, g.block_tables,
                                     g.seq_lens, w.scale, w.max_seq_len, max_num_parts=1_000_000)
