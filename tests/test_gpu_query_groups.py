"""Parity of query groups (num_group query tokens per sequence) with the CPU
oracle: each token of a group attends over its sequence's whole cache, so
the oracle's reference is the same problem with one sequence per query row
(row s * num_group + j taking sequence s's length and pages).
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import workloads
from gpu_util import DEV, check_output, check_partials, run_gpu, say, workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pad.load_library()


CASES = [
    # name, workload kwargs, run kwargs
    ("mfma_g8_ng2_bf16", dict(seed=301, seq_lens=[1, 33, 700, 2049, 0, 512], num_heads=64,
                              num_kv_heads=8, head_size=128, block_size=16, dtype="bf16",
                              num_group=2, poison=True), dict(kernel="mfma")),
    ("mfma_g4_ng3_f16_bs32", dict(seed=302, seq_lens=[1500, 5, 64, 65], num_heads=16,
                                  num_kv_heads=4, head_size=64, block_size=32, dtype="f16",
                                  num_group=3, poison=True), dict(kernel="mfma")),
    ("mfma_mha_ng4", dict(seed=303, seq_lens=[900, 17, 3000], num_heads=4, num_kv_heads=4,
                          head_size=128, block_size=16, dtype="bf16", num_group=4, poison=True),
     dict(kernel="mfma")),
    ("mfma_fp8_alibi_ng2", dict(seed=304, seq_lens=[2500, 1, 130], num_heads=16, num_kv_heads=2,
                                head_size=128, block_size=16, dtype="bf16", kv_cache="fp8",
                                k_scale=0.05, v_scale=0.05, alibi=True, num_group=2, poison=True),
     dict(kernel="mfma")),
    ("valu_f32_ng3", dict(seed=305, seq_lens=[300, 1, 77], num_heads=4, num_kv_heads=2,
                          head_size=64, block_size=8, dtype="f32", num_group=3, poison=True),
     dict(kernel="valu")),
    ("auto_g8_ng3_valu", dict(seed=306, seq_lens=[1000, 40], num_heads=16, num_kv_heads=2,
                              head_size=128, block_size=16, dtype="bf16", num_group=3,
                              poison=True), {}),  # 24 columns: vector kernel
    ("valu_bf16_ng2_grouped", dict(seed=307, seq_lens=[1000, 40], num_heads=16, num_kv_heads=2,
                                   head_size=128, block_size=16, dtype="bf16", num_group=2,
                                   poison=True), dict(kernel="valu")),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_query_groups_match_oracle(orc, case):
    name, wkw, rkw = case
    say(f"query groups {name}")
    w = workloads.custom(name=name, **wkw)
    out, tmp, ml, es = run_gpu(w, **rkw)
    we = w.expanded()
    kernel = rkw.get("kernel", "auto")
    check_partials(we, orc, tmp, ml, es, kernel=kernel)
    check_output(we, orc, out, kernel=kernel)


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_query_groups_with_split_counts(orc, kernel):
    """num_kv_splits with num_group > 1 writes one count per (sequence,
    group); phase 1 and 2 read them in that layout."""
    say(f"query groups with split counts ({kernel})")
    ng = 2
    w = workloads.custom(seed=310, seq_lens=[4000, 3, 900, 2048, 1], num_heads=32, num_kv_heads=8,
                         head_size=128, block_size=32, dtype="bf16", num_group=ng, poison=True)
    ns = torch.empty(w.num_seqs * ng, dtype=torch.int32, device=DEV)
    pad.num_kv_splits(ns, w.seq_lens.to(DEV), ng, w.num_heads, w.num_kv_heads, 16, 256)
    ns = ns.cpu()
    assert np.array_equal(ns.numpy(), orc.num_kv_splits(w.seq_lens.numpy(), ng, w.num_heads,
                                                       w.num_kv_heads, 16, 256))
    out, tmp, ml, es = run_gpu(w, num_splits=ns, max_parts=16, kernel=kernel)
    we = w.expanded()
    check_partials(we, orc, tmp, ml, es, num_splits=ns.numpy(), kernel=kernel)
    check_output(we, orc, out, kernel=kernel)


def test_query_groups_split_runs(orc):
    """Runs of splits per workgroup (16 sequences x 8 kv heads x 32 splits)
    with two query tokens per sequence."""
    say("query groups: split runs")
    lens = [16384, 1, 513, 2047, 2048, 2049, 5000, 0, 100, 16000, 8191, 3, 700, 12345, 64, 15000]
    w = workloads.custom(seed=311, seq_lens=lens, num_heads=64, num_kv_heads=8, head_size=128,
                         block_size=16, dtype="bf16", num_group=2, poison=True)
    out, tmp, ml, es = run_gpu(w, max_parts=32)
    we = w.expanded()
    rows = [0, 1, 2, 3, 14, 15, 18, 19]
    check_partials(we, orc, tmp, ml, es, seqs=rows)
    check_output(we, orc, out, seqs=rows)


@pytest.mark.parametrize("balanced", [False, True])
def test_query_groups_latent_rows(orc, balanced):
    """Latent rows (MLA kernel) with two query tokens per sequence: the
    second token's heads run as their own workgroups."""
    say(f"query groups latent rows balanced={balanced}")
    ng = 2
    w = workloads.mla_custom(seed=312, seq_lens=[300, 1, 1000, 77], num_heads=64, num_group=ng,
                             poison=True)
    if not balanced:
        out, tmp, ml, es = run_gpu(w)
        we = w.expanded()
        check_partials(we, orc, tmp, ml, es)
        check_output(we, orc, out)
        return
    g = w.to(DEV)
    max_parts, workers = 8, 6
    tmp, ml, es = workspace(w, max_parts)
    pad.paged_attn_decode(tmp, es, ml, g.query, g.key_cache, g.value_cache, g.block_tables,
                          g.seq_lens, w.scale, w.max_seq_len, partition_size=0,
                          num_workers=workers, num_group=ng)
    out = torch.full((w.num_seqs * ng, w.num_heads, w.v_head_size), float("nan"), device=DEV)
    pad.paged_attn_reduce(out, tmp, es, ml, g.seq_lens, partition_size=0, num_group=ng)
    torch.cuda.synchronize()
    check_output(w.expanded(), orc, out.cpu())
    # slots past a row's pieces are empty
    mlc = ml.cpu()
    assert torch.isfinite(mlc[:, :, 0]).all() and (mlc[:, :, -1] == -float("inf")).all()


def test_query_groups_rows_checked():
    w = workloads.custom(seed=313, seq_lens=[10, 20], num_heads=4, num_kv_heads=2, head_size=64,
                         block_size=16, dtype="bf16", num_group=2)
    g = w.to(DEV)
    tmp, ml, es = workspace(w, 1)
    with pytest.raises(ValueError):
        pad.paged_attn_decode(tmp, es, ml, g.query, g.key_cache, g.value_cache, g.block_tables,
                              g.seq_lens, w.scale, w.max_seq_len, num_group=3)
