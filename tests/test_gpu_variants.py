"""Parity of the phase-1 variants with the CPU oracle: FP8 E4M3 caches with
k_scale / v_scale, and ALiBi slopes, on every kernel that serves them.

FP8 codes decode exactly. On the vector kernel the rest is fp32, so those
cases take the fp32-cache tolerances; on the matrix-core kernel the codes
are widened to the query's 16-bit type and the probabilities rounded to it,
so those cases take that type's tolerances, as ALiBi there does. Unused cache slots and unreferenced blocks are
poisoned (NaN, or the E4M3 NaN code 0x7F) where the case says so.
"""
import dataclasses

import numpy as np
import pytest
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import workloads
from gpu_util import (DEV, check_output, check_partials, oracle_args, oracle_kw,
                      run_gpu, say, tolerances)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pad.load_library()


CASES = [
    # name, workload kwargs, run kwargs
    ("fp8_gqa_bf16", dict(seed=101, seq_lens=[1, 17, 300, 1000, 2049, 0, 64], num_heads=8,
                          num_kv_heads=2, head_size=128, block_size=16, dtype="bf16",
                          kv_cache="fp8", k_scale=0.05, v_scale=0.08, poison=True), {}),
    ("fp8_gqa_bf16_splits", dict(seed=102, seq_lens=[3000, 5, 700, 1], num_heads=16,
                                 num_kv_heads=2, head_size=128, block_size=16, dtype="bf16",
                                 kv_cache="fp8", k_scale=0.03, v_scale=0.1, poison=True),
     dict(num_splits=[7, 1, 3, 2], max_parts=8)),
    ("fp8_bs8_f32_group4", dict(seed=103, seq_lens=[100, 513, 7], num_heads=4, num_kv_heads=1,
                                head_size=128, block_size=8, dtype="f32", kv_cache="fp8",
                                k_scale=0.05, v_scale=0.05, poison=True), {}),
    ("fp8_bs1_rows_f16", dict(seed=104, seq_lens=[300, 45], num_heads=2, num_kv_heads=2,
                              head_size=128, block_size=1, dtype="f16", kv_cache="fp8",
                              k_scale=0.05, v_scale=0.2, poison=True), dict(partition_size=128)),
    ("fp8_latent_576", dict(seed=105, seq_lens=[600, 31], num_heads=16, num_kv_heads=1,
                            head_size=576, v_head_size=512, block_size=1, dtype="bf16",
                            kv_cache="fp8", k_scale=0.02, v_scale=0.05), {}),
    ("fp8_bs64_mha_f16", dict(seed=106, seq_lens=[2000, 129, 64, 63], num_heads=4, num_kv_heads=4,
                              head_size=64, block_size=64, dtype="f16", kv_cache="fp8",
                              k_scale=0.05, v_scale=0.05, poison=True), dict(partition_size=256)),
    ("alibi_mfma_bf16", dict(seed=111, seq_lens=[1, 2, 33, 1000, 3000], num_heads=32,
                             num_kv_heads=4, head_size=128, block_size=16, dtype="bf16",
                             alibi=True, poison=True), dict(kernel="mfma")),
    ("alibi_mfma_f16_d64_g16", dict(seed=112, seq_lens=[513, 77, 4096], num_heads=32,
                                    num_kv_heads=2, head_size=64, block_size=32, dtype="f16",
                                    alibi=True, poison=True), dict(kernel="mfma")),
    ("alibi_mfma_bf16_splits", dict(seed=113, seq_lens=[5000, 40, 900], num_heads=16,
                                    num_kv_heads=2, head_size=128, block_size=16, dtype="bf16",
                                    alibi=True), dict(kernel="mfma", num_splits=[9, 1, 4],
                                                      max_parts=12)),
    ("alibi_mha_mfma_f16", dict(seed=117, seq_lens=[800, 2, 129], num_heads=4, num_kv_heads=4,
                                head_size=128, block_size=16, dtype="f16", alibi=True,
                                poison=True), dict(kernel="mfma")),
    ("fp8_mha_mfma_bf16", dict(seed=118, seq_lens=[1500, 64, 3], num_heads=4, num_kv_heads=4,
                               head_size=64, block_size=32, dtype="bf16", kv_cache="fp8",
                               k_scale=0.05, v_scale=0.05, poison=True), dict(kernel="mfma")),
    ("alibi_valu_f32", dict(seed=114, seq_lens=[700, 3, 64], num_heads=4, num_kv_heads=4,
                            head_size=128, block_size=16, dtype="f32", alibi=True, poison=True),
     dict(kernel="valu")),
    ("alibi_valu_bf16_group", dict(seed=115, seq_lens=[1500, 9], num_heads=16, num_kv_heads=2,
                                   head_size=128, block_size=16, dtype="bf16", alibi=True),
     dict(kernel="valu")),
    ("alibi_fp8_bf16", dict(seed=116, seq_lens=[2500, 1, 130], num_heads=8, num_kv_heads=1,
                            head_size=128, block_size=16, dtype="bf16", kv_cache="fp8",
                            k_scale=0.05, v_scale=0.05, alibi=True, poison=True),
     dict(kernel="mfma")),
    ("alibi_fp8_bf16_valu", dict(seed=116, seq_lens=[2500, 1, 130], num_heads=8, num_kv_heads=1,
                                 head_size=128, block_size=16, dtype="bf16", kv_cache="fp8",
                                 k_scale=0.05, v_scale=0.05, alibi=True, poison=True),
     dict(kernel="valu")),
    # fp8 caches on the grouped-head matrix-core kernel
    ("fp8_mfma_bf16_bs16", dict(seed=131, seq_lens=[1, 7, 8, 9, 31, 33, 1000, 2049], num_heads=16,
                                num_kv_heads=2, head_size=128, block_size=16, dtype="bf16",
                                kv_cache="fp8", k_scale=0.05, v_scale=0.08, poison=True),
     dict(kernel="mfma")),
    ("fp8_mfma_f16_bs32_d64", dict(seed=132, seq_lens=[4100, 63, 64, 65], num_heads=32,
                                   num_kv_heads=2, head_size=64, block_size=32, dtype="f16",
                                   kv_cache="fp8", k_scale=0.04, v_scale=0.1, poison=True),
     dict(kernel="mfma")),
    ("fp8_mfma_bf16_bs8_g2", dict(seed=133, seq_lens=[777, 5, 100], num_heads=4, num_kv_heads=2,
                                  head_size=128, block_size=8, dtype="bf16", kv_cache="fp8",
                                  k_scale=0.05, v_scale=0.05, poison=True), dict(kernel="mfma")),
    ("fp8_mfma_bf16_bs64_splits", dict(seed=134, seq_lens=[6000, 300, 2], num_heads=8,
                                       num_kv_heads=1, head_size=128, block_size=64, dtype="bf16",
                                       kv_cache="fp8", k_scale=0.05, v_scale=0.05, poison=True),
     dict(kernel="mfma", num_splits=[11, 2, 1], max_parts=16)),
    ("fp8_valu_bf16_group", dict(seed=131, seq_lens=[1, 7, 8, 9, 31, 33, 1000, 2049], num_heads=16,
                                 num_kv_heads=2, head_size=128, block_size=16, dtype="bf16",
                                 kv_cache="fp8", k_scale=0.05, v_scale=0.08, poison=True),
     dict(kernel="valu")),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_variant_matches_oracle(orc, case):
    name, wkw, rkw = case
    say(f"variant {name}")
    w = workloads.custom(name=name, **wkw)
    P = rkw.get("partition_size", 512)
    out, tmp, ml, es = run_gpu(w, **rkw)
    kernel = rkw.get("kernel", "auto")
    check_partials(w, orc, tmp, ml, es, partition_size=P, num_splits=rkw.get("num_splits"),
                   kernel=kernel)
    check_output(w, orc, out, kernel=kernel)


def _live_codes(cache: torch.Tensor, w: workloads.Workload, value: bool) -> torch.Tensor:
    """Codes of every live token of a paged fp8 cache."""
    bs = w.block_size
    parts = []
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        for i in range((L + bs - 1) // bs):
            n = min(bs, L - i * bs)
            blk = cache[int(w.block_tables[s, i])]
            parts.append((blk[:, :, :n] if value else blk[:, :, :n, :]).flatten())
    return torch.cat(parts)


def test_fp8_every_code(orc):
    """Codes uniform over all 254 non-NaN E4M3 codes (subnormals, both zeros,
    448), each present in the live keys and values."""
    say("fp8 every code")
    w = workloads.custom(seed=120, seq_lens=[700, 5, 129], num_heads=4, num_kv_heads=4,
                         head_size=64, block_size=32, dtype="f16", kv_cache="fp8_codes",
                         k_scale=1.0 / 448, v_scale=1.0 / 448, poison=True)
    for value, c in ((False, w.key_cache), (True, w.value_cache)):
        seen = torch.bincount(_live_codes(c, w, value).long(), minlength=256)
        assert int((seen > 0).sum()) == 254 and seen[0x7F] == 0 and seen[0xFF] == 0
    out, tmp, ml, es = run_gpu(w, partition_size=256)
    check_partials(w, orc, tmp, ml, es, partition_size=256)
    check_output(w, orc, out)
    # grouped heads over the same kinds of codes, on the matrix-core kernel
    w = workloads.custom(seed=124, seq_lens=[700, 5, 129], num_heads=16, num_kv_heads=2,
                         head_size=128, block_size=16, dtype="bf16", kv_cache="fp8_codes",
                         k_scale=1.0 / 448, v_scale=1.0 / 448, poison=True)
    for value, c in ((False, w.key_cache), (True, w.value_cache)):
        seen = torch.bincount(_live_codes(c, w, value).long(), minlength=256)
        assert int((seen > 0).sum()) == 254
    out, tmp, ml, es = run_gpu(w, kernel="mfma")
    check_partials(w, orc, tmp, ml, es, kernel="mfma")
    check_output(w, orc, out, kernel="mfma")


def test_alibi_moves_the_output(orc):
    """The slopes are applied: the result is far from the no-ALiBi one."""
    say("alibi changes the output")
    w = workloads.custom(seed=121, seq_lens=[400, 1200], num_heads=16, num_kv_heads=2,
                         head_size=128, block_size=16, dtype="bf16", alibi=True)
    out = run_gpu(w, kernel="mfma")[0].double().numpy()
    plain = orc.attention(*oracle_args(w))
    assert np.abs(out - plain).max() > 20 * tolerances(w)[0]
    ref = orc.attention(*oracle_args(w), **oracle_kw(w))
    assert np.abs(out - ref).max() <= tolerances(w)[0]


@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_alibi_latent_rows(orc, kernel):
    """Latent rows (V aliasing K, page size 1) with ALiBi, 64 and 128 heads on
    the latent-row kernel (auto) and on the vector kernel. On the latent-row
    kernel the bf16 splits start from a reference raised by the bias growth
    over the split; the f16 ones (and any split whose scores outgrow it)
    take the second, exact-reference pass."""
    for H, lens in ((64, [300, 1, 1000, 2049]), (128, [700, 33])):
        say(f"alibi latent rows H={H} kernel={kernel}")
        w = workloads.mla_custom(seed=122 + H, seq_lens=lens, num_heads=H, poison=True)
        w.alibi_slopes = workloads.alibi_slopes(H)
        out, tmp, ml, es = run_gpu(w, kernel=kernel)
        check_partials(w, orc, tmp, ml, es)
        check_output(w, orc, out)


@pytest.mark.parametrize("kv,dtype,H", [("same", "bf16", 128), ("same", "bf16", 64), ("fp8", "bf16", 128),
                                         ("same", "f16", 128), ("fp8", "f16", 64)])
def test_alibi_latent_rows_balanced(orc, kv, dtype, H):
    """ALiBi on the latent-row kernel with balanced splits (the form the MLA
    benchmark runs): every piece's statistics and row against the oracle on
    its token range (max logits moved by the bias offset of the range), and
    the merged output; fp8 rows and f16 queries included."""
    import test_gpu_parity as tp
    say(f"alibi latent rows, balanced: kv={kv} dtype={dtype} H={H}")
    lens = [1, 300, 2049, 0, 1000, 4100]
    w = workloads.mla_custom(seed=140 + H, seq_lens=lens, num_heads=H, poison=True, dtype=dtype, kv_cache=kv)
    w.alibi_slopes = workloads.alibi_slopes(H)
    workers, max_parts = 7, 12
    out, tmp, ml, es = tp.run_balanced(w, workers, max_parts)
    tp.check_balanced_pieces(w, orc, tmp, ml, es, workers, max_parts)
    check_output(w, orc, out)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_alibi_latent_rows_fp8(orc, dtype):
    """ALiBi with fp8 latent rows, fixed 512-token splits."""
    say(f"alibi latent rows, fp8 rows, {dtype}")
    w = workloads.mla_custom(seed=150, seq_lens=[700, 33, 1537, 1], num_heads=128, poison=True, dtype=dtype,
                             kv_cache="fp8")
    w.alibi_slopes = workloads.alibi_slopes(128)
    out, tmp, ml, es = run_gpu(w)
    check_partials(w, orc, tmp, ml, es)
    check_output(w, orc, out)


def test_alibi_latent_rows_reference_guards(orc):
    """The latent-row kernel's raised ALiBi reference and its two reruns.
    One 2048-token split per sequence, slopes 0.07 (the bias grows by ~202
    in base 2 over a split: more than an fp32 exponent below the reference
    can hold). Sequence 0, head 0: the first eight keys are aligned with the
    head's query, so its scores peak in the first chunk, ~202 below the
    raised reference (the kernel must rerun it against the true max; kept,
    its sums would underflow). Sequence 1, head 1: the last eight keys are
    aligned with its query, so its scores outgrow the raised reference by
    more than the headroom (rerun as before). Other heads keep one pass."""
    say("alibi latent rows: raised reference, both reruns")
    w = workloads.mla_custom(seed=131, seq_lens=[2000, 1900], num_heads=128, poison=True)
    w.alibi_slopes = torch.full((128,), 0.07, dtype=torch.float32)
    q = w.query.float()
    scale_nat = w.scale
    # alpha * |q|^2 * scale ~ 160 nats (head 0), 120 nats (head 1)
    for seq, head, toks, nats in ((0, 0, range(0, 8), 160.0), (1, 1, range(1892, 1900), 120.0)):
        qh = q[seq, head]
        alpha = nats / (float(qh.dot(qh)) * scale_nat)
        pages = w.block_tables[seq, list(toks)].long()
        w.latent[pages] = (alpha * qh).to(w.latent.dtype)
    out, tmp, ml, es = run_gpu(w, partition_size=2048)
    assert torch.isfinite(out).all() and torch.isfinite(es).all()
    check_partials(w, orc, tmp, ml, es, partition_size=2048)
    check_output(w, orc, out)


def test_fp8_scales_scale_linearly(orc):
    """Halving v_scale halves the output; k_scale only reshapes the softmax."""
    say("fp8 scales")
    w = workloads.custom(seed=123, seq_lens=[800, 50], num_heads=4, num_kv_heads=1,
                         head_size=128, block_size=16, dtype="bf16", kv_cache="fp8",
                         k_scale=0.05, v_scale=0.1)
    a = run_gpu(w)[0].double()
    b = run_gpu(dataclasses.replace(w, v_scale=0.05))[0].double()  # the same codes
    assert torch.allclose(b * 2, a, rtol=1e-6, atol=1e-7)
    c = run_gpu(dataclasses.replace(w, k_scale=0.1))[0].double()
    assert (c - a).abs().max() > 1e-2
    check_output(dataclasses.replace(w, k_scale=0.1), orc, c.float())


# ---------------------------------------------------------------------------
# the variant workloads at full size, in the launch configuration the
# benchmark times (--kv-cache fp8, --alibi, --num-group); the oracle checks
# sampled sequences
# ---------------------------------------------------------------------------
FULL_VARIANTS = [
    # config, workload kwargs
    (3, dict(kv_cache="fp8")),
    (3, dict(alibi=True)),
    (3, dict(num_group=2)),
    (2, dict(kv_cache="fp8")),
    (2, dict(num_group=4)),
    (4, dict(kv_cache="fp8")),
]


@pytest.mark.parametrize("cfg,kw", FULL_VARIANTS,
                         ids=[f"config{c}_" + "_".join(f"{k}{v}" for k, v in kw.items())
                              for c, kw in FULL_VARIANTS])
def test_full_variant_config(orc, cfg, kw):
    """Every query row's output and every split's statistics."""
    say(f"full variant config {cfg} {kw}")
    w = workloads.config(cfg, poison=True, **kw)
    ns, mp = None, None
    if cfg == 4:
        g = w.to(DEV)
        t = torch.empty(w.num_seqs * w.num_group, dtype=torch.int32, device=DEV)
        pad.num_kv_splits(t, g.seq_lens, w.num_group, w.num_heads, w.num_kv_heads,
                          w.max_kv_splits, w.device_core_count)
        ns, mp = t.cpu().numpy(), w.max_kv_splits
    out, tmp, ml, es = run_gpu(w, num_splits=ns, max_parts=mp)
    we = w.expanded()
    err = check_output(we, orc, out)
    check_partials(we, orc, tmp, ml, es, num_splits=ns)
    say(f"full variant config {cfg} {kw}: all {we.num_seqs} rows, max abs err {err:.2e}")


def test_full_config5_alibi_balanced(orc):
    """The MLA workload with ALiBi slopes as the benchmark runs it (balanced
    splits, one token range per compute unit): every sequence's output."""
    say("full config 5 alibi balanced")
    import test_gpu_parity as tp
    w = workloads.config(5, poison=True, alibi=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    max_parts = -(-w.max_seq_len // 512)
    out, tmp, ml, es = tp.run_balanced(w, cus, max_parts)
    err = check_output(w, orc, out)
    say(f"full config 5 alibi balanced: max abs err {err:.2e}")
