"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer work (token offsets, page_indices, num_kv_splits) must match bit for
bit; attention outputs within max abs error 2e-3 (fp32 caches) or 1e-2
(fp16/bf16 caches) on fp32 outputs. Unused cache slots, unreferenced blocks,
block-table padding and the workspaces are poisoned with NaN (padding points
at a NaN-filled block), so any read of data the method must not read shows.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import workloads
from gpu_util import (DEV, TMP_HALF_ULP, _cache_np, check_output, check_partials, max_parts_for, np64,
                      oracle_args, run_gpu, say, split_lengths, subset)
import pins

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pad.load_library()


# ---------------------------------------------------------------------------
# integer helpers: bit-exact
# ---------------------------------------------------------------------------
def test_token_offsets_worked_example():
    say("token offsets: worked example")
    bt = torch.tensor([[40, 30]], dtype=torch.int32, device=DEV)
    out = torch.full((1, 16), -1, dtype=torch.int64, device=DEV)
    pad.paged_token_offsets(out, bt, torch.tensor([16], dtype=torch.int32, device=DEV), 8, 1, 1)
    rows = [ln.split() for ln in open(pins.GOLDEN + "/worked_example_offsets.txt")
            if ln.strip() and not ln.startswith("#")]
    assert out.cpu()[0].tolist() == [int(r[1]) for r in rows]


@pytest.mark.parametrize("bs", [1, 2, 8, 16, 32, 128])
def test_token_offsets_match_oracle(orc, bs):
    say(f"token offsets bs={bs}")
    rng = np.random.default_rng(bs)
    S = 5
    lens = rng.integers(0, 700, S).astype(np.int32)
    lens[1] = 0
    need = [-(-int(L) // bs) for L in lens]
    nb = sum(need) + 1
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((S, max(need) + 3), nb - 1, dtype=np.int32)
    pos = 0
    for s, n in enumerate(need):
        bt[s, :n] = perm[pos:pos + n]
        pos += n
    block_stride, slot_stride = 8 * 16 * bs * 8, 8
    want = orc.token_offsets(bt, lens, bs, block_stride, slot_stride)
    out = torch.full(want.shape, -1, dtype=torch.int64, device=DEV)
    pad.paged_token_offsets(out, torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV), bs,
                            block_stride, slot_stride)
    assert np.array_equal(out.cpu().numpy(), want)
    # non-unit element stride (every other column of a wider table)
    wide = np.repeat(bt, 2, axis=1)
    view = torch.from_numpy(wide).to(DEV)[:, ::2]
    out2 = torch.full(want.shape, -1, dtype=torch.int64, device=DEV)
    pad.paged_token_offsets(out2, view, torch.from_numpy(lens).to(DEV), bs, block_stride, slot_stride)
    assert np.array_equal(out2.cpu().numpy(), want)


def test_page_indices_match_oracle(orc):
    say("page indices")
    rng = np.random.default_rng(3)
    R, maxB = 37, 3000
    big = rng.integers(0, 1 << 30, (maxB, R)).astype(np.int32)
    big_d = torch.from_numpy(big).to(DEV)
    for contiguous in (True, False):
        # a contiguous [R, maxB] table, then the transposed view of [maxB, R] (stride1 = R)
        bt_np = np.ascontiguousarray(big.T) if contiguous else big.T
        bt_d = big_d.t().contiguous() if contiguous else big_d.t()
        n = rng.integers(0, maxB + 1, R)
        n[[0, 5]] = 0
        n[7] = maxB
        cu = np.zeros(R + 1, dtype=np.int32)
        cu[1:] = np.cumsum(n)
        want = orc.page_indices(bt_np, cu)
        out = torch.full((int(cu[-1]),), -1, dtype=torch.int32, device=DEV)
        pad.build_page_indices(out, bt_d, torch.from_numpy(cu).to(DEV))
        assert np.array_equal(out.cpu().numpy(), want), contiguous


def test_page_indices_long_rows(orc):
    """Rows longer than one round of the copy (8192 entries per round)."""
    say("page indices: long rows")
    rng = np.random.default_rng(4)
    n = np.array([20000, 8193, 8192, 1, 0, 16385], dtype=np.int64)
    bt = rng.integers(0, 1 << 30, (len(n), 20001)).astype(np.int32)
    cu = np.zeros(len(n) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(n)
    want = orc.page_indices(bt, cu)
    out = torch.full((int(cu[-1]),), -1, dtype=torch.int32, device=DEV)
    pad.build_page_indices(out, torch.from_numpy(bt).to(DEV), torch.from_numpy(cu).to(DEV))
    assert np.array_equal(out.cpu().numpy(), want)


def test_page_indices_mla_config(orc):
    say("page indices: MLA config")
    w = workloads.config(5)
    want = orc.page_indices(w.block_tables.numpy(), w.cu_num_blocks.numpy())
    out = torch.full((int(w.cu_num_blocks[-1]),), -1, dtype=torch.int32, device=DEV)
    pad.build_page_indices(out, w.block_tables.to(DEV), w.cu_num_blocks.to(DEV))
    assert np.array_equal(out.cpu().numpy(), want)


def _splits_gpu(lens, g, hq, hk, mx, cores):
    t = torch.as_tensor(lens, dtype=torch.int32, device=DEV)
    out = torch.full((len(lens) * g,), -1, dtype=torch.int32, device=DEV)
    pad.num_kv_splits(out, t, g, hq, hk, mx, cores)
    return out.cpu().numpy()


def test_num_kv_splits_golden():
    say("num_kv_splits golden")
    for ln in open(pins.GOLDEN + "/num_kv_splits_pins.txt"):
        if not ln.strip() or ln.startswith("#"):
            continue
        f = [c.strip() for c in ln.split("|")]
        lens = [int(v) for v in f[1].split(",")]
        g, hq, hk, mx, cores = (int(v) for v in f[2:7])
        want = [int(v) for v in f[7].split(",")]
        assert _splits_gpu(lens, g, hq, hk, mx, cores).tolist() == want, f[0]


def test_num_kv_splits_random(orc):
    say("num_kv_splits random")
    rng = np.random.default_rng(11)
    for trial in range(200):
        S = int(rng.integers(1, 3000))
        lens = np.exp(rng.normal(math.log(rng.integers(1, 20000)), rng.uniform(0, 2), S))
        lens = np.clip(np.rint(lens), -3, 200000).astype(np.int32)
        g = int(rng.integers(1, 4))
        hk = int(rng.integers(1, 9))
        hq = hk * int(rng.choice([1, 2, 4, 8, 16, 32]))
        mx = int(rng.integers(1, 65))
        cores = int(rng.choice([1, 80, 256, 304]))
        want = orc.num_kv_splits(lens, g, hq, hk, mx, cores)
        got = _splits_gpu(lens, g, hq, hk, mx, cores)
        assert np.array_equal(got, want), trial


def test_num_kv_splits_skewed_config(orc):
    say("num_kv_splits: skewed config")
    w = workloads.config(4)
    want = orc.num_kv_splits(w.seq_lens.numpy(), 1, w.num_heads, w.num_kv_heads, w.max_kv_splits,
                             w.device_core_count)
    got = _splits_gpu(w.seq_lens.tolist(), 1, w.num_heads, w.num_kv_heads, w.max_kv_splits,
                      w.device_core_count)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# attention: small cases spanning several chunks / partitions, ragged tails
# ---------------------------------------------------------------------------
SMALL = [
    # name, dtype, lens, H, Hkv, D, bs, partition
    ("f32_mha_bs8", "f32", [16, 13, 300, 1, 0, 129], 2, 2, 64, 8, 64),
    ("f32_gqa_bs4", "f32", [200, 77, 64], 8, 2, 64, 4, 128),
    ("f32_d128_bs1", "f32", [70, 3], 4, 4, 128, 1, 64),
    ("f16_mha_bs16", "f16", [1, 17, 511, 512, 513, 1300], 4, 4, 128, 16, 512),
    ("f16_mha_bs2", "f16", [33, 140], 2, 2, 64, 2, 64),
    ("bf16_mha_bs128", "bf16", [1000, 129, 255], 2, 2, 128, 128, 256),
    ("bf16_gqa8_bs16", "bf16", [1, 31, 32, 33, 700, 1500, 64], 16, 2, 128, 16, 512),
    ("bf16_gqa8_p64", "bf16", [333, 65], 8, 1, 128, 16, 64),
    ("bf16_gqa4_bs32", "bf16", [2047, 96, 5], 8, 2, 128, 32, 512),
    ("bf16_gqa16_bs8", "bf16", [190, 9], 32, 2, 64, 8, 128),
    ("bf16_gqa2_bs64", "bf16", [450, 700], 4, 2, 128, 64, 192),
    ("f16_gqa8_bs16", "f16", [900, 37], 16, 2, 128, 16, 256),
    ("f16_gqa3_d64", "f16", [129, 400], 6, 2, 64, 16, 128),
    ("bf16_d256_gqa4", "bf16", [300, 41], 8, 2, 256, 16, 128),
    ("f32_gqa4_d256", "f32", [150], 4, 1, 256, 16, 64),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_decode_small(orc, case):
    name, dt, lens, H, Hkv, D, bs, P = case
    say(f"decode small {name}")
    w = workloads.custom(seed=zlib.crc32(name.encode()) % 10007, seq_lens=lens, num_heads=H, num_kv_heads=Hkv,
                         head_size=D, block_size=bs, dtype=dt, partition_size=P, poison=True)
    kernels = ["auto", "valu"]
    if dt != "f32" and D in (64, 128) and bs >= 8 and H // Hkv <= 16:
        kernels.append("mfma")  # the grouped-head kernel (also one column: MHA)
    for kernel in kernels:
        out, tmp, ml, es = run_gpu(w, partition_size=P, kernel=kernel)
        check_partials(w, orc, tmp, ml, es, partition_size=P)
        check_output(w, orc, out)


@pytest.mark.parametrize("bs", [256, 1024])
@pytest.mark.parametrize("kv", ["same", "fp8"])
def test_decode_largest_blocks(orc, bs, kv):
    """Block sizes up to the ABI's largest (1024): a split lies inside one or
    two blocks, a sequence may end anywhere in its last block; every
    phase-1 kernel that takes the shape (auto = the grouped-head one, and
    the vector one), query-dtype and fp8 caches."""
    say(f"decode block size {bs} kv={kv}")
    w = workloads.custom(seed=60 + bs, seq_lens=[3000, 1, bs, bs + 1, 0, 700, 2 * bs - 1], num_heads=16,
                         num_kv_heads=2, head_size=128, block_size=bs, dtype="bf16", kv_cache=kv,
                         k_scale=0.05 if kv == "fp8" else 1.0, v_scale=0.05 if kv == "fp8" else 1.0,
                         poison=True)
    for kernel in ("auto", "valu"):
        out, tmp, ml, es = run_gpu(w, kernel=kernel)
        check_partials(w, orc, tmp, ml, es)
        check_output(w, orc, out)


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16])
def test_decode_output_dtypes(orc, out_dtype):
    say(f"decode output dtype {out_dtype}")
    w = workloads.custom(seed=5, seq_lens=[900, 3, 64], num_heads=16, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16", poison=True)
    out, *_ = run_gpu(w, out_dtype=out_dtype)
    check_output(w, orc, out)


def test_decode_csr_page_list(orc):
    say("decode CSR page list")
    w = workloads.custom(seed=6, seq_lens=[515, 1, 250], num_heads=8, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16", poison=True)
    out, tmp, ml, es = run_gpu(w, csr=True)
    check_partials(w, orc, tmp, ml, es)
    check_output(w, orc, out)


def test_decode_strided_caches_and_table(orc):
    """K and V interleaved in one allocation (outer strides larger than packed)
    and a block table read with element stride 2."""
    say("decode strided caches")
    w = workloads.custom(seed=8, seq_lens=[300, 45], num_heads=8, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="f16", poison=True)
    NB = w.num_blocks
    kv = torch.stack([w.key_cache.reshape(NB, -1), w.value_cache.reshape(NB, -1)], dim=1).to(DEV)
    kd = kv[:, 0].view(w.key_cache.shape)    # block stride 2 * Hkv * D * bs
    vd = kv[:, 1].view(w.value_cache.shape)
    assert kd.stride(0) == 2 * 2 * 128 * 16 and vd.stride(0) == kd.stride(0)
    g = w.to(DEV)
    wide = torch.repeat_interleave(w.block_tables, 2, dim=1).to(DEV)[:, ::2]
    P = 512
    mp = max_parts_for(w, P)
    tmp = torch.full((2, 8, mp, 128), float("nan"), device=DEV)
    ml = torch.full((2, 8, mp), float("nan"), device=DEV)
    es = torch.full((2, 8, mp), float("nan"), device=DEV)
    pad.paged_attn_decode(tmp, es, ml, g.query, kd, vd, wide, g.seq_lens, w.scale, w.max_seq_len)
    out = torch.empty((2, 8, 128), device=DEV)
    pad.paged_attn_reduce(out, tmp, es, ml, g.seq_lens)
    check_output(w, orc, out.cpu())


def test_decode_num_splits(orc):
    """Split counts from the heuristic on the device, consumed by both phases."""
    say("decode num_splits")
    w = workloads.custom(seed=9, seq_lens=[3000, 17, 400, 1, 1024, 2500], num_heads=16,
                         num_kv_heads=4, head_size=128, block_size=32, dtype="bf16", poison=True)
    g = w.to(DEV)
    ns = torch.empty(w.num_seqs, dtype=torch.int32, device=DEV)
    pad.num_kv_splits(ns, g.seq_lens, 1, w.num_heads, w.num_kv_heads, 16, 256)
    nsc = ns.cpu().numpy()
    assert np.array_equal(nsc, orc.num_kv_splits(w.seq_lens.numpy(), 1, 16, 4, 16, 256))
    for kernel in ("auto", "valu"):
        out, tmp, ml, es = run_gpu(w, num_splits=nsc, max_parts=16, kernel=kernel)
        check_partials(w, orc, tmp, ml, es, num_splits=nsc)
        check_output(w, orc, out)
    # clamped to max_num_parts
    out, tmp, ml, es = run_gpu(w, num_splits=[40] * 6, max_parts=4)
    check_partials(w, orc, tmp, ml, es, num_splits=[40] * 6)
    check_output(w, orc, out)


# ---------------------------------------------------------------------------
# MLA-style latent rows (page size 1, V = leading columns of K)
# ---------------------------------------------------------------------------
MLA_CASES = [
    # name, heads, lens, partition
    ("g128_ragged", 128, [1, 15, 16, 17, 100, 513, 1030], 512),
    ("g64_p64", 64, [64, 65, 300, 7], 64),
    ("g128_long", 128, [2500, 4097], 1024),
]


@pytest.mark.parametrize("case", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_decode_mla(orc, case):
    name, H, lens, P = case
    say(f"decode mla {name}")
    w = workloads.mla_custom(seed=zlib.crc32(name.encode()) % 10007, seq_lens=lens, num_heads=H,
                             poison=True)
    for kernel in ("auto", "valu"):
        out, tmp, ml, es = run_gpu(w, partition_size=P, kernel=kernel, csr=True)
        check_partials(w, orc, tmp, ml, es, partition_size=P)
        check_output(w, orc, out)


def test_decode_mla_num_splits(orc):
    say("decode mla num_splits")
    w = workloads.mla_custom(seed=77, seq_lens=[3000, 129, 1, 900], num_heads=128, poison=True)
    g = w.to(DEV)
    ns = torch.empty(w.num_seqs, dtype=torch.int32, device=DEV)
    pad.num_kv_splits(ns, g.seq_lens, 1, 128, 1, 8, 256)
    nsc = ns.cpu().numpy()
    out, tmp, ml, es = run_gpu(w, num_splits=nsc, max_parts=8, csr=True)
    check_partials(w, orc, tmp, ml, es, num_splits=nsc)
    check_output(w, orc, out)


def _mla_f16_late_scores(orc, seed, lens, num_heads):
    """f16 latent rows whose later scores pass each split's first-chunk max
    by 16 to 64 (base 2) for some head, and by less than 64 for every head:
    the rope columns (512..575, which V does not read) of every token after
    the first 32 of its sequence are scaled by a factor f, chosen as the
    smallest of a fixed list that puts the batch in that window. A
    probability 2^d with d >= 16 is +inf in f16."""
    base = workloads.mla_custom(seed=seed, seq_lens=lens, num_heads=num_heads, dtype="f16",
                                poison=True)
    for f in (3.0, 4.0, 5.0, 6.0, 8.0, 10.0, 12.0, 16.0):
        w = workloads.mla_custom(seed=seed, seq_lens=lens, num_heads=num_heads, dtype="f16",
                                 poison=True)
        for s, L in enumerate(lens):
            rows = w.block_tables[s, 32:L].long()
            w.latent[rows, 512:] = (w.latent[rows, 512:].float() * f).to(torch.float16)
        # each sequence is one split (L <= 512): chunk maxima from 32-token splits
        _, m32, _ = orc.partials(*oracle_args(w), max_num_parts=16, partition_size=32)
        over = []
        for s, L in enumerate(lens):
            n = -(-L // 32)
            over.append((m32[s, :, :n].max(axis=1) - m32[s, :, 0]) / math.log(2.0))
        over = np.concatenate(over)
        if over.max() > 20.0 and over.max() < 60.0:
            say(f"f16 latent rows: rope scale {f}, largest pass of the first-chunk max "
                f"{over.max():.1f} (base 2)")
            return w
    raise AssertionError(f"no scale puts the scores in the window (base seed {seed}, {base.name})")


@pytest.mark.parametrize("mode", ["fixed", "balanced1", "balanced3"])
def test_decode_mla_f16_overflow_window(orc, mode):
    """f16 latent rows on the matrix-core kernel with later scores 16..64
    (base 2) above the first chunk's max: every probability must stay finite
    and the output match the oracle."""
    say(f"decode mla f16 overflow window {mode}")
    w = _mla_f16_late_scores(orc, 4242, [300, 200, 45, 511], 128)
    if mode == "fixed":
        out, tmp, ml, es = run_gpu(w, partition_size=512, csr=True)
        check_partials(w, orc, tmp, ml, es, partition_size=512)
    else:
        workers = 1 if mode == "balanced1" else 3
        out, tmp, ml, es = run_balanced(w, workers, 4)
        check_balanced_pieces(w, orc, tmp, ml, es, workers, 4)
    assert torch.isfinite(out).all()
    check_output(w, orc, out)


@pytest.mark.parametrize("H", [64, 128])
def test_decode_mla_f16(orc, H):
    """f16 latent rows, fixed and balanced splits, plain and with ALiBi."""
    say(f"decode mla f16 H={H}")
    w = workloads.mla_custom(seed=90 + H, seq_lens=[1, 15, 700, 1030, 33], num_heads=H,
                             dtype="f16", poison=True)
    out, tmp, ml, es = run_gpu(w, partition_size=256, csr=True)
    check_partials(w, orc, tmp, ml, es, partition_size=256)
    check_output(w, orc, out)
    out, tmp, ml, es = run_balanced(w, 5, 8)
    check_balanced_pieces(w, orc, tmp, ml, es, 5, 8)
    check_output(w, orc, out)
    w.alibi_slopes = workloads.alibi_slopes(H)
    out, tmp, ml, es = run_gpu(w, partition_size=256, csr=True)
    check_partials(w, orc, tmp, ml, es, partition_size=256)
    check_output(w, orc, out)
    out, *_ = run_balanced(w, 5, 8)
    check_output(w, orc, out)


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_block_permutation_is_bit_identical(kernel):
    say(f"block permutation {kernel}")
    w = workloads.custom(seed=12, seq_lens=[700, 90], num_heads=8, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16", num_blocks=80)
    out1, *_ = run_gpu(w, kernel=kernel)
    perm = torch.randperm(80, generator=torch.Generator().manual_seed(1))
    w2 = subset(w, [0, 1])
    w2.key_cache = torch.empty_like(w.key_cache)
    w2.value_cache = torch.empty_like(w.value_cache)
    w2.key_cache[perm] = w.key_cache
    w2.value_cache[perm] = w.value_cache
    w2.block_tables = perm[w.block_tables.long()].to(torch.int32)
    out2, *_ = run_gpu(w2, kernel=kernel)
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("kernel", ["auto", "valu"])
def test_length_one_returns_the_value_row(kernel):
    say(f"length one {kernel}")
    w = workloads.custom(seed=13, seq_lens=[1, 1, 1], num_heads=8, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16", poison=True)
    out, *_ = run_gpu(w, kernel=kernel)
    for s in range(3):
        blk = int(w.block_tables[s, 0])
        for h in range(8):
            assert torch.equal(out[s, h], w.value_cache[blk, h // 4, :, 0].float())


def test_partition_size_invariance():
    say("partition invariance")
    w = workloads.custom(seed=14, seq_lens=[1500, 600], num_heads=8, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16")
    ref, *_ = run_gpu(w, partition_size=2048)
    for P in (64, 192, 512):
        out, *_ = run_gpu(w, partition_size=P)
        assert (out - ref).abs().max().item() < 1e-2


def test_constant_values():
    say("constant values")
    w = workloads.custom(seed=15, seq_lens=[777, 40], num_heads=16, num_kv_heads=2, head_size=64,
                         block_size=16, dtype="bf16")
    w.value_cache[:] = 1.5
    for kernel in ("auto", "valu"):
        out, *_ = run_gpu(w, kernel=kernel)
        assert (out - 1.5).abs().max().item() < 1e-6


# ---------------------------------------------------------------------------
# reduce alone, fed oracle partials
# ---------------------------------------------------------------------------
def test_reduce_with_oracle_partials(orc):
    say("reduce with oracle partials")
    w = workloads.custom(seed=16, seq_lens=[2000, 5, 0, 513], num_heads=4, num_kv_heads=1,
                         head_size=64, v_head_size=64, block_size=16, dtype="f32", poison=True)
    P = 64
    mp = max_parts_for(w, P) + 2
    otmp, oml, oes = orc.partials(*oracle_args(w), max_num_parts=mp, partition_size=P)
    want = orc.reduce(np.nan_to_num(otmp, nan=0.0), oml, oes, w.seq_lens.numpy(), partition_size=P)
    tmp = torch.from_numpy(otmp).float().to(DEV)  # NaN stays in the empty splits
    ml = torch.from_numpy(oml).float().to(DEV)
    es = torch.from_numpy(oes).float().to(DEV)
    out = torch.empty((4, 4, 64), device=DEV)
    pad.paged_attn_reduce(out, tmp, es, ml, w.seq_lens.to(DEV), partition_size=P)
    got = out.cpu().double().numpy()
    assert np.abs(got - want).max() < 1e-5
    assert np.all(got[2] == 0)


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times; the
# oracle checks every sequence's output and every split's statistics
# ---------------------------------------------------------------------------
FULL = [1, 2, 3, 4, 5]


@pytest.mark.parametrize("cfg", FULL, ids=[f"config{c}" for c in FULL])
def test_full_config(orc, cfg):
    say(f"full config {cfg}")
    w = workloads.config(cfg, poison=True)
    ns = None
    mp = None
    if cfg == 4:
        g = w.to(DEV)
        t = torch.empty(w.num_seqs, dtype=torch.int32, device=DEV)
        pad.num_kv_splits(t, g.seq_lens, 1, w.num_heads, w.num_kv_heads, w.max_kv_splits,
                          w.device_core_count)
        ns = t.cpu().numpy()
        assert np.array_equal(ns, orc.num_kv_splits(w.seq_lens.numpy(), 1, w.num_heads,
                                                    w.num_kv_heads, w.max_kv_splits,
                                                    w.device_core_count))
        mp = w.max_kv_splits
    out, tmp, ml, es = run_gpu(w, num_splits=ns, max_parts=mp, csr=(cfg == 5))
    err = check_output(w, orc, out)
    check_partials(w, orc, tmp, ml, es, num_splits=ns)
    say(f"full config {cfg}: all {w.num_seqs} sequences, max abs err {err:.2e}")


# ---------------------------------------------------------------------------
# balanced splits (partition_size 0): equal token ranges over the batch
# ---------------------------------------------------------------------------
PIECE_CHARGE = 256  # virtual tokens before each non-empty sequence (pagedattn.h)


def balanced_pieces(lens, workers, max_parts):
    """Per sequence, the (slot, start, end) pieces of the balanced split rule
    stated in pagedattn.h."""
    L = [max(0, int(x)) for x in lens]
    T = sum(Ls + PIECE_CHARGE for Ls in L if Ls > 0)
    maxL = max(L + [0])
    U = max(-(-T // workers), -(-maxL // (max_parts - 1)))
    U = max(-(-U // 32) * 32, 32)
    out, v = [], 0
    for Ls in L:
        pieces = []
        if Ls > 0:
            off = v + PIECE_CHARGE  # position of the sequence's first token
            w0, w1 = off // U, (off + Ls - 1) // U
            for w in range(w0, w1 + 1):
                pieces.append((w - w0, max(w * U, off) - off, min((w + 1) * U, off + Ls) - off))
            v += Ls + PIECE_CHARGE
        out.append(pieces)
    return out


def run_balanced(w, workers, max_parts, out_dtype=torch.float32, tmp_dtype=torch.float32):
    g = w.to(DEV)
    tmp, ml, es = workspace_nan(w, max_parts, tmp_dtype)
    cu = torch.zeros(w.num_seqs + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(w.seq_lens.clamp(min=0), 0)
    indptr = cu.to(DEV)
    flat = torch.full((max(int(cu[-1]), 1),), -1, dtype=torch.int32, device=DEV)
    pad.build_page_indices(flat, g.block_tables, indptr)
    pad.paged_attn_decode(tmp, es, ml, g.query, g.key_cache, g.value_cache, flat, g.seq_lens,
                          w.scale, w.max_seq_len, partition_size=0, num_workers=workers,
                          kv_indptr=indptr, alibi_slopes=g.alibi_slopes, num_group=w.num_group,
                          k_scale=w.k_scale, v_scale=w.v_scale)
    out = torch.full((w.num_seqs * w.num_group, w.num_heads, w.v_head_size), float("nan"),
                     dtype=out_dtype, device=DEV)
    pad.paged_attn_reduce(out, tmp, es, ml, g.seq_lens, partition_size=0, num_group=w.num_group)
    torch.cuda.synchronize()
    return out.cpu(), tmp.cpu(), ml.cpu(), es.cpu()


def workspace_nan(w, max_parts, tmp_dtype=torch.float32):
    S, H, Dv = w.num_seqs * w.num_group, w.num_heads, w.v_head_size
    return (torch.full((S, H, max_parts, Dv), float("nan"), dtype=tmp_dtype, device=DEV),
            torch.full((S, H, max_parts), float("nan"), device=DEV),
            torch.full((S, H, max_parts), float("nan"), device=DEV))


def check_balanced_pieces(w, orc, tmp, ml, es, workers, max_parts):
    """Each piece's statistics and normalised row against the oracle on that
    token range alone (every piece of the batch, in one oracle call that
    treats each piece as a sequence of its own); slots past a sequence's
    pieces marked empty."""
    pieces = balanced_pieces(w.seq_lens.tolist(), workers, max_parts)
    flat = [(s, slot, a, b) for s, ps in enumerate(pieces) for slot, a, b in ps]
    if flat:
        width = max(b - a for _, _, a, b in flat)
        bt = np.zeros((len(flat), width), np.int32)
        for i, (s, _, a, b) in enumerate(flat):
            bt[i, :b - a] = w.block_tables[s, a:b].numpy()
        rows = [s * w.num_group for s, _, _, _ in flat]
        q = np64(w.query[rows])
        lens = np.array([b - a for _, _, a, b in flat], np.int32)
        P = -(-width // 64) * 64
        # With ALiBi a piece [a, b) run as a sequence of its own gets the
        # bias slope * (t - (b - 1)) instead of slope * (t - (L - 1)): every
        # score of head h moves by the constant slope_h * (b - L), which
        # leaves the normalised row and the exp sum (taken against the
        # piece's own max) unchanged and moves the max logit by it.
        kw = {} if w.alibi_slopes is None else dict(alibi=w.alibi_slopes.numpy())
        t_o, m_o, l_o = orc.partials(q, _cache_np(w.key_cache), _cache_np(w.value_cache), bt, lens, w.scale,
                                     1, partition_size=P, k_scale=w.k_scale, v_scale=w.v_scale, **kw)
        if kw:
            slopes = w.alibi_slopes.double().numpy()
            for i, (s, _, _, b) in enumerate(flat):
                m_o[i, :, 0] += slopes * (b - int(w.seq_lens[s]))
        atol, ltol = (1e-2, 4e-3) if w.dtype == torch.bfloat16 else (1e-2, 2e-3)
        for i, (s, slot, a, b) in enumerate(flat):
            r = s * w.num_group
            m_g, l_g, t_g = ml[r, :, slot].double().numpy(), es[r, :, slot].double().numpy(), tmp[r, :, slot].double().numpy()
            assert np.all(np.abs(m_g - m_o[i, :, 0]) <= 2e-4 + 1e-5 * np.abs(m_o[i, :, 0])), (s, slot)
            # the exp-sum bound widened by the scores' rounding at the max's magnitude
            lb = ltol + 2.0 * 2.0 ** -23 * np.abs(m_o[i, :, 0])
            assert np.all(np.abs(l_g - l_o[i, :, 0]) <= lb * np.abs(l_o[i, :, 0])), (s, slot)
            et = np.abs(t_g - t_o[i, :, 0]) - TMP_HALF_ULP[tmp.dtype] * np.abs(t_o[i, :, 0])
            assert et.max() <= atol, (s, slot)
    for s, ps in enumerate(pieces):
        for slot in range(len(ps), max_parts):
            assert torch.all(ml[s * w.num_group, :, slot] == -math.inf) and \
                torch.all(es[s * w.num_group, :, slot] == 0), (s, slot)


BAL_CASES = [
    # name, heads, lens, workers, max_parts
    ("g128_w1", 128, [1, 15, 16, 17, 100, 513, 1030, 0, 700, 33], 1, 8),
    ("g128_w5", 128, [1, 15, 16, 17, 100, 513, 1030, 0, 700, 33], 5, 8),
    ("g128_w64_p2", 128, [1, 15, 16, 17, 100, 513, 1030, 0, 700, 33], 64, 2),
    ("g64_w3", 64, [64, 65, 300, 7], 3, 4),
    ("g128_one_long", 128, [2100], 7, 16),
]


@pytest.mark.parametrize("case", BAL_CASES, ids=[c[0] for c in BAL_CASES])
def test_decode_mla_balanced(orc, case):
    name, H, lens, workers, max_parts = case
    say(f"decode mla balanced {name}")
    w = workloads.mla_custom(seed=zlib.crc32(name.encode()) % 10007, seq_lens=lens, num_heads=H,
                             poison=True)
    out, tmp, ml, es = run_balanced(w, workers, max_parts)
    check_balanced_pieces(w, orc, tmp, ml, es, workers, max_parts)
    check_output(w, orc, out)


def test_decode_mla_balanced_all_empty():
    say("decode mla balanced, all sequences empty")
    w = workloads.mla_custom(seed=5, seq_lens=[0, 0, 0], num_heads=128, max_blocks=4, poison=True)
    out, tmp, ml, es = run_balanced(w, 4, 3)
    assert torch.all(out == 0)
    assert torch.all(ml == -math.inf) and torch.all(es == 0)


BAL_REDUCE_CASES = [
    # name, Dv, split-row dtype, max_parts, live slots per row (0: empty sequence)
    ("dv512_bf16", 512, torch.bfloat16, 16, [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 0]),
    ("dv128_f32", 128, torch.float32, 40, [1, 4, 15, 16, 17, 31, 32, 33, 39, 40, 0, 8]),
]


@pytest.mark.parametrize("case", BAL_REDUCE_CASES, ids=[c[0] for c in BAL_REDUCE_CASES])
def test_reduce_balanced_slot_counts(orc, case):
    """Phase 2 on balanced-split partials alone: each row's live slots are a
    prefix of its slots (m = -inf, l = 0 and NaN rows after it), of every
    length from one slot to all of them, around the merge's batch
    boundaries. Against the oracle's merge over that many splits (a split
    count k with lengths 6400 k gives exactly k splits of 6400 tokens)."""
    name, Dv, tdt, P, counts = case
    say(f"reduce balanced slot counts {name}")
    gen = torch.Generator().manual_seed(zlib.crc32(name.encode()))
    S, H = len(counts), 4
    ml = torch.randn((S, H, P), generator=gen) * 3.0
    es = torch.rand((S, H, P), generator=gen) * 50.0 + 0.5
    tmp = torch.randn((S, H, P, Dv), generator=gen).to(tdt)
    for s, k in enumerate(counts):
        ml[s, :, k:] = -math.inf
        es[s, :, k:] = 0.0
        tmp[s, :, k:] = float("nan")
    lens = torch.tensor([6400 * k for k in counts], dtype=torch.int32)
    out = torch.full((S, H, Dv), float("nan"), device=DEV)
    pad.paged_attn_reduce(out, tmp.to(DEV), es.to(DEV), ml.to(DEV), lens.to(DEV), partition_size=0)
    torch.cuda.synchronize()
    want = orc.reduce(np64(tmp), np64(ml), np64(es), lens.numpy(), partition_size=64,
                      num_splits=np.array([max(k, 1) for k in counts], dtype=np.int32))
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - want)
    assert (err <= 2e-6 + 2e-6 * np.abs(want)).all(), err.max()


def test_decode_mla_balanced_config5(orc):
    """The MLA workload as the benchmark runs it (one token range per compute
    unit): every sequence's output and every piece's statistics."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"decode mla balanced config5 ({cus} workers)")
    w = workloads.config(5, poison=True)
    max_parts = -(-w.max_seq_len // 512)
    out, tmp, ml, es = run_balanced(w, cus, max_parts)
    check_balanced_pieces(w, orc, tmp, ml, es, cus, max_parts)
    err = check_output(w, orc, out)
    say(f"decode mla balanced config5: max abs err {err:.2e}")


# ---------------------------------------------------------------------------
# runs of consecutive splits per workgroup (grouped-head matrix-core kernel,
# fixed split size): the launcher picks 1-4 splits per workgroup so that the
# grid is about one workgroup per SIMD; these batches reach runs of 2, 3 and
# 4 on a 256-CU device. Ragged lengths leave runs partly empty and end runs
# mid-split.
# ---------------------------------------------------------------------------
RUN_LENS = [16384, 1, 513, 2047, 2048, 2049, 5000, 0, 100, 16000, 8191, 3, 700, 12345, 64, 15000]


@pytest.mark.parametrize("nseq,kv,d", [(8, "same", 128), (12, "same", 128), (16, "same", 128),
                                       (16, "fp8", 128), (16, "same", 64)])
def test_split_runs(orc, nseq, kv, d):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    units = nseq * 8 * 32
    say(f"split runs: {nseq} seqs, kv {kv}, head size {d}, run {max(1, min(4, units // (4 * cus)))}")
    w = workloads.custom(seed=(200 if d == 128 else 300) + nseq, seq_lens=RUN_LENS[:nseq], num_heads=64, num_kv_heads=8,
                         head_size=d, block_size=16, dtype="bf16", kv_cache=kv,
                         k_scale=0.05, v_scale=0.05, poison=True)
    out, tmp, ml, es = run_gpu(w, max_parts=32)
    seqs = [0, 1, 2, 5, 7] + ([9, 13] if nseq > 13 else [])
    check_partials(w, orc, tmp, ml, es, seqs=seqs)
    check_output(w, orc, out, seqs=seqs)
    assert torch.isfinite(out).all()


# ---------------------------------------------------------------------------
# persistent workers (grouped-head matrix-core kernel with per-sequence split
# counts): each worker takes the splits whose first token falls in its equal
# share of the batch's tokens. Batches longer than one 256-sequence scan
# step, more workers than tokens, lengths 0 and 1, counts clamped into
# [1, max_num_parts], fp8 caches with ALiBi, and above 2048 sequences the
# one-workgroup-per-split grid.
# ---------------------------------------------------------------------------
def _ragged_lens(seed, n, hi):
    r = np.random.default_rng(seed)
    lens = r.integers(2, hi, n)
    lens[::17] = 0
    lens[5::23] = 1
    return lens.tolist()


PERSIST_CASES = [
    # name, workload kwargs, split counts, max_num_parts
    ("s300_heuristic_bs32", dict(seed=401, seq_lens=_ragged_lens(401, 300, 3000), num_heads=32,
                                 num_kv_heads=8, head_size=128, block_size=32, dtype="bf16"),
     "heuristic", 32),
    ("s70_counts_clamped_g8_f16", dict(seed=402, seq_lens=_ragged_lens(402, 70, 5000), num_heads=16,
                                       num_kv_heads=2, head_size=128, block_size=16, dtype="f16"),
     "random", 16),
    ("s5_fewer_tokens_than_workers", dict(seed=403, seq_lens=[1, 3, 0, 64, 65], num_heads=8,
                                          num_kv_heads=8, head_size=64, block_size=8, dtype="bf16"),
     "heuristic", 8),
    ("s40_fp8_alibi", dict(seed=404, seq_lens=_ragged_lens(404, 40, 9000), num_heads=32,
                           num_kv_heads=4, head_size=128, block_size=16, dtype="bf16",
                           kv_cache="fp8", k_scale=0.05, v_scale=0.05, alibi=True),
     "heuristic", 32),
    ("s2100_grid", dict(seed=405, seq_lens=_ragged_lens(405, 2100, 200), num_heads=8,
                        num_kv_heads=2, head_size=64, block_size=16, dtype="bf16"),
     "heuristic", 8),
    ("s24_one_kv_head_g16", dict(seed=406, seq_lens=_ragged_lens(406, 24, 6000), num_heads=16,
                                 num_kv_heads=1, head_size=128, block_size=32, dtype="bf16"),
     "heuristic", 16),
    ("s20_d64_runs", dict(seed=408, seq_lens=_ragged_lens(408, 20, 9000), num_heads=16,
                          num_kv_heads=4, head_size=64, block_size=16, dtype="bf16"),
     "random", 24),
    ("s30_fp8_bs8_runtime_block", dict(seed=407, seq_lens=_ragged_lens(407, 30, 3000), num_heads=8,
                                       num_kv_heads=2, head_size=128, block_size=8, dtype="f16",
                                       kv_cache="fp8_codes", k_scale=0.02, v_scale=0.03),
     "random", 12),
]


@pytest.mark.parametrize("case", PERSIST_CASES, ids=[c[0] for c in PERSIST_CASES])
def test_persistent_workers(orc, case):
    name, wkw, counts, mp = case
    say(f"persistent workers {name}")
    w = workloads.custom(name=name, poison=True, **wkw)
    if counts == "heuristic":
        t = torch.empty(w.num_seqs, dtype=torch.int32, device=DEV)
        pad.num_kv_splits(t, w.seq_lens.to(DEV), 1, w.num_heads, w.num_kv_heads, mp, 256)
        ns = t.cpu().numpy()
    else:
        ns = np.random.default_rng(7).integers(-2, 3 * mp, w.num_seqs).astype(np.int32)
    out, tmp, ml, es = run_gpu(w, num_splits=ns, max_parts=mp)
    # every sequence: live splits finite, empty ones -inf / 0 with tmp untouched
    lens = split_lengths(w, 512, ns, mp)
    for s in range(w.num_seqs):
        L = int(w.seq_lens[s])
        n = 0 if L <= 0 else -(-L // lens[s])
        assert (ml[s, :, n:] == -math.inf).all() and (es[s, :, n:] == 0).all(), (s, n)
        assert torch.isnan(tmp[s, :, n:]).all(), (s, n)
        assert torch.isfinite(ml[s, :, :n]).all() and torch.isfinite(tmp[s, :, :n]).all(), (s, n)
        assert torch.isfinite(out[s]).all(), s
    L = w.seq_lens.numpy()
    order = np.argsort(L, kind="stable")
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(L) // 2]),
                   int(np.flatnonzero(L == L[L > 0].min())[0]), 1, w.num_seqs - 1})
    check_partials(w, orc, tmp, ml, es, num_splits=ns, seqs=seqs)
    check_output(w, orc, out, seqs=seqs)


# ---------------------------------------------------------------------------
# 16-bit split workspaces: phase 1 stores each split's output converted to the
# workspace's element type ([PAv2] converts at the store to tmp_output's
# type), rounded to nearest even; phase 2 reads it back widened to fp32
# ---------------------------------------------------------------------------
TMP16_CASES = [
    # name, dtype, lens, H, Hkv, D, bs, partition, tmp dtype
    ("f16_mha_tmp_f16", "f16", [1, 17, 511, 512, 513, 1300], 4, 4, 128, 16, 512, torch.float16),
    ("bf16_gqa8_tmp_bf16", "bf16", [1, 31, 32, 33, 700, 1500, 64], 16, 2, 128, 16, 512, torch.bfloat16),
    ("bf16_gqa4_tmp_f16", "bf16", [2047, 96, 5], 8, 2, 128, 32, 256, torch.float16),
    ("f32_gqa4_tmp_bf16", "f32", [200, 77, 64], 8, 2, 64, 4, 128, torch.bfloat16),
]


@pytest.mark.parametrize("case", TMP16_CASES, ids=[c[0] for c in TMP16_CASES])
def test_decode_tmp16(orc, case):
    name, dt, lens, H, Hkv, D, bs, P, tdt = case
    say(f"decode 16-bit workspace {name}")
    w = workloads.custom(seed=zlib.crc32(name.encode()) % 10007, seq_lens=lens, num_heads=H, num_kv_heads=Hkv,
                         head_size=D, block_size=bs, dtype=dt, partition_size=P, poison=True)
    for kernel in ["auto", "valu"]:
        out, tmp, ml, es = run_gpu(w, partition_size=P, kernel=kernel, tmp_dtype=tdt)
        assert tmp.dtype == tdt
        check_partials(w, orc, tmp, ml, es, partition_size=P)
        check_output(w, orc, out, tmp=tmp)


def _same(a, b):
    """Equal, NaN slots (never written) included."""
    return torch.equal(torch.isnan(a), torch.isnan(b)) and torch.equal(a.nan_to_num(0.0), b.nan_to_num(0.0))


def test_decode_tmp16_is_the_rounded_f32_workspace():
    """A 16-bit workspace holds exactly the fp32 workspace's values rounded to
    nearest even (same kernel, same inputs), and the statistics are the
    same bits."""
    say("16-bit workspace = rounded fp32 workspace")
    w = workloads.custom(seed=77, seq_lens=[900, 3, 64, 1500], num_heads=16, num_kv_heads=2, head_size=128,
                         block_size=16, dtype="bf16", poison=True)
    for kernel in ["auto", "valu"]:
        _, t32, m32, e32 = run_gpu(w, kernel=kernel)
        for tdt in (torch.bfloat16, torch.float16):
            _, t16, m16, e16 = run_gpu(w, kernel=kernel, tmp_dtype=tdt)
            assert _same(m16, m32) and _same(e16, e32), (kernel, tdt)
            assert _same(t16, t32.to(tdt)), (kernel, tdt)


def test_reduce_reads_16bit_workspaces(orc):
    """Phase 2 on oracle partials rounded to 16 bits equals the oracle's merge
    of the rounded values (the reduce widens them exactly)."""
    say("reduce of 16-bit oracle partials")
    w = workloads.custom(seed=16, seq_lens=[2000, 5, 0, 513], num_heads=4, num_kv_heads=1,
                         head_size=64, v_head_size=64, block_size=16, dtype="f32", poison=True)
    P = 64
    mp = max_parts_for(w, P) + 2
    otmp, oml, oes = orc.partials(*oracle_args(w), max_num_parts=mp, partition_size=P)
    for tdt in (torch.bfloat16, torch.float16):
        t16 = torch.from_numpy(otmp).to(tdt)
        want = orc.reduce(np.nan_to_num(t16.double().numpy(), nan=0.0), oml, oes, w.seq_lens.numpy(),
                          partition_size=P)
        out = torch.empty((4, 4, 64), device=DEV)
        pad.paged_attn_reduce(out, t16.to(DEV), torch.from_numpy(oes).float().to(DEV),
                              torch.from_numpy(oml).float().to(DEV), w.seq_lens.to(DEV), partition_size=P)
        got = out.cpu().double().numpy()
        assert np.abs(got - want).max() < 1e-5, tdt
        assert np.all(got[2] == 0)


def test_decode_mla_balanced_tmp_bf16(orc):
    """The MLA workload as the benchmark runs it, with the split outputs in a
    bf16 workspace."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"decode mla balanced config5, bf16 workspace ({cus} workers)")
    w = workloads.config(5, poison=True)
    max_parts = -(-w.max_seq_len // 512)
    out, tmp, ml, es = run_balanced(w, cus, max_parts, tmp_dtype=torch.bfloat16)
    check_balanced_pieces(w, orc, tmp, ml, es, cus, max_parts)
    err = check_output(w, orc, out, tmp=tmp)
    say(f"decode mla balanced config5, bf16 workspace: max abs err {err:.2e}")


def test_full_config3_tmp_bf16(orc):
    """The long-context GQA workload in the benchmark's launch with a bf16
    workspace: every sequence's output and every split's statistics."""
    say("full config 3, bf16 workspace")
    w = workloads.config(3, poison=True)
    out, tmp, ml, es = run_gpu(w, tmp_dtype=torch.bfloat16)
    err = check_output(w, orc, out, tmp=tmp)
    check_partials(w, orc, tmp, ml, es)
    say(f"full config 3, bf16 workspace: max abs err {err:.2e}")


# ---------------------------------------------------------------------------
# fp8 E4M3 latent rows on the latent-row kernel ([PAv2] wrapper arguments
# kv_cache_dtype, k_scale, v_scale): codes copied to LDS as they are, widened
# to the query's type there (exactly), k_scale on the scores, v_scale on the
# output
# ---------------------------------------------------------------------------
FP8_MLA_CASES = [
    # name, heads, lens, dtype, k_scale, v_scale
    ("g128_bf16", 128, [600, 31, 1, 2049, 64], "bf16", 0.02, 0.05),
    ("g64_bf16", 64, [300, 1000, 7], "bf16", 1.0 / 32, 1.0 / 32),
    ("g128_f16", 128, [777, 40], "f16", 0.04, 0.03),
]


@pytest.mark.parametrize("case", FP8_MLA_CASES, ids=[c[0] for c in FP8_MLA_CASES])
def test_decode_mla_fp8(orc, case):
    name, H, lens, dt, ks, vs = case
    say(f"decode mla fp8 {name}")
    w = workloads.mla_custom(seed=zlib.crc32(name.encode()) % 10007, seq_lens=lens, num_heads=H,
                             dtype=dt, kv_cache="fp8", k_scale=ks, v_scale=vs, poison=True)
    out, tmp, ml, es = run_gpu(w, partition_size=512)
    check_partials(w, orc, tmp, ml, es, partition_size=512)
    check_output(w, orc, out)
    # the vector kernel on the same codes, within its own (fp32) bounds
    out_v, *_ = run_gpu(w, partition_size=512, kernel="valu")
    check_output(w, orc, out_v, kernel="valu")


def test_decode_mla_fp8_balanced(orc):
    say("decode mla fp8 balanced")
    w = workloads.mla_custom(seed=511, seq_lens=[1, 15, 16, 17, 100, 513, 1030, 0, 700, 33], num_heads=128,
                             kv_cache="fp8", k_scale=0.03, v_scale=0.06, poison=True)
    out, tmp, ml, es = run_balanced(w, 5, 8)
    check_balanced_pieces(w, orc, tmp, ml, es, 5, 8)
    check_output(w, orc, out)


def test_decode_mla_fp8_balanced_g64(orc):
    """64 heads over fp8 latent rows (one widened slot, two workgroups a
    compute unit), balanced splits over 16 token ranges."""
    say("decode mla fp8 balanced, 64 heads")
    w = workloads.mla_custom(seed=512, seq_lens=[1, 15, 16, 17, 100, 513, 1030, 0, 700, 33, 2200], num_heads=64,
                             kv_cache="fp8", k_scale=0.04, v_scale=0.05, poison=True)
    out, tmp, ml, es = run_balanced(w, 16, 12)
    check_balanced_pieces(w, orc, tmp, ml, es, 16, 12)
    check_output(w, orc, out)


def test_decode_mla_fp8_balanced_config5(orc):
    """The MLA workload with fp8 latent rows as the benchmark runs it
    (balanced splits, one token range per compute unit): every sequence's
    output and every piece's statistics."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    say(f"decode mla fp8 balanced config5 ({cus} workers)")
    w = workloads.config(5, poison=True, kv_cache="fp8")
    max_parts = -(-w.max_seq_len // 512)
    out, tmp, ml, es = run_balanced(w, cus, max_parts)
    check_balanced_pieces(w, orc, tmp, ml, es, cus, max_parts)
    err = check_output(w, orc, out)
    say(f"decode mla fp8 balanced config5: max abs err {err:.2e}")


# ---------------------------------------------------------------------------
# Cache offsets past 2^31 elements: every decode kernel forms a cache address
# as a 64-bit page id times a 64-bit page stride. The same step on a cache
# whose used blocks sit past element 2^31 (the rest NaN) must give the same
# bits as on the compact cache, and match the oracle.

BIG_OFFSET_CASES = [
    ("grouped_heads_bf16", lambda: workloads.custom(seed=41, seq_lens=[700, 33, 1100], num_heads=16, num_kv_heads=2,
                                                    head_size=128, block_size=16, dtype="bf16")),
    ("one_column_f16", lambda: workloads.custom(seed=42, seq_lens=[900, 5, 1300], num_heads=4, num_kv_heads=4,
                                                head_size=128, block_size=16, dtype="f16")),
    ("latent_rows_bf16", lambda: workloads.mla_custom(seed=43, seq_lens=[600, 70], num_heads=128)),
    ("latent_rows_fp8", lambda: workloads.mla_custom(seed=44, seq_lens=[600, 70], num_heads=128, kv_cache="fp8")),
]


def _page_elems(t: torch.Tensor) -> int:
    return t[0].numel()


@pytest.mark.parametrize("case", BIG_OFFSET_CASES, ids=[c[0] for c in BIG_OFFSET_CASES])
def test_cache_offsets_past_2_31_elements(orc, case):
    name, make = case
    w = make()
    say(f"cache offsets past 2^31 elements: {name}")
    want = run_gpu(w)
    g = w.to(DEV)
    fp8 = g.key_cache.dtype == torch.uint8
    poison = dict(fill_value=workloads.FP8_NAN_CODE) if fp8 else dict(fill_value=float("nan"))
    nb = g.key_cache.shape[0]
    if w.latent is not None:
        off = 2 ** 31 // _page_elems(g.latent) + 1000
        big = torch.full((off + nb, *g.latent.shape[1:]), dtype=g.latent.dtype, device=DEV, **poison)
        big[off:] = g.latent
        kc, vc = workloads._mla_views(big, w.v_head_size)
    else:
        off = 2 ** 31 // _page_elems(g.key_cache) + 1000
        kc = torch.full((off + nb, *g.key_cache.shape[1:]), dtype=g.key_cache.dtype, device=DEV, **poison)
        vc = torch.full((off + nb, *g.value_cache.shape[1:]), dtype=g.value_cache.dtype, device=DEV, **poison)
        kc[off:] = g.key_cache
        vc[off:] = g.value_cache
    assert off * kc.stride(0) > 2 ** 31 and off * vc.stride(0) > 2 ** 31
    bt = g.block_tables + off
    assert int(bt.max()) < kc.shape[0]
    R = w.num_seqs * w.num_group
    max_parts = max_parts_for(w, 512)
    tmp = torch.full((R, w.num_heads, max_parts, w.v_head_size), float("nan"), device=DEV)
    ml = torch.full((R, w.num_heads, max_parts), float("nan"), device=DEV)
    es = torch.full((R, w.num_heads, max_parts), float("nan"), device=DEV)
    pad.paged_attn_decode(tmp, es, ml, g.query, kc, vc, bt, g.seq_lens, w.scale, w.max_seq_len,
                          partition_size=512, alibi_slopes=g.alibi_slopes, k_scale=w.k_scale,
                          v_scale=w.v_scale, num_group=w.num_group)
    out = torch.full((R, w.num_heads, w.v_head_size), float("nan"), device=DEV)
    pad.paged_attn_reduce(out, tmp, es, ml, g.seq_lens, partition_size=512, num_group=w.num_group)
    torch.cuda.synchronize()
    got = (out.cpu(), tmp.cpu(), ml.cpu(), es.cpu())
    del kc, vc, tmp, ml, es, out
    if w.latent is not None:
        del big
    torch.cuda.empty_cache()
    for a, b, what in zip(got, want, ("output", "tmp_output", "max_logits", "exp_sums")):
        torch.testing.assert_close(a, b, rtol=0, atol=0, equal_nan=True, msg=f"{name}: {what}")
    check_output(w, orc, got[0])
