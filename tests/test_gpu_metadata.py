"""Parity of the decode-metadata launch (normal_decode_set_metadata, through
the C ABI) with the CPU oracle: every output bit for bit.

Output buffers are filled with a sentinel first, so entries the call must
write and does not, or must not write and does, show.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import workloads
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu

SENTINEL = -123456789


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pad.load_library()


def _strided(t: torch.Tensor, step: int) -> torch.Tensor:
    """The same values as t, as a view whose last dimension has stride `step`."""
    shape = list(t.shape)
    big = torch.full(shape[:-1] + [shape[-1] * step], SENTINEL, dtype=t.dtype, device=t.device)
    big[..., ::step] = t
    return big[..., ::step]


def run_metadata(c: workloads.MetadataCase, strided: bool = False, swa: bool = None):
    """GPU outputs as numpy arrays (cache_seqlens, cu, page_table, swa_table)."""
    B, P = c.batch, c.max_seq_pages
    swa = c.full_to_swa is not None if swa is None else swa
    seq_lens = c.seq_lens.to(DEV)
    rtt = c.req_to_token.to(DEV)
    rows = c.req_pool_indices.to(DEV)
    f2s = c.full_to_swa.to(DEV) if swa else None
    if strided:
        seq_lens, rtt, rows = _strided(seq_lens, 3), _strided(rtt, 2), _strided(rows, 2)
        f2s = _strided(f2s, 2) if swa else None
        # outputs: padded rows / spaced elements
        cs_buf = torch.full((2 * B,), SENTINEL, dtype=torch.int32, device=DEV)
        cu_buf = torch.full((3 * (B + 1),), SENTINEL, dtype=torch.int32, device=DEV)
        pt_buf = torch.full((B, P + 5), SENTINEL, dtype=torch.int32, device=DEV)
        cs, cu, pt = cs_buf[::2], cu_buf[::3], pt_buf[:, :P]
        sw_buf = torch.full((B, 2 * P + 1), SENTINEL, dtype=torch.int32, device=DEV)
        sw = sw_buf[:, 1::2][:, :P] if swa else None
    else:
        cs = torch.full((B,), SENTINEL, dtype=torch.int32, device=DEV)
        cu = torch.full((B + 1,), SENTINEL, dtype=torch.int32, device=DEV)
        pt = torch.full((B, P), SENTINEL, dtype=torch.int32, device=DEV)
        sw = torch.full((B, P), SENTINEL, dtype=torch.int32, device=DEV) if swa else None
    pad.normal_decode_set_metadata(cs, cu, pt, rtt, rows, P, seq_lens, c.seq_len_delta,
                                   c.page_size, swa_page_table=sw, full_to_swa=f2s)
    torch.cuda.synchronize()
    out = [cs.cpu().numpy(), cu.cpu().numpy(), pt.cpu().numpy(), None if sw is None else sw.cpu().numpy()]
    if strided:  # the gaps between strided outputs are untouched
        assert (cs_buf.view(B, 2)[:, 1] == SENTINEL).all() if B else True
        assert (cu_buf.view(B + 1, 3)[:, 1:] == SENTINEL).all()
        assert (pt_buf[:, P:] == SENTINEL).all()
        if swa:
            assert (sw_buf[:, 0::2] == SENTINEL).all()
    return out


def check(orc, c, strided=False):
    got = run_metadata(c, strided=strided)
    want = orc.decode_metadata(c.seq_lens.numpy(), c.req_to_token.numpy(),
                               c.req_pool_indices.numpy(), c.max_seq_pages, c.page_size,
                               c.seq_len_delta,
                               None if c.full_to_swa is None else c.full_to_swa.numpy())
    for name, g, w in zip(("cache_seqlens", "cu_seqlens_k", "page_table", "swa_page_table"), got, want):
        if w is None:
            assert g is None
            continue
        assert g.shape == w.shape, name
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[:3].tolist()}"
    return got


CASES = [
    # name, seed, lens, page size, delta, swa, pool rows
    ("ps1_mla_like", 1, "mla", 1, 0, False, None),
    ("ps16_ragged_delta", 2, [1, 15, 16, 17, 2048, 1000, 0, 33], 16, 1, False, None),
    ("ps32_swa_skewed", 3, "skewed", 32, 0, True, 600),
    ("ps8_many_tiles", 4, "many", 8, 1, False, None),
    ("ps4_swa_ragged", 5, [3, 0, 129, 4, 5], 4, -1, True, None),
    ("ps1024_few_pages", 6, [5000, 1, 1024, 1025], 1024, 0, True, None),
]


def _lens(spec, seed):
    g = np.random.default_rng(seed)
    if spec == "mla":
        return g.integers(1024, 8193, 64).tolist()
    if spec == "skewed":
        return np.clip(np.rint(np.exp(np.log(1024) + g.standard_normal(256))), 1, 16384).astype(int).tolist()
    if spec == "many":  # scan over three 2048-entry tiles, gather over many rows
        return g.integers(0, 300, 5000).tolist()
    return spec


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_metadata_matches_oracle(orc, case):
    name, seed, lens, ps, delta, swa, pool = case
    say(f"metadata {name}")
    c = workloads.metadata_case(seed=seed, seq_lens=_lens(lens, seed), page_size=ps,
                                seq_len_delta=delta, swa=swa, pool_rows=pool)
    _, _, pt, _ = check(orc, c)
    # the page table reproduces the block table the slots were laid out from
    for b, L in enumerate(c.seq_lens.tolist()):
        n = (max(0, L) + ps - 1) // ps
        assert np.array_equal(pt[b, :n], c.block_tables.numpy()[b, :n])


@pytest.mark.parametrize("swa", [False, True])
def test_metadata_strided(orc, swa):
    say(f"metadata strided swa={swa}")
    c = workloads.metadata_case(seed=11, seq_lens=[70, 3, 0, 257, 64], page_size=16,
                                seq_len_delta=2, swa=swa)
    check(orc, c, strided=True)


def test_metadata_empty_and_no_pages(orc):
    say("metadata empty")
    cu = torch.full((1,), SENTINEL, dtype=torch.int32, device=DEV)
    e32 = torch.zeros(0, dtype=torch.int32, device=DEV)
    e64 = torch.zeros(0, dtype=torch.int64, device=DEV)
    pad.normal_decode_set_metadata(e32, cu, torch.zeros((0, 4), dtype=torch.int32, device=DEV),
                                   torch.zeros((1, 64), dtype=torch.int32, device=DEV), e64, 4,
                                   e64, 0, 16)
    torch.cuda.synchronize()
    assert cu.tolist() == [0]
    c = workloads.metadata_case(seed=12, seq_lens=[9, 1, 40], page_size=4, seq_len_delta=1,
                                max_seq_pages=0)
    cs, cuo, pt, _ = check(orc, c)
    assert pt.shape == (3, 0) and cs.tolist() == [10, 2, 41]


def test_metadata_negative_slots_and_wrap(orc):
    say("metadata negative slots / int32 wrap")
    rng = np.random.default_rng(13)
    B, P, ps = 6, 40, 8
    rtt = rng.integers(-2**31, 2**31 - 1, (B + 2, P * ps), dtype=np.int64).astype(np.int32)
    lens = np.array([2**31 - 1, 2**31 - 8, 5, 0, 2**30, 7], np.int64)
    c = workloads.MetadataCase(seq_lens=torch.from_numpy(lens), req_to_token=torch.from_numpy(rtt),
                               req_pool_indices=torch.tensor([7, 0, 3, 3, 5, 1]),
                               block_tables=torch.zeros((B, 1), dtype=torch.int32), page_size=ps,
                               max_seq_pages=P, seq_len_delta=3)
    cs, cu, pt, _ = check(orc, c)
    assert (pt < 0).any() and (cu < 0).any()  # the cases this test is for occurred


# ---------------------------------------------------------------------------
# speculative SWA page table (prepare_swa_spec_page_table)
# ---------------------------------------------------------------------------
def _spec_inputs(seed, bs, R, LA, LB, over=False):
    rng = np.random.default_rng(seed)
    a = rng.integers(0, 2**31 - 1, (bs, LA)).astype(np.int32)
    b = rng.integers(0, 2**31 - 1, (bs * R, LB)).astype(np.int32)
    hi_a, hi_b = (LA + 40, LB + 7) if over else (LA, LB)
    la = rng.integers(-3 if over else 0, hi_a + 1, bs).astype(np.int32)
    lb = rng.integers(0, hi_b + 1, bs * R).astype(np.int32)
    return a, b, la, lb


def run_spec(a, b, la, lb, R, strided=False):
    bs, LA, LB = a.shape[0], a.shape[1], b.shape[1]
    ta, tb = torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)
    if strided:  # a as a transposed view, b with a column stride of 2, dst with padded rows
        ta = ta.t().contiguous().t()
        tb = _strided(tb, 2)
        buf = torch.full((bs * R, LA + LB + 9), SENTINEL, dtype=torch.int32, device=DEV)
        dst = buf[:, :LA + LB]
    else:
        dst = torch.full((bs * R, LA + LB), SENTINEL, dtype=torch.int32, device=DEV)
    pad.prepare_swa_spec_page_table(dst, ta, tb, torch.from_numpy(la).to(DEV),
                                    torch.from_numpy(lb).to(DEV), R)
    torch.cuda.synchronize()
    if strided:
        assert (buf[:, LA + LB:] == SENTINEL).all()
    return dst.cpu().numpy()


SPEC_CASES = [
    # name, seed, bs, R, LA, LB, lengths past the widths / negative
    ("mla_like", 31, 64, 4, 8192, 8, False),
    ("small_ragged", 32, 7, 3, 300, 17, False),
    ("over_widths", 33, 9, 2, 1030, 5, True),
    ("one_draft", 34, 33, 1, 2049, 1, False),
]


@pytest.mark.parametrize("case", SPEC_CASES, ids=[c[0] for c in SPEC_CASES])
@pytest.mark.parametrize("strided", [False, True])
def test_spec_page_table_matches_oracle(orc, case, strided):
    name, seed, bs, R, LA, LB, over = case
    say(f"spec page table {name} strided={strided}")
    a, b, la, lb = _spec_inputs(seed, bs, R, LA, LB, over)
    got = run_spec(a, b, la, lb, R, strided=strided)
    want = orc.swa_spec_page_table(a, b, la, lb, R, fill=SENTINEL)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


def test_spec_page_table_empty():
    say("spec page table empty")
    dst = torch.full((0, 12), SENTINEL, dtype=torch.int32, device=DEV)
    e = torch.zeros(0, dtype=torch.int32, device=DEV)
    pad.prepare_swa_spec_page_table(dst, torch.zeros((0, 8), dtype=torch.int32, device=DEV),
                                    torch.zeros((0, 4), dtype=torch.int32, device=DEV), e, e, 3)
    torch.cuda.synchronize()
