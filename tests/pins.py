"""Pins for the CPU oracle: checks against facts the pages and the mathematics
fix, never against the oracle itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees. The real oracle must pass all of them; every planted-mistake
build of the oracle must fail at least one (test_oracle_mutants.py).

What pins what:
  token offsets  worked example of triton issue 2522 (golden file); numpy
                 fancy indexing of a real 5-D cache for bs in 1..32 (brute force)
  attention      numpy/scipy brute force on tiny inputs; torch SDPA (float64,
                 enable_gqa) on identity block tables; closed forms (scale 0 ->
                 mean of V, length 1 -> that V row, constant V, one-hot limit);
                 block relabelling invariance; MLA latent rows by brute force
  partials       per-partition softmax statistics by brute force; merge of any
                 partitioning equals the unpartitioned definition
  reduce         closed form of a two-partition merge; one partition -> identity
  num_kv_splits  hand evaluations of the sglang formula (golden file)
  page_indices   numpy concatenation of the table rows, incl. strided views
  decode meta    page table read back from slots laid out by a block table;
                 prefix-sum identities and int32 wrap; floor division of
                 negative slots; SWA map invariants (identity, page relabel);
                 empty batch
  spec page tbl  numpy concatenation of the two prefixes per draft row;
                 zeros past the table widths; untouched past the total
  fp8 caches     every E4M3 code against torch's float8_e4m3fn, through a
                 value row and through one-hot queries on keys
  ALiBi          geometric-series closed form with zero scores (weights,
                 max logit, exp sum, both slope signs); zero slopes = plain
"""
from __future__ import annotations

import math
import os

import numpy as np
import scipy.special
import torch

from paged_attention_decode_tables_amd import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _np(t):
    return t.float().numpy() if isinstance(t, torch.Tensor) else np.asarray(t)


def brute_attention(q, kc, vc, bt, seq_lens, scale, indptr=None):
    """float64 softmax attention through numpy fancy indexing of the paged cache."""
    q = np.asarray(q, np.float64)
    kc = np.asarray(kc, np.float64)
    vc = np.asarray(vc, np.float64)
    S, H, D = q.shape
    NB, Hkv, Dx, bs, x = kc.shape
    Dv = vc.shape[2]
    G = H // Hkv
    out = np.zeros((S, H, Dv))
    for s in range(S):
        L = int(seq_lens[s])
        if L <= 0:
            continue
        t = np.arange(L)
        if indptr is None:
            pb = np.asarray(bt)[s, t // bs]
        else:
            pb = np.asarray(bt)[int(indptr[s]) + t // bs]
        o = t % bs
        for kvh in range(Hkv):
            K = kc[pb, kvh, :, o, :].reshape(L, D)
            V = vc[pb, kvh, :, o]
            for g in range(G):
                h = kvh * G + g
                z = scale * (K @ q[s, h])
                out[s, h] = scipy.special.softmax(z) @ V
    return out


def _run(o, w, scale=None, **kw):
    return o.attention(_np(w.query), _np(w.key_cache), _np(w.value_cache), w.block_tables.numpy(),
                       w.seq_lens.numpy(), w.scale if scale is None else scale, **kw)


def _brute(w, scale=None):
    return brute_attention(_np(w.query), _np(w.key_cache), _np(w.value_cache),
                           w.block_tables.numpy(), w.seq_lens.numpy(),
                           w.scale if scale is None else scale)


TINY_CASES = [
    # seed, lens, H, Hkv, D, Dv, bs
    (11, [5], 1, 1, 8, 8, 1),
    (12, [17, 1, 9], 2, 1, 16, 8, 2),
    (13, [40, 33], 4, 2, 8, 12, 8),
    (14, [3, 0, 26], 2, 2, 16, 16, 8),
    (15, [31], 6, 3, 4, 4, 4),
]


def pin_worked_example(o):
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "worked_example_offsets.txt"))
            if ln.strip() and not ln.startswith("#")]
    expected = [int(r[1]) for r in rows]
    got = o.token_offsets(np.array([[40, 30]], dtype=np.int32), [16], 8, 1, 1)
    assert got[0].tolist() == expected, got


def pin_offsets_bruteforce(o):
    rng = np.random.default_rng(7)
    for bs in (1, 2, 4, 8, 16, 32):
        S, Hkv, D, x = 3, 2, 8, 4
        lens = rng.integers(0, 65, S)
        need = [-(-int(L) // bs) for L in lens]
        NB = sum(need) + 3
        perm = rng.permutation(NB)
        bt = np.full((S, max(need + [1])), -7, dtype=np.int32)
        pos = 0
        for s, n in enumerate(need):
            bt[s, :n] = perm[pos:pos + n]
            pos += n
        cache = np.arange(NB * Hkv * (D // x) * bs * x, dtype=np.int64).reshape(NB, Hkv, D // x, bs, x)
        est = [st // 8 for st in cache.strides]
        off = o.token_offsets(bt, lens, bs, block_stride=est[0], slot_stride=est[3])
        flat = cache.reshape(-1)
        for s in range(S):
            L = int(lens[s])
            assert (off[s, L:] == -1).all()
            t = np.arange(L)
            for kvh in range(Hkv):
                for d in range(D):
                    want = cache[bt[s, t // bs], kvh, d // x, t % bs, d % x]
                    got = flat[off[s, :L] + kvh * est[1] + (d // x) * est[2] + d % x]
                    assert np.array_equal(want, got), (bs, s, kvh, d)
        # the same lists in CSR form give the same offsets
        ind = np.zeros(S + 1, dtype=np.int32)
        ind[1:] = np.cumsum(need)
        flatp = np.concatenate([bt[s, :need[s]] for s in range(S)] + [np.zeros(1, np.int32)])
        off2 = o.token_offsets(flatp.astype(np.int32), lens, bs, est[0], est[3], indptr=ind)
        assert np.array_equal(off, off2)


def pin_attention_bruteforce(o):
    for seed, lens, H, Hkv, D, Dv, bs in TINY_CASES:
        w = workloads.custom(seed=seed, seq_lens=lens, num_heads=H, num_kv_heads=Hkv, head_size=D,
                             v_head_size=Dv, block_size=bs, dtype="f32", poison=True)
        got = _run(o, w)
        want = _brute(w)
        assert np.abs(got - want).max() < 1e-12, (seed, np.abs(got - want).max())


def pin_attention_sdpa(o):
    """Identity block table + contiguous cache: the result must equal torch's
    scaled_dot_product_attention (float64, GQA by enable_gqa)."""
    gen = torch.Generator().manual_seed(3)
    for (S, H, Hkv, D, Dv, bs, nblk, lens) in [(2, 4, 2, 16, 8, 4, 5, [20, 13]),
                                               (1, 8, 1, 8, 8, 8, 3, [24]),
                                               (3, 3, 3, 4, 4, 2, 4, [1, 8, 5])]:
        x = 4
        NB = S * nblk
        kc = torch.randn(NB, Hkv, D // x, bs, x, generator=gen, dtype=torch.float32)
        vc = torch.randn(NB, Hkv, Dv, bs, generator=gen, dtype=torch.float32)
        q = torch.randn(S, H, D, generator=gen, dtype=torch.float32)
        bt = torch.arange(NB, dtype=torch.int32).reshape(S, nblk)
        scale = 0.37
        got = o.attention(q.numpy(), kc.numpy(), vc.numpy(), bt.numpy(), np.array(lens), scale)
        for s in range(S):
            L = lens[s]
            blocks = kc.double()[s * nblk:(s + 1) * nblk]
            K = blocks.permute(1, 0, 3, 2, 4).reshape(Hkv, nblk * bs, D)[:, :L]
            V = vc.double()[s * nblk:(s + 1) * nblk].permute(1, 0, 3, 2).reshape(Hkv, nblk * bs, Dv)[:, :L]
            ref = torch.nn.functional.scaled_dot_product_attention(
                q.double()[s][None, :, None, :], K[None].contiguous(), V[None].contiguous(),
                scale=scale, enable_gqa=True)[0, :, 0, :]
            assert np.abs(got[s] - ref.numpy()).max() < 1e-12, s


def pin_closed_forms(o):
    w = workloads.custom(seed=21, seq_lens=[37, 1, 12], num_heads=4, num_kv_heads=2, head_size=16,
                         v_head_size=8, block_size=4, dtype="f32", poison=True)
    # scale 0: every token weighs the same, the output is the mean V row
    got = _run(o, w, scale=0.0)
    vc = _np(w.value_cache).astype(np.float64)
    for s in range(3):
        L = int(w.seq_lens[s])
        t = np.arange(L)
        pb = w.block_tables.numpy()[s, t // 4]
        for h in range(4):
            mean = vc[pb, h // 2, :, t % 4].mean(axis=0)
            assert np.abs(got[s, h] - mean).max() < 1e-13
    # length 1: exactly that token's V row
    got = _run(o, w)
    pb = int(w.block_tables[1, 0])
    for h in range(4):
        assert np.array_equal(got[1, h], vc[pb, h // 2, :, 0]), h
    # constant V rows: the output is that constant
    w2 = workloads.custom(seed=22, seq_lens=[29, 7], num_heads=2, num_kv_heads=1, head_size=8,
                          block_size=8, dtype="f32")
    w2.value_cache[:] = 1.25
    got = _run(o, w2)
    assert np.abs(got - 1.25).max() < 1e-14
    # one-hot limit: a key much closer to q than the others takes all the weight
    w3 = workloads.custom(seed=23, seq_lens=[19], num_heads=1, num_kv_heads=1, head_size=8,
                          block_size=4, dtype="f32")
    tstar = 11
    blk, slot = int(w3.block_tables[0, tstar // 4]), tstar % 4
    w3.key_cache[blk, 0, :, slot, :] = (60.0 * w3.query[0, 0]).reshape(2, 4)
    got = _run(o, w3, scale=1.0)
    assert np.abs(got[0, 0] - _np(w3.value_cache)[blk, 0, :, slot]).max() < 1e-9


def pin_block_permutation(o):
    w = workloads.custom(seed=31, seq_lens=[23, 40], num_heads=2, num_kv_heads=1, head_size=8,
                         block_size=4, dtype="f32", num_blocks=30)
    base = _run(o, w)
    perm = torch.randperm(30, generator=torch.Generator().manual_seed(5))
    kc2 = torch.empty_like(w.key_cache)
    vc2 = torch.empty_like(w.value_cache)
    kc2[perm] = w.key_cache
    vc2[perm] = w.value_cache
    bt2 = perm[w.block_tables.long()].to(torch.int32)
    got = o.attention(w.query.numpy(), kc2.numpy(), vc2.numpy(), bt2.numpy(), w.seq_lens.numpy(), w.scale)
    assert np.array_equal(base, got)


def _brute_partials(w, lens_of_split):
    """Per-split (m, l, normalised output) by brute force over each split range."""
    q = _np(w.query).astype(np.float64)
    kc = _np(w.key_cache).astype(np.float64)
    vc = _np(w.value_cache).astype(np.float64)
    S, H, D = q.shape
    bs = w.block_size
    G = H // w.num_kv_heads
    res = {}
    for s in range(S):
        L = int(w.seq_lens[s])
        ln = lens_of_split[s]
        p = 0
        while p * ln < L:
            t = np.arange(p * ln, min((p + 1) * ln, L))
            pb = w.block_tables.numpy()[s, t // bs]
            for h in range(H):
                K = kc[pb, h // G, :, t % bs, :].reshape(len(t), D)
                V = vc[pb, h // G, :, t % bs]
                z = w.scale * (K @ q[s, h])
                m = z.max()
                e = np.exp(z - m)
                res[(s, h, p)] = (m, e.sum(), (e @ V) / e.sum())
            p += 1
    return res


def pin_partitions(o):
    w = workloads.custom(seed=41, seq_lens=[70, 1, 0, 130, 64], num_heads=4, num_kv_heads=2,
                         head_size=8, v_head_size=4, block_size=4, dtype="f32", poison=True)
    full = _run(o, w)
    args = (_np(w.query), _np(w.key_cache), _np(w.value_cache), w.block_tables.numpy(),
            w.seq_lens.numpy(), w.scale)
    for P in (1, 3, 8, 64, 512):
        npart = -(-130 // P)
        tmp, ml, es = o.partials(*args, max_num_parts=npart + 1, partition_size=P)
        want = _brute_partials(w, [P] * 5)
        for (s, h, p), (m, l, out) in want.items():
            assert abs(ml[s, h, p] - m) < 1e-12 and abs(es[s, h, p] - l) < 1e-9 * l
            assert np.abs(tmp[s, h, p] - out).max() < 1e-12
        for s in range(5):
            n = -(-max(int(w.seq_lens[s]), 0) // P)
            assert (ml[s, :, n:] == -np.inf).all() and (es[s, :, n:] == 0).all()
            assert np.isnan(tmp[s, :, n:]).all()
        merged = o.reduce(tmp, ml, es, w.seq_lens.numpy(), partition_size=P)
        assert np.abs(merged - full).max() < 1e-12, P
    # split counts (heuristic style): length rounded up to the 64-token granule
    for ns in ([1, 1, 1, 1, 1], [2, 5, 3, 3, 7], [9, 9, 9, 9, 9]):
        maxp = 4
        tmp, ml, es = o.partials(*args, max_num_parts=maxp, num_splits=np.array(ns))
        lens = []
        for s in range(5):
            n = min(max(ns[s], 1), maxp)
            L = max(int(w.seq_lens[s]), 1)
            per_split = math.ceil(L / n)
            lens.append(math.ceil(per_split / 64) * 64)
        want = _brute_partials(w, lens)
        for (s, h, p), (m, l, out) in want.items():
            assert abs(ml[s, h, p] - m) < 1e-12 and np.abs(tmp[s, h, p] - out).max() < 1e-12
        merged = o.reduce(tmp, ml, es, w.seq_lens.numpy(), num_splits=np.array(ns))
        assert np.abs(merged - full).max() < 1e-12, ns


def pin_reduce_closed_form(o):
    # two partitions: m = (0, ln 3), l = (2, 1) -> weights proportional to 2 and 3
    a = np.array([1.0, -2.0, 0.5])
    b = np.array([4.0, 0.0, -1.0])
    tmp = np.stack([a, b])[None, None]
    ml = np.array([[[0.0, math.log(3.0)]]])
    es = np.array([[[2.0, 1.0]]])
    got = o.reduce(tmp, ml, es, np.array([1024]), partition_size=512)
    assert np.abs(got[0, 0] - (2 * a + 3 * b) / 5).max() < 1e-15
    # one partition: the merge returns its row unchanged ("redundant but correct")
    got = o.reduce(tmp[:, :, :1], ml[:, :, :1] + 7.0, es[:, :, :1], np.array([300]), partition_size=512)
    assert np.array_equal(got[0, 0], a)
    # unused partitions past the sequence are never read, even when NaN
    tmp2 = np.concatenate([tmp, np.full((1, 1, 1, 3), np.nan)], axis=2)
    ml2 = np.concatenate([ml, np.full((1, 1, 1), np.nan)], axis=2)
    es2 = np.concatenate([es, np.full((1, 1, 1), np.nan)], axis=2)
    got = o.reduce(tmp2, ml2, es2, np.array([1024]), partition_size=512)
    assert np.abs(got[0, 0] - (2 * a + 3 * b) / 5).max() < 1e-15


def pin_num_kv_splits(o):
    for ln in open(os.path.join(GOLDEN, "num_kv_splits_pins.txt")):
        if not ln.strip() or ln.startswith("#"):
            continue
        f = [c.strip() for c in ln.split("|")]
        name = f[0]
        lens = [int(v) for v in f[1].split(",")]
        g, hq, hk, mx, cores = (int(v) for v in f[2:7])
        want = [int(v) for v in f[7].split(",")]
        got = o.num_kv_splits(lens, g, hq, hk, mx, cores)
        assert got.tolist() == want, (name, got.tolist(), want)
    # lengths <= 0 count as 1
    assert o.num_kv_splits([0, 16], 1, 2, 2, 8, 256).tolist() == \
        o.num_kv_splits([1, 16], 1, 2, 2, 8, 256).tolist()


def pin_page_indices(o):
    rng = np.random.default_rng(9)
    R, maxB = 6, 50
    big = rng.integers(0, 10**6, (maxB, R)).astype(np.int32)
    for bt in (big.T.copy(), big.T):  # contiguous, then a transposed view (stride1 != 1)
        n = rng.integers(0, maxB + 1, R)
        n[2] = 0
        cu = np.zeros(R + 1, dtype=np.int32)
        cu[1:] = np.cumsum(n)
        got = o.page_indices(bt, cu)
        want = np.concatenate([np.asarray(bt)[r, :n[r]] for r in range(R)])
        assert np.array_equal(got, want)
    assert o.page_indices(np.zeros((0, 4), np.int32), np.zeros(1, np.int32)).size == 0


def pin_mla(o):
    w = workloads.mla_custom(seed=51, seq_lens=[9, 30, 1], num_heads=4, head_size=24, v_head_size=16)
    lat = w.latent.float().numpy().astype(np.float64)
    q = w.query.float().numpy().astype(np.float64)
    pages = w.block_tables.numpy()
    got = o.attention(_np(w.query), _np(w.key_cache), _np(w.value_cache), pages,
                      w.seq_lens.numpy(), w.scale)
    for s in range(3):
        L = int(w.seq_lens[s])
        rows = lat[pages[s, :L]]
        for h in range(4):
            z = w.scale * rows @ q[s, h]
            want = scipy.special.softmax(z) @ rows[:, :16]
            assert np.abs(got[s, h] - want).max() < 1e-12
    # the same pages as a flat CSR list (page size 1)
    cu = w.cu_num_blocks.numpy()
    flat = o.page_indices(pages, cu)
    got2 = o.attention(_np(w.query), _np(w.key_cache), _np(w.value_cache), flat,
                       w.seq_lens.numpy(), w.scale, indptr=cu)
    assert np.array_equal(got, got2)


def _md(o, c, **kw):
    """Run the oracle's decode metadata on a MetadataCase (numpy views)."""
    args = dict(seq_lens=c.seq_lens.numpy(), req_to_token=c.req_to_token.numpy(),
                req_pool_indices=c.req_pool_indices.numpy(), max_seq_pages=c.max_seq_pages,
                page_size=c.page_size, seq_len_delta=c.seq_len_delta,
                full_to_swa=None if c.full_to_swa is None else c.full_to_swa.numpy())
    args.update(kw)
    return o.decode_metadata(**args)


def pin_metadata_roundtrip(o):
    """Token slots laid out page by page from a block table: reading every
    page_size-th slot and dividing by the page size gives the block table
    back (the page table's meaning), for shuffled pool rows and strided
    inputs. Columns past a row's pages hold its stale slots, divided."""
    for ps in (1, 4, 16):
        c = workloads.metadata_case(seed=60 + ps, seq_lens=[37, 1, 0, 64, 19], page_size=ps,
                                    seq_len_delta=1)
        _, _, pt, swa = _md(o, c)
        assert swa is None
        rows = c.req_pool_indices.numpy()
        rtt = c.req_to_token.numpy()
        for b, L in enumerate(c.seq_lens.tolist()):
            n = (L + ps - 1) // ps
            assert np.array_equal(pt[b, :n], c.block_tables.numpy()[b, :n]), (ps, b)
            for col in range(n, c.max_seq_pages):  # stale slots, floor-divided
                assert pt[b, col] == math.floor(int(rtt[rows[b], col * ps]) / ps)
        # strided views of every input give the same tables
        big = np.zeros((rtt.shape[0], 2 * rtt.shape[1]), np.int32)
        big[:, ::2] = rtt
        sl = np.zeros(2 * c.batch, np.int64)
        sl[::2] = c.seq_lens.numpy()
        rp = np.zeros(3 * c.batch, np.int64)
        rp[::3] = rows
        _, _, pt2, _ = _md(o, c, req_to_token=big[:, ::2], seq_lens=sl[::2], req_pool_indices=rp[::3])
        assert np.array_equal(pt2, pt)


def pin_metadata_prefix(o):
    """cache_seqlens = seq_len + delta; cu_seqlens_k starts at 0, steps by
    cache_seqlens and ends at their sum; int32 two's complement wrap."""
    c = workloads.metadata_case(seed=70, seq_lens=[5, 0, 9, 1, 300], page_size=8, seq_len_delta=1)
    cs, cu, _, _ = _md(o, c)
    want = c.seq_lens.numpy() + 1
    assert np.array_equal(cs, want)
    assert cu[0] == 0 and np.array_equal(np.diff(cu), want) and cu[-1] == want.sum()
    cs, cu, _, _ = _md(o, c, seq_len_delta=-1)
    assert np.array_equal(cs, c.seq_lens.numpy() - 1)
    # 2^31 - 1 + 1 wraps to -2^31; the running sum wraps the same way
    big = np.array([2**31 - 1, 2**31 - 2], np.int64)
    cs, cu, _, _ = o.decode_metadata(big, np.zeros((2, 4), np.int32), np.array([0, 1], np.int64),
                                     0, 4, seq_len_delta=1)
    assert cs.tolist() == [-2**31, 2**31 - 1]
    assert cu.tolist() == [0, -2**31, -1]


def pin_metadata_floor(o):
    """Negative slots divide toward minus infinity: floor(-5/4) = -2,
    floor(-1/4) = -1, floor(-4/4) = -1, floor(3/4) = 0, floor(8/4) = 2."""
    slots = [-5, -1, -4, 3, 8]
    rtt = np.zeros((1, 4 * len(slots)), np.int32)
    rtt[0, ::4] = slots
    _, _, pt, _ = o.decode_metadata(np.array([20], np.int64), rtt, np.array([0], np.int64),
                                    len(slots), 4)
    assert pt[0].tolist() == [-2, -1, -1, 0, 2]


def pin_metadata_swa(o):
    """The SWA table follows the map from full-pool slots to SWA slots: with
    the identity map it equals the page table; with a map that relabels whole
    pages by sigma it is sigma applied to the page table."""
    for ps in (1, 8):
        c = workloads.metadata_case(seed=80 + ps, seq_lens=[33, 2, 17], page_size=ps, swa=True)
        _, _, pt, swa = _md(o, c)
        assert np.array_equal(swa, c.swa_block_of.numpy()[pt])
        nslots = c.full_to_swa.shape[0]
        _, _, pt2, swa2 = _md(o, c, full_to_swa=np.arange(nslots, dtype=np.int32))
        assert np.array_equal(swa2, pt2) and np.array_equal(pt2, pt)


def pin_metadata_empty(o):
    """An empty batch still writes cu_seqlens_k[0] = 0; max_seq_pages = 0
    leaves the page table untouched and still fills the lengths."""
    cs, cu, pt, _ = o.decode_metadata(np.zeros(0, np.int64), np.zeros((1, 4), np.int32),
                                      np.zeros(0, np.int64), 4, 4)
    assert cu.tolist() == [0] and cs.size == 0 and pt.size == 0
    c = workloads.metadata_case(seed=90, seq_lens=[3, 4], page_size=2, seq_len_delta=2)
    cs, cu, pt, _ = _md(o, c, max_seq_pages=0)
    assert cs.tolist() == [5, 6] and cu.tolist() == [0, 5, 11] and pt.shape == (2, 0)


def pin_spec_page_table(o):
    """Each destination row is the concatenation of its request's page-table
    prefix and its draft row's prefix (numpy concatenate), nothing written
    past the total; with one draft token and empty drafts it is the plain
    page table, with empty request rows the draft table."""
    rng = np.random.default_rng(21)
    bs, R, LA, LB = 5, 3, 37, 11
    a = rng.integers(0, 10**6, (bs, LA)).astype(np.int32)
    bt = rng.integers(0, 10**6, (LB, bs * R)).astype(np.int32)
    for b in (bt.T.copy(), bt.T):  # contiguous, then a transposed view
        la = rng.integers(0, LA + 1, bs).astype(np.int32)
        lb = rng.integers(0, LB + 1, bs * R).astype(np.int32)
        la[1], lb[4] = 0, 0
        out = o.swa_spec_page_table(a, b, la, lb, R, fill=-9)
        for m in range(bs * R):
            n = la[m // R] + lb[m]
            want = np.concatenate([a[m // R, :la[m // R]], np.asarray(b)[m, :lb[m]]])
            assert np.array_equal(out[m, :n], want), m
            assert (out[m, n:] == -9).all(), m
    out = o.swa_spec_page_table(a, np.zeros((bs, 4), np.int32), np.full(bs, 20, np.int32),
                                np.zeros(bs, np.int32), 1, fill=-9)
    assert np.array_equal(out[:, :20], a[:, :20]) and (out[:, 20:] == -9).all()
    out = o.swa_spec_page_table(a, bt.T.copy(), np.zeros(bs, np.int32), np.full(bs * R, LB, np.int32),
                                R, fill=-9)
    assert np.array_equal(out[:, :LB], bt.T) and (out[:, LB:] == -9).all()


def pin_spec_page_table_widths(o):
    """Lengths past a table's width read zeros there (the masked loads), and
    the destination stops at LEN_A + LEN_B columns."""
    a = np.arange(1, 5, dtype=np.int32)[None, :]          # LEN_A = 4
    b = np.arange(101, 104, dtype=np.int32)[None, :]      # LEN_B = 3
    out = o.swa_spec_page_table(a, b, np.array([6], np.int32), np.array([2], np.int32), 1, fill=-9)
    assert out.tolist() == [[1, 2, 3, 4, 0, 0, 101]]
    out = o.swa_spec_page_table(a, b, np.array([2], np.int32), np.array([1], np.int32), 1, fill=-9)
    assert out.tolist() == [[1, 2, 101, -9, -9, -9, -9]]


def _fp8_values(codes):
    """float32 values of OCP E4M3 codes (torch's float8_e4m3fn)."""
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def pin_fp8_dequant(o):
    """fp8 caches: one token of 256 value codes comes back as v_scale times
    the E4M3 value of each code (NaN codes included); keys: with a one-hot
    query per head the max logit is scale * k_scale * E4M3(code)."""
    codes = np.arange(256, dtype=np.uint8)
    # values: Dv = 256, one token, one block
    vc = codes.reshape(1, 1, 256, 1)
    kc = np.full((1, 1, 1, 1, 16), 0x38, np.uint8)  # keys 1.0
    q = np.zeros((1, 1, 16), np.float32)
    out = o.attention(q, kc, vc, np.zeros((1, 1), np.int32), [1], 1.0, k_scale=0.5, v_scale=0.25)
    want = 0.25 * _fp8_values(codes).astype(np.float64)
    assert np.array_equal(np.isnan(out[0, 0]), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(out[0, 0][fin], want[fin])
    # keys: 16 heads over one kv head, block s holds codes 16s .. 16s+15 of token 0 of seq s
    finite = codes[(codes & 0x7F) != 0x7F]
    n = len(finite) // 16
    kc = finite[:16 * n].reshape(n, 1, 1, 1, 16)
    vc = np.full((n, 1, 1, 1), 0x38, np.uint8)
    q = np.tile(np.eye(16, dtype=np.float32)[None], (n, 1, 1))
    pages = np.arange(n, dtype=np.int32).reshape(n, 1)
    _, ml, _ = o.partials(q, kc, vc, pages, np.ones(n, np.int32), 2.0, 1, partition_size=64,
                          k_scale=0.75, v_scale=1.0)
    want = 2.0 * 0.75 * _fp8_values(finite[:16 * n]).astype(np.float64).reshape(n, 16)
    assert np.array_equal(ml[:, :, 0], want)


def pin_alibi_geometric(o):
    """ALiBi with zero scores: the weights of tokens 0..L-1 are r^(L-1-t)
    normalised, r = exp(-slope) (a geometric series), the max logit is the
    bias of the best token (0 at t = L-1 for a positive slope, -slope*(L-1)
    at t = 0 for a negative one) and the exp sum (1 - r^L) / (1 - r)."""
    L, H = 7, 4
    slopes = np.array([0.5, 1.0, 0.125, -0.25], np.float32)
    q = np.zeros((1, H, 4), np.float32)
    kc = np.ones((L, 1, 1, 1, 4), np.float32)
    vc = np.zeros((L, 1, L, 1), np.float32)
    for t in range(L):
        vc[t, 0, t, 0] = 1.0  # V_t = e_t
    pages = np.arange(L, dtype=np.int32)[None]
    out = o.attention(q, kc, vc, pages, [L], 1.0, alibi=slopes)
    _, ml, es = o.partials(q, kc, vc, pages, [L], 1.0, 1, partition_size=64, alibi=slopes)
    for h, sl in enumerate(slopes.astype(np.float64)):
        r = math.exp(-sl)
        w = np.array([r ** (L - 1 - t) for t in range(L)]) * (1 - r) / (1 - r ** L)
        assert np.allclose(out[0, h], w, rtol=1e-12, atol=0), h
        m = 0.0 if sl >= 0 else -sl * (L - 1)
        assert abs(ml[0, h, 0] - m) < 1e-12, h
        assert abs(es[0, h, 0] * math.exp(m) - (1 - r ** L) / (1 - r)) < 1e-9, h


def pin_alibi_zero_slopes(o):
    """Zero slopes leave the plain result unchanged (bit for bit)."""
    w = workloads.custom(seed=33, seq_lens=[9, 30], num_heads=4, num_kv_heads=2, head_size=16,
                         block_size=4)
    a = (_np(w.query), _np(w.key_cache), _np(w.value_cache), w.block_tables.numpy(),
         w.seq_lens.numpy(), w.scale)
    assert np.array_equal(o.attention(*a), o.attention(*a, alibi=np.zeros(4, np.float32)))


ALL_PINS = [pin_worked_example, pin_offsets_bruteforce, pin_attention_bruteforce,
            pin_attention_sdpa, pin_closed_forms, pin_block_permutation, pin_partitions,
            pin_reduce_closed_form, pin_num_kv_splits, pin_page_indices, pin_mla,
            pin_metadata_roundtrip, pin_metadata_prefix, pin_metadata_floor, pin_metadata_swa,
            pin_metadata_empty, pin_spec_page_table, pin_spec_page_table_widths,
            pin_fp8_dequant, pin_alibi_geometric, pin_alibi_zero_slopes]
