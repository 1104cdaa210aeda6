"""Seeded synthetic inputs for split-KV PagedAttention decode.

This module draws inputs only: sequence lengths, block permutations, block
tables and N(0, 1) query/key/value tensors in the paged layouts. It contains
none of the method's arithmetic, and it is the one module that both the GPU
path (tests, benchmark) and the CPU oracle's callers share.

Draw order for every workload, from ``torch.Generator().manual_seed(seed)``:
lengths, then the physical-block permutation (consumed in order by sequence,
then logical block), then Q, then the key cache, then the value cache. Each
is drawn as fp32 N(0, 1) and cast to the workload dtype, so the bits are the
same wherever the same seed is used.

Layouts (from the kernel signatures of paged_attention_v2_triton.py):
  query        [S, H, D]
  key_cache    [NB, Hkv, D/x, block_size, x]   x = 16 // element_size
  value_cache  [NB, Hkv, Dv, block_size]
  block_tables [S, max_blocks] int32
The MLA-style workload stores one latent row of 576 values per page (page
size 1); its key cache is that row viewed as [NB, 1, 72, 1, 8] and its value
cache the first 512 values of the same row ([NB, 1, 512, 1], strides
(576, 576, 1, 1)).

FP8 caches (``custom(kv_cache="fp8" | "fp8_codes")``) are uint8 tensors of
E4M3 codes in the same layouts with x = 16. "fp8": N(0, 1) draws divided by
the scale and rounded to E4M3 by torch's float8_e4m3fn cast, the way a
serving engine quantises its cache; "fp8_codes": codes uniform over the 254
that are not NaN. ALiBi slopes, when asked for, are 2^(-8 i / H), i = 1..H
(no draw).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class Workload:
    name: str
    description: str
    dtype: torch.dtype
    seq_lens: torch.Tensor            # [S] int32
    block_tables: torch.Tensor        # [S, max_blocks] int32
    query: torch.Tensor               # [S, H, D]
    key_cache: torch.Tensor           # [NB, Hkv, D/x, bs, x]
    value_cache: torch.Tensor         # [NB, Hkv, Dv, bs] (may alias key_cache storage)
    scale: float
    num_heads: int
    num_kv_heads: int
    head_size: int
    v_head_size: int
    block_size: int
    x: int
    num_blocks: int
    partition_size: int = 512
    # Split-count heuristic inputs (None: fixed partition_size splits).
    max_kv_splits: Optional[int] = None
    device_core_count: Optional[int] = None
    # CSR page list inputs (MLA-style workload): indptr over block_tables rows.
    cu_num_blocks: Optional[torch.Tensor] = None
    latent: Optional[torch.Tensor] = None
    poison_block: Optional[int] = None
    notes: List[str] = field(default_factory=list)
    # FP8 E4M3 caches: kv_dtype torch.uint8 (None: caches hold dtype)
    kv_dtype: Optional[torch.dtype] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    alibi_slopes: Optional[torch.Tensor] = None  # fp32 [H]
    # query tokens per sequence: query rows s * num_group + j
    num_group: int = 1

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def elem_size(self) -> int:
        return torch.tensor([], dtype=self.dtype).element_size()

    @property
    def kv_elem_size(self) -> int:
        return 1 if self.kv_dtype is not None else self.elem_size

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.clamp(min=0).sum())

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0

    @property
    def kv_aliased(self) -> bool:
        return self.latent is not None

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of one decode step: every live token's K and V
        read once per kv head ((D + Dv) * elem), or D * elem when V aliases K."""
        per_tok = self.head_size if self.kv_aliased else self.head_size + self.v_head_size
        return self.total_tokens * self.num_kv_heads * per_tok * self.kv_elem_size

    def subset(self, seqs) -> "Workload":
        """The same workload restricted to some sequences (shares the caches)."""
        idx = torch.as_tensor(list(seqs), dtype=torch.long)
        ng = self.num_group
        rows = (idx[:, None] * ng + torch.arange(ng)[None, :]).reshape(-1)
        kw = {k: getattr(self, k) for k in self.__dataclass_fields__}
        kw["seq_lens"] = self.seq_lens[idx].clone()
        kw["block_tables"] = self.block_tables[idx].clone()
        kw["query"] = self.query[rows].clone()
        kw["cu_num_blocks"] = None
        kw["notes"] = list(self.notes)
        return Workload(**kw)

    def expanded(self) -> "Workload":
        """With query groups: one sequence per query row (row s * num_group + j
        gets sequence s's length and pages), num_group 1. Shares the caches."""
        ng = self.num_group
        kw = {k: getattr(self, k) for k in self.__dataclass_fields__}
        kw["seq_lens"] = self.seq_lens.repeat_interleave(ng)
        kw["block_tables"] = self.block_tables.repeat_interleave(ng, dim=0)
        kw["cu_num_blocks"] = None
        kw["num_group"] = 1
        kw["notes"] = list(self.notes)
        return Workload(**kw)

    def to(self, device) -> "Workload":
        kw = {k: getattr(self, k) for k in self.__dataclass_fields__}
        for k in ("seq_lens", "block_tables", "query", "cu_num_blocks", "alibi_slopes"):
            if kw[k] is not None:
                kw[k] = kw[k].to(device)
        if self.latent is not None:
            lat = self.latent.to(device)
            kw["latent"] = lat
            kw["key_cache"], kw["value_cache"] = _mla_views(lat, self.v_head_size)
        else:
            kw["key_cache"] = self.key_cache.to(device)
            kw["value_cache"] = self.value_cache.to(device)
        kw["notes"] = list(self.notes)
        return Workload(**kw)


def _mla_views(latent: torch.Tensor, dv: int):
    nb, d = latent.shape
    x = 16 // latent.element_size()
    k = latent.view(nb, 1, d // x, 1, x)
    v = torch.as_strided(latent, (nb, 1, dv, 1), (d, d, 1, 1))
    return k, v


def _randn(gen, shape, dtype):
    return torch.randn(shape, generator=gen, dtype=torch.float32).to(dtype)


FP8_NAN_CODE = 0x7F


def _fp8_cache(gen, shape, kind: str, scale: float) -> torch.Tensor:
    """uint8 E4M3 codes: "fp8" quantises N(0, 1) / scale (clamped to the
    largest finite value, 448), "fp8_codes" draws the 254 non-NaN codes
    uniformly."""
    if kind == "fp8":
        z = torch.randn(shape, generator=gen, dtype=torch.float32) / scale
        return z.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    if kind == "fp8_codes":
        c = torch.randint(0, 254, shape, generator=gen, dtype=torch.int64)
        c = c + (c >= FP8_NAN_CODE).to(torch.int64)  # skip 0x7F; 0xFF is past the range
        return c.to(torch.uint8)
    raise ValueError(f"unknown fp8 cache kind {kind}")


def alibi_slopes(num_heads: int) -> torch.Tensor:
    """fp32 [H]: 2^(-8 i / H), i = 1..H."""
    i = torch.arange(1, num_heads + 1, dtype=torch.float64)
    return torch.pow(2.0, -8.0 * i / num_heads).to(torch.float32)


def _assign_blocks(perm: torch.Tensor, nblocks: List[int], max_blocks: int, pad: int) -> torch.Tensor:
    """Block table rows filled from perm in order (seq, then logical block)."""
    bt = torch.full((len(nblocks), max(max_blocks, 1)), pad, dtype=torch.int32)
    pos = 0
    for s, n in enumerate(nblocks):
        bt[s, :n] = perm[pos:pos + n].to(torch.int32)
        pos += n
    return bt


def _blocks_needed(lens, bs):
    return [max(0, (int(L) + bs - 1) // bs) for L in lens]


def custom(*, seed: int, seq_lens, num_heads: int, num_kv_heads: int, head_size: int,
           v_head_size: Optional[int] = None, block_size: int, dtype="f32",
           num_blocks: Optional[int] = None, partition_size: int = 512,
           max_blocks: Optional[int] = None, poison: bool = False, name="custom",
           kv_cache: str = "same", k_scale: float = 1.0, v_scale: float = 1.0,
           alibi: bool = False, num_group: int = 1) -> Workload:
    """Standard layout workload with the given lengths (drawn in the standard
    order). kv_cache "fp8" / "fp8_codes" gives uint8 E4M3 caches (see the
    module docstring) with the given scales; alibi adds ALiBi slopes;
    num_group > 1 draws num_group query rows per sequence."""
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    fp8 = kv_cache != "same"
    esz = 1 if fp8 else torch.tensor([], dtype=dt).element_size()
    x = 16 // esz
    dv = v_head_size or head_size
    gen = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(seq_lens, dtype=torch.int32).clone()
    need = _blocks_needed(lens.tolist(), block_size)
    total = sum(need)
    nb = num_blocks if num_blocks is not None else total + (1 if poison else 0)
    if nb < total + (1 if poison else 0):
        raise ValueError("not enough physical blocks")
    perm = torch.randperm(nb, generator=gen)
    S = lens.shape[0]
    q = _randn(gen, (S * num_group, num_heads, head_size), dt)
    kshape, vshape = (nb, num_kv_heads, head_size // x, block_size, x), (nb, num_kv_heads, dv, block_size)
    if fp8:
        kc = _fp8_cache(gen, kshape, kv_cache, k_scale)
        vc = _fp8_cache(gen, vshape, kv_cache, v_scale)
    else:
        kc, vc = _randn(gen, kshape, dt), _randn(gen, vshape, dt)
    poison_block = int(perm[total]) if poison else None
    mb = max_blocks if max_blocks is not None else max(need + [1])
    bt = _assign_blocks(perm, need, mb, poison_block if poison else 0)
    w = Workload(name=name, description=name, dtype=dt, seq_lens=lens, block_tables=bt, query=q,
                 key_cache=kc, value_cache=vc, scale=1.0 / math.sqrt(head_size),
                 num_heads=num_heads, num_kv_heads=num_kv_heads, head_size=head_size,
                 v_head_size=dv, block_size=block_size, x=x, num_blocks=nb,
                 partition_size=partition_size, poison_block=poison_block,
                 kv_dtype=torch.uint8 if fp8 else None, k_scale=k_scale, v_scale=v_scale,
                 alibi_slopes=alibi_slopes(num_heads) if alibi else None, num_group=num_group)
    if poison:
        _poison(w, need)
    return w


def _poison(w: Workload, need: List[int]):
    """NaN in every unreferenced block and in the unused slots of each
    sequence's last block; block-table padding points at a NaN block."""
    used = torch.zeros(w.num_blocks, dtype=torch.bool)
    for s, n in enumerate(need):
        used[w.block_tables[s, :n].long()] = True
    nan = FP8_NAN_CODE if w.key_cache.dtype == torch.uint8 else float("nan")
    w.key_cache[~used] = nan
    w.value_cache[~used] = nan
    bs = w.block_size
    for s, n in enumerate(need):
        L = int(w.seq_lens[s])
        if n == 0 or L % bs == 0:
            continue
        last = int(w.block_tables[s, n - 1])
        w.key_cache[last, :, :, L % bs:, :] = nan
        w.value_cache[last, :, :, L % bs:] = nan


CONFIG_NAMES = {
    1: "tiny_f32",
    2: "mha_f16",
    3: "gqa_long_bf16",
    4: "gqa_skewed_bf16",
    5: "mla_bf16",
}


def _draw_lengths(cfg: int, gen: torch.Generator) -> torch.Tensor:
    """The first draw of configs 2-5: the sequence lengths (int32)."""
    if cfg == 2:
        return torch.randint(1, 2049, (32,), generator=gen, dtype=torch.int64).to(torch.int32)
    if cfg == 3:
        return torch.full((8,), 32768, dtype=torch.int32)
    if cfg == 4:
        z = torch.randn((256,), generator=gen, dtype=torch.float64)
        return torch.exp(math.log(1024.0) + 1.0 * z).round().clamp(1, 16384).to(torch.int32)
    if cfg == 5:
        return torch.randint(1024, 8193, (64,), generator=gen, dtype=torch.int64).to(torch.int32)
    raise ValueError(f"config {cfg} has no length draw")


def config_lengths(cfg: int) -> torch.Tensor:
    """Sequence lengths of config 2-5 alone (the same values config() draws)."""
    return _draw_lengths(cfg, torch.Generator().manual_seed(cfg))


# Scales of the fp8 forms of the standard workloads: N(0, 1) values land on
# codes of magnitude up to about 5 * 32 = 160, inside E4M3's 448.
FP8_WORKLOAD_SCALE = 1.0 / 32


def config(cfg: int, *, poison: bool = False, kv_cache: str = "same",
           alibi: bool = False, num_group: int = 1, mla_heads: int = 128) -> Workload:
    """The five reference workloads (seed = config number). Configs 2-4 also
    come with fp8 caches (kv_cache "fp8", both scales FP8_WORKLOAD_SCALE,
    name suffix "_kvfp8"), with ALiBi slopes (suffix "_alibi") and with
    num_group query tokens per sequence (configs 2-5, suffix "_qg<n>"; the
    query draw has num_group rows per sequence). Config 5 also comes with 64
    query heads over its latent head (mla_heads=64, suffix "_h64": the same
    lengths and draw order, a query of 64 heads)."""
    if kv_cache != "same" and cfg not in (2, 3, 4, 5):
        raise ValueError("fp8 caches are drawn for configs 2-5")
    if num_group != 1 and cfg not in (2, 3, 4, 5):
        raise ValueError("query groups are drawn for configs 2-5")
    if mla_heads != 128 and (cfg != 5 or mla_heads != 64):
        raise ValueError("config 5 alone comes with 64 heads")
    w = _config(cfg, poison=poison, kv_cache=kv_cache, num_group=num_group, mla_heads=mla_heads)
    if num_group != 1:
        w.name += f"_qg{num_group}"
    if alibi:
        w.alibi_slopes = alibi_slopes(w.num_heads)
        w.name += "_alibi"
    return w


def _config(cfg: int, *, poison: bool, kv_cache: str, num_group: int = 1, mla_heads: int = 128) -> Workload:
    gen = torch.Generator().manual_seed(cfg)
    kv = dict(kv_cache=kv_cache, num_group=num_group)
    if cfg == 1:
        # 2 seqs, lengths 16 and 13, block size 8, 64 physical blocks; seq 0
        # uses the block table [40, 30] of the Triton issue 2522 example, seq 1
        # two distinct random blocks from the other 62.
        lens = torch.tensor([16, 13], dtype=torch.int32)
        others = torch.tensor([b for b in range(64) if b not in (40, 30)], dtype=torch.int64)
        pick = others[torch.randperm(62, generator=gen)[:2]]
        bt = torch.tensor([[40, 30], [int(pick[0]), int(pick[1])]], dtype=torch.int32)
        dt, H, Hkv, D, bs, nb = torch.float32, 2, 2, 64, 8, 64
        x = 4
        q = _randn(gen, (2, H, D), dt)
        kc = _randn(gen, (nb, Hkv, D // x, bs, x), dt)
        vc = _randn(gen, (nb, Hkv, D, bs), dt)
        w = Workload(name=CONFIG_NAMES[1], description="tiny paged decode fp32", dtype=dt,
                     seq_lens=lens, block_tables=bt, query=q, key_cache=kc, value_cache=vc,
                     scale=1.0 / math.sqrt(D), num_heads=H, num_kv_heads=Hkv, head_size=D,
                     v_head_size=D, block_size=bs, x=x, num_blocks=nb)
        if poison:
            used = set(bt.flatten().tolist())
            w.poison_block = next(b for b in range(nb) if b not in used)
            _poison(w, [2, 2])
        return w
    if cfg == 2:
        lens = _draw_lengths(2, gen)
        return _standard(gen, CONFIG_NAMES[2], "MHA decode fp16", lens, H=32, Hkv=32, D=128,
                         bs=16, dt=torch.float16, nb=8192, poison=poison, **kv)
    if cfg == 3:
        lens = _draw_lengths(3, gen)
        return _standard(gen, CONFIG_NAMES[3], "long-context GQA decode bf16", lens, H=64, Hkv=8,
                         D=128, bs=16, dt=torch.bfloat16, nb=20000, poison=poison, **kv)
    if cfg == 4:
        lens = _draw_lengths(4, gen)
        w = _standard(gen, CONFIG_NAMES[4], "skewed-batch GQA decode bf16", lens, H=32, Hkv=8,
                      D=128, bs=32, dt=torch.bfloat16, nb=None, poison=poison, **kv)
        w.max_kv_splits = 32
        w.device_core_count = 256
        return w
    if cfg == 5:
        return _mla(gen, poison=poison, num_group=num_group, kv_cache=kv_cache, H=mla_heads)
    raise ValueError(f"unknown config {cfg}")


def _standard(gen, name, desc, lens, *, H, Hkv, D, bs, dt, nb, poison, kv_cache="same",
              num_group=1):
    need = _blocks_needed(lens.tolist(), bs)
    total = sum(need)
    if nb is None:
        nb = total + (1 if poison else 0)
    perm = torch.randperm(nb, generator=gen)
    fp8 = kv_cache != "same"
    x = 16 if fp8 else 16 // torch.tensor([], dtype=dt).element_size()
    S = lens.shape[0]
    q = _randn(gen, (S * num_group, H, D), dt)
    if fp8:
        sc = FP8_WORKLOAD_SCALE
        kc = _fp8_cache(gen, (nb, Hkv, D // x, bs, x), kv_cache, sc)
        vc = _fp8_cache(gen, (nb, Hkv, D, bs), kv_cache, sc)
        name += "_kvfp8"
    else:
        kc = _randn(gen, (nb, Hkv, D // x, bs, x), dt)
        vc = _randn(gen, (nb, Hkv, D, bs), dt)
    poison_block = int(perm[total]) if poison else None
    bt = _assign_blocks(perm, need, max(need), poison_block if poison else 0)
    w = Workload(name=name, description=desc, dtype=dt, seq_lens=lens, block_tables=bt, query=q,
                 key_cache=kc, value_cache=vc, scale=1.0 / math.sqrt(D), num_heads=H,
                 num_kv_heads=Hkv, head_size=D, v_head_size=D, block_size=bs, x=x, num_blocks=nb,
                 poison_block=poison_block, kv_dtype=torch.uint8 if fp8 else None,
                 k_scale=FP8_WORKLOAD_SCALE if fp8 else 1.0,
                 v_scale=FP8_WORKLOAD_SCALE if fp8 else 1.0, num_group=num_group)
    if poison:
        _poison(w, need)
    return w


def _latent_rows(gen, nb, D, dt, kv_cache):
    """[nb, D] latent rows: N(0, 1) draws of the query's type, or (kv_cache
    "fp8") uint8 E4M3 codes of N(0, 1) / FP8_WORKLOAD_SCALE."""
    if kv_cache == "same":
        return _randn(gen, (nb, D), dt)
    return _fp8_cache(gen, (nb, D), kv_cache, FP8_WORKLOAD_SCALE)


def _poison_rows(latent, rows):
    """NaN in unused latent rows: the float NaN, or the E4M3 NaN code."""
    if latent.dtype == torch.uint8:
        latent[rows] = FP8_NAN_CODE
    else:
        latent[rows] = float("nan")


def _mla(gen, *, poison, num_group=1, kv_cache="same", H=128):
    S, D, Dv = 64, 576, 512
    lens = _draw_lengths(5, gen)
    total = int(lens.sum())
    nb = total + (1 if poison else 0)
    perm = torch.randperm(nb, generator=gen)
    dt = torch.bfloat16
    q = _randn(gen, (S * num_group, H, D), dt)
    latent = _latent_rows(gen, nb, D, dt, kv_cache)
    poison_block = int(perm[total]) if poison else None
    bt = _assign_blocks(perm, lens.tolist(), 8192, poison_block if poison else 0)
    cu = torch.zeros(S + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0).to(torch.int32)
    if poison:
        _poison_rows(latent, poison_block)
        used = torch.zeros(nb, dtype=torch.bool)
        used[perm[:total]] = True
        _poison_rows(latent, ~used)
    k, v = _mla_views(latent, Dv)
    fp8 = kv_cache != "same"
    sc = FP8_WORKLOAD_SCALE if fp8 else 1.0
    name = CONFIG_NAMES[5] + ("_h64" if H == 64 else "") + ("_kvfp8" if fp8 else "")
    return Workload(name=name, description="MLA-style decode bf16",
                    dtype=dt, seq_lens=lens, block_tables=bt, query=q, key_cache=k, value_cache=v,
                    scale=1.0 / math.sqrt(192.0), num_heads=H, num_kv_heads=1, head_size=D,
                    v_head_size=Dv, block_size=1, x=16 if fp8 else 8, num_blocks=nb, cu_num_blocks=cu,
                    latent=latent, poison_block=poison_block, num_group=num_group,
                    kv_dtype=torch.uint8 if fp8 else None, k_scale=sc, v_scale=sc)


def mla_custom(*, seed, seq_lens, num_heads=128, head_size=576, v_head_size=512, max_blocks=None,
               poison=False, num_group=1, dtype="bf16", kv_cache="same", k_scale=None,
               v_scale=None) -> Workload:
    """Smaller MLA-style workload (page size 1, V aliasing the first Dv values
    of K). kv_cache "fp8": the latent rows are E4M3 codes (k_scale and
    v_scale default to FP8_WORKLOAD_SCALE)."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(seq_lens, dtype=torch.int32).clone()
    S = lens.shape[0]
    total = int(lens.clamp(min=0).sum())
    nb = total + (1 if poison else 0)
    perm = torch.randperm(nb, generator=gen)
    dt = DTYPES[dtype] if isinstance(dtype, str) else dtype
    q = _randn(gen, (S * num_group, num_heads, head_size), dt)
    latent = _latent_rows(gen, nb, head_size, dt, kv_cache)
    poison_block = int(perm[total]) if poison else None
    mb = max_blocks or max(1, int(lens.max()))
    bt = _assign_blocks(perm, [max(0, int(L)) for L in lens], mb, poison_block if poison else 0)
    cu = torch.zeros(S + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens.clamp(min=0), 0).to(torch.int32)
    if poison:
        _poison_rows(latent, poison_block)
    k, v = _mla_views(latent, v_head_size)
    fp8 = kv_cache != "same"
    ks = (FP8_WORKLOAD_SCALE if k_scale is None else k_scale) if fp8 else 1.0
    vs = (FP8_WORKLOAD_SCALE if v_scale is None else v_scale) if fp8 else 1.0
    return Workload(name="mla_custom", description="MLA-style custom", dtype=dt, seq_lens=lens,
                    block_tables=bt, query=q, key_cache=k, value_cache=v,
                    scale=1.0 / math.sqrt(192.0), num_heads=num_heads, num_kv_heads=1,
                    head_size=head_size, v_head_size=v_head_size, block_size=1,
                    x=16 if fp8 else 16 // latent.element_size(), num_blocks=nb, cu_num_blocks=cu,
                    latent=latent, poison_block=poison_block, num_group=num_group,
                    kv_dtype=torch.uint8 if fp8 else None, k_scale=ks, v_scale=vs)


# ---------------------------------------------------------------------------
# Decode-metadata inputs (the step before the path): a request -> token-slot
# table of a KV pool, as a serving engine keeps it.
# ---------------------------------------------------------------------------
@dataclass
class MetadataCase:
    """Inputs of one decode-metadata call plus the block table they encode.

    ``req_to_token[req_pool_indices[b], t]`` is the pool slot of token t of
    request b: ``block_tables[b, t // page_size] * page_size + t % page_size``
    for t < seq_lens[b], and a stale slot (any earlier occupant's) beyond.
    ``full_to_swa`` (optional) maps every full-pool slot to a sliding-window
    pool slot, page by page: slot ``blk * page_size + o`` goes to
    ``swa_block_of[blk] * page_size + o``.
    """
    seq_lens: torch.Tensor          # int64 [B]
    req_to_token: torch.Tensor      # int32 [pool_rows, max_context]
    req_pool_indices: torch.Tensor  # int64 [B]
    block_tables: torch.Tensor      # int32 [B, max_pages]
    page_size: int
    max_seq_pages: int
    seq_len_delta: int
    full_to_swa: Optional[torch.Tensor] = None   # int32 [num_slots]
    swa_block_of: Optional[torch.Tensor] = None  # int64 [num_blocks]

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])


def metadata_case(*, seed: int, seq_lens, page_size: int, pool_rows: Optional[int] = None,
                  max_context: Optional[int] = None, seq_len_delta: int = 0, swa: bool = False,
                  max_seq_pages: Optional[int] = None) -> MetadataCase:
    """Seeded decode-metadata inputs. Draw order: pool row permutation, block
    permutation, stale slots, then the SWA block map."""
    gen = torch.Generator().manual_seed(seed)
    lens = torch.as_tensor(seq_lens, dtype=torch.int64).clone()
    B = lens.shape[0]
    ps = page_size
    need = [(max(0, int(L)) + ps - 1) // ps for L in lens]
    max_pages = max(need + [1])
    pool_rows = pool_rows or 2 * B + 3
    max_context = max_context or max_pages * ps
    assert pool_rows >= B and max_context >= max_pages * ps
    rows = torch.randperm(pool_rows, generator=gen)[:B].to(torch.int64)
    nblocks = sum(need) + 8
    perm = torch.randperm(nblocks, generator=gen)
    bt = _assign_blocks(perm, need, max_pages, 0)
    nslots = nblocks * ps
    # stale slots everywhere, then each request's live tokens
    rtt = torch.randint(0, nslots, (pool_rows, max_context), generator=gen, dtype=torch.int64)
    for b in range(B):
        L = max(0, int(lens[b]))
        t = torch.arange(L)
        rtt[int(rows[b]), :L] = bt[b, t // ps].to(torch.int64) * ps + t % ps
    f2s = swa_of = None
    if swa:
        swa_of = torch.randperm(nblocks, generator=gen).to(torch.int64)
        s = torch.arange(nslots)
        f2s = (swa_of[s // ps] * ps + s % ps).to(torch.int32)
    if max_seq_pages is None:
        max_seq_pages = max_pages if B else 0
    return MetadataCase(seq_lens=lens, req_to_token=rtt.to(torch.int32), req_pool_indices=rows,
                        block_tables=bt, page_size=ps, max_seq_pages=int(max_seq_pages),
                        seq_len_delta=seq_len_delta, full_to_swa=f2s, swa_block_of=swa_of)
