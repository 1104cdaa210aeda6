"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import paged_attention_decode_tables_amd as pad
from paged_attention_decode_tables_amd import workloads

DEV = "cuda:0"

# Tolerances on fp32 outputs against the float64 oracle (max abs error):
# 2e-3 for fp32 caches, 1e-2 for fp16/bf16 caches.
ATOL = {torch.float32: 2e-3, torch.float16: 1e-2, torch.bfloat16: 1e-2}
# exp_sums relative tolerance: the matrix-core path rounds each probability
# to the cache type before the P.V product and sums the rounded values
# (relative rounding <= 2^-9 for bf16, 2^-11 for f16); the vector path sums
# fp32 values.
LTOL = {torch.float32: 1e-5, torch.float16: 2e-3, torch.bfloat16: 4e-3}


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def _cache_np(t: torch.Tensor) -> np.ndarray:
    """fp8 caches stay uint8 codes (the oracle decodes them); others fp32."""
    return t.cpu().numpy() if t.dtype == torch.uint8 else np64(t)


def oracle_args(w: workloads.Workload):
    return (np64(w.query), _cache_np(w.key_cache), _cache_np(w.value_cache),
            w.block_tables.numpy(), w.seq_lens.numpy(), w.scale)


def oracle_kw(w: workloads.Workload) -> dict:
    """The variant arguments (ALiBi slopes, fp8 scales) of the oracle calls."""
    return dict(alibi=None if w.alibi_slopes is None else w.alibi_slopes.cpu().numpy(),
                k_scale=w.k_scale, v_scale=w.v_scale)


def tolerances(w: workloads.Workload, kernel: str = "auto"):
    """(tmp/output atol, exp-sum rtol). FP8 codes decode exactly; on the
    vector kernel everything after is fp32 (the fp32 bounds), on the
    matrix-core kernel the probabilities are rounded to the query's 16-bit
    type as for 16-bit caches (that type's bounds)."""
    if w.kv_dtype is not None and (kernel == "valu" or w.dtype == torch.float32):
        return ATOL[torch.float32], LTOL[torch.float32]
    return ATOL[w.dtype], LTOL[w.dtype]


# Split outputs stored in a 16-bit workspace are rounded to nearest even:
# relative error at most half an ulp (2^-9 bf16, 2^-11 f16). Phase 2 forms a
# convex combination of the stored rows, so the merged output moves by at
# most that much of the largest stored value.
TMP_HALF_ULP = {torch.float32: 0.0, torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -9}


def workspace(w: workloads.Workload, max_parts: int, device=DEV, tmp_dtype=torch.float32):
    S, H, Dv = w.num_seqs * w.num_group, w.num_heads, w.v_head_size
    nan = float("nan")
    tmp = torch.full((S, H, max_parts, Dv), nan, dtype=tmp_dtype, device=device)
    ml = torch.full((S, H, max_parts), nan, dtype=torch.float32, device=device)
    es = torch.full((S, H, max_parts), nan, dtype=torch.float32, device=device)
    return tmp, ml, es


def max_parts_for(w: workloads.Workload, partition_size: int) -> int:
    return max(1, math.ceil(max(w.max_seq_len, 1) / partition_size))


def run_gpu(w: workloads.Workload, *, partition_size=512, num_splits=None, max_parts=None,
            kernel="auto", out_dtype=torch.float32, csr=False, block_tables=None,
            tmp_dtype=torch.float32):
    """Phase 1 + phase 2 on the GPU. Returns (out, tmp, ml, es) on the CPU."""
    g = w.to(DEV)
    if max_parts is None:
        max_parts = max_parts_for(w, partition_size) if num_splits is None else 32
    tmp, ml, es = workspace(w, max_parts, tmp_dtype=tmp_dtype)
    ns = None if num_splits is None else torch.as_tensor(num_splits, dtype=torch.int32, device=DEV)
    R = w.num_seqs * w.num_group  # query rows
    bt = g.block_tables if block_tables is None else block_tables.to(DEV)
    indptr = None
    if csr:
        cu = torch.zeros(w.num_seqs + 1, dtype=torch.int32)
        nblk = [(max(int(L), 0) + w.block_size - 1) // w.block_size for L in w.seq_lens]
        cu[1:] = torch.cumsum(torch.tensor(nblk, dtype=torch.int32), 0)
        indptr = cu.to(DEV)
        flat = torch.full((max(int(cu[-1]), 1),), -1, dtype=torch.int32, device=DEV)
        pad.build_page_indices(flat, bt, indptr)
        bt = flat
    pad.paged_attn_decode(tmp, es, ml, g.query, g.key_cache, g.value_cache, bt, g.seq_lens,
                          w.scale, w.max_seq_len, partition_size=partition_size,
                          num_splits=ns, kv_indptr=indptr, kernel=kernel,
                          alibi_slopes=g.alibi_slopes, k_scale=w.k_scale, v_scale=w.v_scale,
                          num_group=w.num_group)
    out = torch.full((R, w.num_heads, w.v_head_size), float("nan"), dtype=out_dtype, device=DEV)
    pad.paged_attn_reduce(out, tmp, es, ml, g.seq_lens, partition_size=partition_size,
                          num_splits=ns, num_group=w.num_group)
    torch.cuda.synchronize()
    return out.cpu(), tmp.cpu(), ml.cpu(), es.cpu()


def split_lengths(w, partition_size, num_splits, max_parts):
    """Per-sequence split length under the documented split rule."""
    out = []
    for s in range(w.num_seqs):
        if num_splits is None:
            out.append(partition_size)
        else:
            n = min(max(int(num_splits[s]), 1), max_parts)
            L = max(int(w.seq_lens[s]), 1)
            out.append(math.ceil(math.ceil(L / n) / 64) * 64)
    return out


def check_partials(w, orc, tmp, ml, es, *, partition_size=512, num_splits=None, seqs=None,
                   kernel="auto"):
    """Compare the GPU phase-1 outputs with the oracle's per-split statistics."""
    P = tmp.shape[2]
    sub = w if seqs is None else subset(w, seqs)
    otmp, oml, oes = orc.partials(*oracle_args(sub), max_num_parts=P, partition_size=partition_size,
                                  num_splits=None if num_splits is None else
                                  np.asarray(num_splits)[seqs if seqs is not None else slice(None)],
                                  **oracle_kw(sub))
    idx = list(range(w.num_seqs)) if seqs is None else list(seqs)
    lens = split_lengths(sub, partition_size, None if num_splits is None else
                         np.asarray(num_splits)[idx], P)
    atol, ltol = tolerances(w, kernel)
    for i, s in enumerate(idx):
        L = int(w.seq_lens[s])
        n = 0 if L <= 0 else min(math.ceil(L / lens[i]), P)
        gm, ge, gt = ml[s].double().numpy(), es[s].double().numpy(), tmp[s].double().numpy()
        # empty splits: -inf / 0, tmp untouched (still NaN)
        assert np.all(gm[:, n:] == -np.inf) and np.all(ge[:, n:] == 0), (s, n)
        assert np.all(np.isnan(gt[:, n:])), s
        if n == 0:
            continue
        em = np.abs(gm[:, :n] - oml[i, :, :n])
        assert em.max() <= 2e-4 + 1e-5 * np.abs(oml[i, :, :n]).max(), (s, em.max())
        # the split's scores are fp32 numbers of magnitude up to |m| (ALiBi
        # makes |m| large far from the last token): each carries rounding of
        # about one ulp of |m|, and every exp(score - m) in the sum inherits it
        el = np.abs(ge[:, :n] / oes[i, :, :n] - 1.0)
        bound = ltol + 2.0 * 2.0 ** -23 * np.abs(oml[i, :, :n])
        assert (el <= bound).all(), (s, el.max(), float((el - bound).max()))
        et = np.abs(gt[:, :n] - otmp[i, :, :n]) - TMP_HALF_ULP[tmp.dtype] * np.abs(otmp[i, :, :n])
        assert et.max() <= atol, (s, et.max())


def subset(w: workloads.Workload, seqs) -> workloads.Workload:
    return w.subset(seqs)


def check_output(w, orc, out, seqs=None, kernel="auto", tmp=None):
    """Compare final outputs (any dtype) with the oracle's attention. tmp:
    the 16-bit workspace the output was merged from (its rounding bound is
    added: half an ulp of the largest stored value of each (row, head))."""
    idx = list(range(w.num_seqs)) if seqs is None else list(seqs)
    sub = w if seqs is None else subset(w, idx)
    ref = orc.attention(*oracle_args(sub), **oracle_kw(sub))
    got = out[idx].double().numpy()
    tol = tolerances(w, kernel)[0]
    if tmp is not None and TMP_HALF_ULP[tmp.dtype] > 0:
        rows = [r for s in idx for r in range(s * w.num_group, (s + 1) * w.num_group)]
        t = tmp[rows].double().abs().nan_to_num(0.0).amax(dim=(2, 3)).numpy()  # [rows, H]
        tol = tol + TMP_HALF_ULP[tmp.dtype] * t.reshape(got.shape[0], got.shape[1], 1)
    if out.dtype == torch.float32:
        err = np.abs(got - ref)
        assert np.all(err <= tol), float(np.max(err - tol))
    else:
        # output rounded to a 16-bit type: allow its half ulp on top
        half_ulp = 2.0 ** (-8 if out.dtype == torch.bfloat16 else -10)
        err = np.abs(got - ref) - half_ulp * np.abs(ref)
        assert np.all(err <= tol), float(np.max(err - tol))
    return float(np.abs(got - ref).max())
