#!/usr/bin/env python3
"""Benchmark: split-KV PagedAttention decode on one MI355X.

One step = one decode step of the whole hot path for a batch: phase 1
(paged_attn_decode) and phase 2 (paged_attn_reduce), plus num_kv_splits /
build_page_indices for the workloads that use them. Inputs are synthetic and
seeded (the workloads module) and already resident in HBM when timing starts.

Default workload: long-context GQA decode, bf16 -- 8 sequences x 32768
tokens, 64 query heads over 8 kv heads, head_dim 128, block size 16, 20000
physical blocks in random order, 512-token partitions (64 per sequence).

Prints one JSON line: KV read GB/s (value), microseconds per step, the
roofline of the dominant kernel (phase 1), the same GPU's plain read rate on
the workload's gather pattern and on contiguous memory (read_stream), the
same step captured into a HIP graph and replayed (graph_replay), and the
CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import paged_attention_decode_tables_amd as pad  # noqa: E402
from paged_attention_decode_tables_amd import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD published peak
METRIC = "paged-decode KV read GB/s (% of MI355X HBM peak) + µs/decode step"
KERNEL_SOURCES = {"mfma": "decode_mfma.hip", "valu": "decode_valu.hip", "mla": "decode_mla.hip"}
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_kind(w) -> str:
    """Which phase-1 kernel the library dispatches for workload `w` with the
    automatic kernel hint, from its shapes alone (the rule include/pagedattn.h
    states; the library's own answer, paged_attn_decode_kernel, needs device
    buffers and is what the measured step reports)."""
    group = w.num_heads // w.num_kv_heads
    low = w.dtype in (torch.float16, torch.bfloat16)
    if low and w.head_size == 576 and w.v_head_size == 512 and w.block_size == 1 \
            and group in (64, 128) and w.latent is not None:
        return "mla"
    cols = group * w.num_group  # (query token, head) pairs of a kv head
    if low and (cols >= 2 or w.kv_dtype is not None) and cols <= 16 and w.block_size >= 8 \
            and w.head_size in (64, 128):
        return "mfma"
    return "valu"


def balanced_workers(w: workloads.Workload, cus: int) -> int:
    """Token ranges for the latent-row kernel's balanced splits: one
    workgroup a compute unit at 128 heads per kv head, two at 64 (the
    library's rule for num_workers)."""
    return cus * (2 if w.num_heads // w.num_kv_heads == 64 else 1)


def kernel_source_hash(kind: str) -> str:
    path = os.path.join(ROOT, "paged_attention_decode_tables_amd", "csrc", KERNEL_SOURCES[kind])
    h = hashlib.sha256()
    for p in (path, os.path.join(os.path.dirname(path), "common.h")):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


class Step:
    """Device buffers and the launches of one decode step."""

    def __init__(self, w: workloads.Workload, out_dtype=torch.bfloat16, balanced_workers=0,
                 tmp_dtype=torch.float32, kernel="auto"):
        self.w = w
        self.kernel = kernel
        self.g = g = w.to("cuda")
        self.ns = None
        self.indptr = None
        # balanced splits: equal token ranges, one per worker (partition_size 0)
        self.workers = balanced_workers
        self.partition = 0 if balanced_workers else w.partition_size
        if w.max_kv_splits is not None:
            self.max_parts = w.max_kv_splits
            self.ns = torch.empty(w.num_seqs * w.num_group, dtype=torch.int32, device="cuda")
        else:
            self.max_parts = -(-w.max_seq_len // w.partition_size)
        if w.cu_num_blocks is not None:
            self.indptr = w.cu_num_blocks.to("cuda")
            self.flat = torch.empty(int(w.cu_num_blocks[-1]), dtype=torch.int32, device="cuda")
        S, H, Dv = w.num_seqs * w.num_group, w.num_heads, w.v_head_size  # query rows
        self.tmp = torch.empty((S, H, self.max_parts, Dv), dtype=tmp_dtype, device="cuda")
        self.ml = torch.empty((S, H, self.max_parts), dtype=torch.float32, device="cuda")
        self.es = torch.empty((S, H, self.max_parts), dtype=torch.float32, device="cuda")
        self.out = torch.empty((S, H, Dv), dtype=out_dtype, device="cuda")

    def pre(self):
        w, g = self.w, self.g
        if self.ns is not None:
            pad.num_kv_splits(self.ns, g.seq_lens, w.num_group, w.num_heads, w.num_kv_heads, w.max_kv_splits,
                              w.device_core_count)
        if self.indptr is not None:
            pad.build_page_indices(self.flat, g.block_tables, self.indptr)

    def _decode_args(self):
        w, g = self.w, self.g
        bt = self.flat if self.indptr is not None else g.block_tables
        return ((self.tmp, self.es, self.ml, g.query, g.key_cache, g.value_cache, bt, g.seq_lens, w.scale,
                 w.max_seq_len),
                dict(partition_size=self.partition, num_splits=self.ns, kv_indptr=self.indptr,
                     num_workers=self.workers, alibi_slopes=g.alibi_slopes, k_scale=w.k_scale,
                     v_scale=w.v_scale, num_group=w.num_group, kernel=self.kernel))

    def decode(self):
        args, kw = self._decode_args()
        pad.paged_attn_decode(*args, **kw)

    def kernel_kind(self) -> str:
        """The phase-1 kernel the library launches for this step."""
        args, kw = self._decode_args()
        return pad.paged_attn_decode_kernel(*args, **kw)

    def reduce(self):
        w, g = self.w, self.g
        pad.paged_attn_reduce(self.out, self.tmp, self.es, self.ml, g.seq_lens,
                              partition_size=self.partition, num_splits=self.ns,
                              num_group=w.num_group)

    def run(self):
        self.pre()
        self.decode()
        self.reduce()


def recorded_traffic(workload: str, kind: str, launches_kv_bytes: int):
    """HBM traffic per phase-1 launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"paged_attn_decode_{kind}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or m.group(1) != kernel_source_hash(kind):
        return None
    m = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def cpu_baseline(w: workloads.Workload, out: torch.Tensor, sample_seqs: int, min_seconds: float):
    """The oracle, as it stands, on the first `sample_seqs` sequences (all of
    them by default), run repeatedly until `min_seconds` of CPU time have
    passed; KV bytes per second of the mean run."""
    import ctypes

    import oracle

    orc = oracle.get()
    n = w.num_seqs if sample_seqs <= 0 else min(sample_seqs, w.num_seqs)
    sub = w.subset(range(n))
    rows = sub.expanded()  # with query groups: one oracle sequence per query row

    def cache(t):  # fp8 caches go to the oracle as their codes
        return t.numpy() if t.dtype == torch.uint8 else t.float().numpy()

    args = (rows.query.float().numpy(), cache(rows.key_cache), cache(rows.value_cache),
            rows.block_tables.numpy(), rows.seq_lens.numpy(), rows.scale)
    kw = dict(alibi=None if w.alibi_slopes is None else w.alibi_slopes.numpy(),
              k_scale=w.k_scale, v_scale=w.v_scale)
    runs, total = 0, 0.0
    while runs == 0 or total < min_seconds:
        t0 = time.perf_counter()
        ref = orc.attention(*args, **kw)
        total += time.perf_counter() - t0
        runs += 1
    dt = total / runs
    try:
        threads = int(ctypes.CDLL(orc.lib._name).omp_get_max_threads())
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    threads = min(threads, n * w.num_kv_heads)  # one (sequence, kv head) per thread
    kv = sub.kv_bytes()
    err = float(np.abs(out[:n * w.num_group].float().cpu().numpy() - ref).max())
    return ({"value": kv / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
             "sample": f"{n} of {w.num_seqs} sequences (all heads), {kv} KV bytes, "
                       f"{runs} runs in {total:.1f} s", "seconds": dt},
            {"sample_seqs": n, "max_abs_err": err})


def read_stream(w: workloads.Workload, step: "Step", reps: int):
    """The same GPU's plain read rate (pa_read_probe, no arithmetic), on 1 GiB
    of contiguous memory and on the workload's own gather: every live block
    of every sequence through its page list, one run per kv head for keys
    (and values), or every latent row for the MLA layout. Each leg is timed
    with 2, 4 and 8 probe workgroups per compute unit and the fastest
    counts."""
    from paged_attention_decode_tables_amd import api

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grids = (2, 4, 8)  # workgroups per compute unit; the fastest one counts
    sinks = {k: torch.empty(k * cus * 1024, dtype=torch.int32, device="cuda") for k in grids}
    best_grid = {}

    def timed(*args, **kw):
        best = None
        for k in grids:
            sink = sinks[k]
            for _ in range(2):
                api.read_probe(sink, *args, **kw)
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for _ in range(reps):
                api.read_probe(sink, *args, **kw)
            stop.record()
            torch.cuda.synchronize()
            t = start.elapsed_time(stop) / reps * 1e-3  # seconds per launch
            if best is None or t < best[0]:
                best = (t, k)
        best_grid[len(best_grid)] = best[1]
        return best[0]

    n = 1 << 30
    buf = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    pages = torch.arange(n // 4096, dtype=torch.int32, device="cuda")
    t_contig = timed(buf, pages, 1, 4096, 0, 4096)
    del buf, pages
    g = step.g
    if w.latent is not None:
        esz = w.latent.element_size()
        step.pre()  # the flat page list of the step
        pages = step.flat if step.indptr is not None else g.block_tables.reshape(-1)
        row = w.head_size * esz
        t_gather = timed(g.latent, pages, 1, row, 0, row)
        nbytes = pages.numel() * row
        pattern = f"{pages.numel()} latent rows of {row} B at random pages"
    else:
        esz = w.kv_elem_size
        live = [w.block_tables[s, :(max(int(L), 0) + w.block_size - 1) // w.block_size]
                for s, L in enumerate(w.seq_lens)]
        pages = torch.cat(live).to(torch.int32).to("cuda")
        kc, vc = g.key_cache, g.value_cache
        run = w.head_size * w.block_size * esz
        t_gather = timed(kc, pages, w.num_kv_heads, kc.stride(0) * esz, kc.stride(1) * esz, run, base1=vc)
        nbytes = pages.numel() * w.num_kv_heads * run * 2
        pattern = (f"{pages.numel()} blocks x {w.num_kv_heads} kv heads, keys and values, "
                   f"runs of {run} B at random blocks")
    gc = n / t_contig / 1e9
    gg = nbytes / t_gather / 1e9
    return {"kernel": "pa_read_probe", "contiguous_gbs": round(gc, 1),
            "contiguous_frac": round(gc / HBM_PEAK_GBS, 4), "paged_gather_gbs": round(gg, 1),
            "paged_gather_frac": round(gg / HBM_PEAK_GBS, 4), "gather_pattern": pattern,
            "gather_bytes": int(nbytes), "gather_us": round(t_gather * 1e6, 2),
            "contiguous_us": round(t_contig * 1e6, 2),
            "workgroups_per_cu": {"contiguous": best_grid[0], "gather": best_grid[1]}}


# Decode-metadata workloads: the batches of configs 4 and 5 as a serving
# engine's request -> token-slot table (page size 32 with a sliding-window
# map, and page size 1).
MD_WORKLOADS = {
    "metadata_skewed_ps32_swa": dict(cfg=4, page_size=32, swa=True, pool_rows=512, delta=1),
    "metadata_mla_ps1": dict(cfg=5, page_size=1, swa=False, pool_rows=128, delta=1),
}


def bench_metadata(args):
    """One JSON line for normal_decode_set_metadata: GPU µs per launch
    (launches queued back to back on one stream) and algorithmic bytes against
    HBM peak; the rate of back-to-back calls from Python is reported beside it."""
    spec = MD_WORKLOADS[args.md_workload]
    lens = workloads.config_lengths(spec["cfg"]).to(torch.int64)
    c = workloads.metadata_case(seed=100 + spec["cfg"], seq_lens=lens, page_size=spec["page_size"],
                                pool_rows=spec["pool_rows"], seq_len_delta=spec["delta"],
                                swa=spec["swa"])
    B, P = c.batch, c.max_seq_pages
    dev = "cuda"
    sl, rtt, rows = c.seq_lens.to(dev), c.req_to_token.to(dev), c.req_pool_indices.to(dev)
    f2s = c.full_to_swa.to(dev) if spec["swa"] else None
    cs = torch.empty(B, dtype=torch.int32, device=dev)
    cu = torch.empty(B + 1, dtype=torch.int32, device=dev)
    pt = torch.empty((B, P), dtype=torch.int32, device=dev)
    sw = torch.empty((B, P), dtype=torch.int32, device=dev) if spec["swa"] else None

    def launch():
        pad.normal_decode_set_metadata(cs, cu, pt, rtt, rows, P, sl, c.seq_len_delta, c.page_size,
                                       swa_page_table=sw, full_to_swa=f2s)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    K = args.steps
    # GPU time per launch: the K launches are queued behind a short GPU spin
    # (longer than it takes the host to enqueue them), so the events bracket
    # the launches running back to back on the GPU and no host time.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(50e6))  # ~20 ms of GPU cycles
    start.record()
    for _ in range(K):
        launch()
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) / K * 1e3
    # back-to-back calls from Python (bound by the host-side argument marshalling)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(K):
        launch()
    stop.record()
    torch.cuda.synchronize()
    us_b2b = start.elapsed_time(stop) / K * 1e3
    tables = 2 if spec["swa"] else 1
    # reads: lengths and pool rows (8 B each), one slot per page entry (+ one
    # map entry with SWA); writes: lengths, prefix sum, the table(s)
    nbytes = B * 16 + B * P * 4 * tables + B * 4 + (B + 1) * 4 + B * P * 4 * tables
    res = {
        "metric": "decode-metadata µs/launch",
        "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(us * 1e-3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": args.md_workload, "batch": B, "max_seq_pages": P,
                   "page_size": c.page_size, "swa": spec["swa"], "seq_len_delta": c.seq_len_delta,
                   "pool_rows": spec["pool_rows"], "bytes_per_launch": nbytes},
        "roofline": {"bound": "hbm", "kernel": "normal_decode_set_metadata",
                     "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(us, 3)},
        "back_to_back_us_per_call": round(us_b2b, 3),
    }
    if not args.no_cpu_baseline:
        import oracle

        orc = oracle.get()
        a = (c.seq_lens.numpy(), c.req_to_token.numpy(), c.req_pool_indices.numpy(), P,
             c.page_size, c.seq_len_delta, None if f2s is None else c.full_to_swa.numpy())
        t0 = time.perf_counter()
        want = orc.decode_metadata(*a)
        dt = time.perf_counter() - t0
        got = [cs.cpu().numpy(), cu.cpu().numpy(), pt.cpu().numpy(),
               None if sw is None else sw.cpu().numpy()]
        same = all((g is None and w is None) or np.array_equal(g, w) for g, w in zip(got, want))
        res["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "us", "cores": 1,
                               "kind": "oracle", "sample": "the whole launch, one call"}
        res["parity_sample"] = {"bit_exact": bool(same)}
    print(json.dumps(res), flush=True)


def bench_spec_table(args):
    """One JSON line for prepare_swa_spec_page_table on the MLA batch: 64
    requests (page size 1, so a page table row per token), 4 draft tokens
    each with up to 4 extra pages; GPU µs per launch as in bench_metadata."""
    lens = workloads.config_lengths(5).numpy().astype(np.int32)
    bs, R, LB = lens.shape[0], 4, 4
    LA = int(lens.max())
    rng = np.random.default_rng(105)
    a = torch.from_numpy(rng.integers(0, 2**31 - 1, (bs, LA)).astype(np.int32)).cuda()
    b = torch.from_numpy(rng.integers(0, 2**31 - 1, (bs * R, LB)).astype(np.int32)).cuda()
    la = torch.from_numpy(lens).cuda()
    lb_np = rng.integers(1, LB + 1, bs * R).astype(np.int32)
    lb = torch.from_numpy(lb_np).cuda()
    dst = torch.empty((bs * R, LA + LB), dtype=torch.int32, device="cuda")

    def launch():
        pad.prepare_swa_spec_page_table(dst, a, b, la, lb, R)

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    K = args.steps
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(50e6))
    start.record()
    for _ in range(K):
        launch()
    stop.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(stop) / K * 1e3
    # each written entry is one 4-byte read and one 4-byte write, plus the lengths
    written = int(np.repeat(lens, R).astype(np.int64).sum() + lb_np.astype(np.int64).sum())
    nbytes = 8 * written + 4 * (bs + bs * R)
    res = {
        "metric": "speculative SWA page table µs/launch",
        "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(us * 1e-3, 6), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "int32", "data": "synthetic",
        "config": {"workload": "spec_table_mla_batch", "bs": bs, "draft_tokens": R, "len_a": LA,
                   "len_b": LB, "entries_written": written, "bytes_per_launch": nbytes},
        "roofline": {"bound": "hbm", "kernel": "prepare_swa_spec_page_table",
                     "achieved": round(nbytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(us, 3)},
    }
    if not args.no_cpu_baseline:
        import oracle

        orc = oracle.get()
        an, bn = a.cpu().numpy(), b.cpu().numpy()
        t0 = time.perf_counter()
        want = orc.swa_spec_page_table(an, bn, lens, lb_np, R)
        dt = time.perf_counter() - t0
        got = dst.cpu().numpy()
        mask = want != -1  # entries the call writes
        res["cpu_baseline"] = {"value": round(dt * 1e6, 1), "unit": "us", "cores": 1,
                               "kind": "oracle", "sample": "the whole launch, one call"}
        res["parity_sample"] = {"bit_exact": bool(np.array_equal(got[mask], want[mask]))}
    print(json.dumps(res), flush=True)


def build_parser() -> argparse.ArgumentParser:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload number (3 = long-context GQA)")
    ap.add_argument("--cpu-sample-seqs", type=int, default=0,
                    help="sequences the CPU oracle baseline runs (0 = all)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle baseline until this many seconds have passed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB first (a kernel of known "
                         "traffic for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="size of the buffer read before each step of the cold-cache pass "
                         "(0: no cold-cache pass)")
    ap.add_argument("--no-read-stream", action="store_true",
                    help="skip the plain read-stream legs (pa_read_probe)")
    ap.add_argument("--fixed-splits", action="store_true",
                    help="run the MLA workload with its fixed 512-token partitions instead of "
                         "balanced splits")
    ap.add_argument("--op", choices=("decode", "metadata", "spec_table"), default="decode",
                    help="decode: one decode step of --config (the default); metadata: the "
                         "decode-metadata launch on --md-workload; spec_table: the speculative "
                         "SWA page-table concat on the MLA batch")
    ap.add_argument("--md-workload", choices=sorted(MD_WORKLOADS), default="metadata_skewed_ps32_swa")
    ap.add_argument("--kv-cache", choices=("same", "fp8"), default="same",
                    help="fp8: the same workload with FP8 E4M3 caches (configs 2-5)")
    ap.add_argument("--alibi", action="store_true", help="the same workload with ALiBi slopes")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph_replay field (one step captured into a HIP graph, replayed K times)")
    ap.add_argument("--kernel", choices=("auto", "valu"), default="auto",
                    help="phase-1 kernel hint (valu: the vector-ALU kernel, for comparison)")
    ap.add_argument("--tmp-dtype", choices=("query", "f32"), default="query",
                    help="element type of the split-output workspace: the query's type (phase 1 "
                         "stores each split's output converted to it) or fp32")
    ap.add_argument("--num-group", type=int, default=1,
                    help="query tokens per sequence (configs 2-5): each attends over the whole "
                         "sequence; the grouped-head kernel reads the cache once for all of them")
    ap.add_argument("--mla-heads", type=int, choices=(128, 64), default=128,
                    help="query heads over config 5's latent head (64: the same lengths, a "
                         "64-head query)")
    return ap


def main():
    args = build_parser().parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark measures one GPU only: the decode path has no "
                                   "multi-GPU mode, run it with --gpus 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: calibration copy of {n} bytes done")
        del src, dst

    if args.op == "metadata":
        bench_metadata(args)
        return
    if args.op == "spec_table":
        bench_spec_table(args)
        return

    log(f"bench: generating workload {args.config}")
    w = workloads.config(args.config, kv_cache=args.kv_cache, alibi=args.alibi,
                         num_group=args.num_group, mla_heads=args.mla_heads)
    # The MLA workload's split policy is not fixed by its definition: it runs
    # with balanced splits, as many token ranges as workgroups fit at once.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    mla = kernel_kind(w) == "mla" and args.kernel == "auto" and not args.fixed_splits
    workers = balanced_workers(w, cus) if mla else 0
    tmp_dtype = w.dtype if args.tmp_dtype == "query" else torch.float32
    step = Step(w, balanced_workers=workers, tmp_dtype=tmp_dtype, kernel=args.kernel)
    kind = step.kernel_kind()  # the library's own choice
    torch.cuda.synchronize()

    log(f"bench: warmup {args.warmup}")
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()

    K = args.steps
    # Timed region: K back-to-back steps, bracketed by events and a sync.
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"bench: timing {K} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(K):
        step.run()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(stop) / K

    # Kernel region: the same K steps with events around each launch (the
    # extra event packets add gaps, so the step time is taken above).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for k in range(K):
        step.pre()
        ev[k][0].record()
        step.decode()
        ev[k][1].record()
        step.reduce()
        ev[k][2].record()
    torch.cuda.synchronize()
    dec_ev_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    red_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))

    # Phase-1 region: K phase-1 launches back to back (after one step's
    # split counts and page list), bracketed by two events: the kernel's
    # average duration plus the launch gaps, without an event packet next to
    # every launch (those add a few microseconds each).
    step.pre()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    d0.record()
    for _ in range(K):
        step.decode()
    d1.record()
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / K

    # Graph region: one step captured into a HIP graph (the library
    # allocates nothing and never synchronises, so a captured step serves
    # every replay), replayed K times back to back.
    graph = None
    if not args.no_graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step.run()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step.run()
            for _ in range(2):
                g.replay()
            gs, ge = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            gs.record()
            for _ in range(K):
                g.replay()
            ge.record()
            torch.cuda.synchronize()
            g_ms = gs.elapsed_time(ge) / K
            graph = {"us_per_step": round(g_ms * 1e3, 2), "kv_gbs": round(w.kv_bytes() / (g_ms * 1e-3) / 1e9, 1)}
            del g
        except Exception as e:  # reported, not fatal: the eager step is the measurement
            graph = {"error": str(e)[:200]}
    kv = w.kv_bytes()
    value = kv / (ms_step * 1e-3) / 1e9
    achieved = kv / (dec_ms * 1e-3) / 1e9
    traffic = recorded_traffic(w.name, kind, kv)

    # Cold-cache region: before each step a sum reads a buffer larger than
    # the L2s and the 256 MB Infinity Cache, so no KV byte of the previous
    # step is still on chip (a read leaves clean lines: the step pays no
    # write-back of the flush). One pass brackets whole steps with events,
    # a second pass phase 1 alone (events between the launches of a step
    # would add their own gaps to the step).
    cold = None
    if args.flush_mib:
        junk = torch.ones((args.flush_mib << 20) // 4, dtype=torch.float32, device="cuda")
        sink = torch.empty((), dtype=torch.float32, device="cuda")

        def cold_pass(phase1_only):
            evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
            torch.cuda.synchronize()
            for k in range(K):
                torch.sum(junk, dim=0, out=sink)
                if phase1_only:
                    step.pre()
                evc[k][0].record()
                if phase1_only:
                    step.decode()
                else:
                    step.run()
                evc[k][1].record()
                if phase1_only:
                    step.reduce()
            torch.cuda.synchronize()
            return float(np.median([e[0].elapsed_time(e[1]) for e in evc]))

        c_step, c_dec = cold_pass(False), cold_pass(True)
        del junk, sink
        cold = {"flush_mib": args.flush_mib, "us_per_step_median": round(c_step * 1e3, 2),
                "phase1_us_median": round(c_dec * 1e3, 2),
                "kv_gbs": round(kv / (c_step * 1e-3) / 1e9, 1),
                "phase1_frac_of_hbm_peak": round(kv / (c_dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "us_per_step": round(ms_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}[w.dtype]
                 + ("/kv-fp8-e4m3" if w.kv_dtype is not None else ""),
        "data": "synthetic",
        "config": {"workload": w.name, "seqs": w.num_seqs, "seq_len_max": w.max_seq_len,
                   "tokens": w.total_tokens, "heads": w.num_heads, "kv_heads": w.num_kv_heads,
                   "head_dim": w.head_size, "v_head_dim": w.v_head_size,
                   "block_size": w.block_size, "num_blocks": w.num_blocks,
                   "partition": (f"balanced ({workers} token ranges)" if workers else
                                 w.partition_size if w.max_kv_splits is None else "num_kv_splits"),
                   "kv_bytes_per_step": kv,
                   "kv_cache": (f"fp8 e4m3, k_scale = v_scale = {w.k_scale}" if w.kv_dtype is not None
                                else "query dtype"),
                   "alibi": w.alibi_slopes is not None, "num_group": w.num_group,
                   "split_workspace": {torch.bfloat16: "bf16", torch.float16: "f16",
                                       torch.float32: "f32"}[tmp_dtype],
                   "kernel_hint": args.kernel,
                   "query_tokens_per_s": round(w.num_seqs * w.num_group / (ms_step * 1e-3), 1)},
        "roofline": {"bound": "hbm", "kernel": f"paged_attn_decode ({kind})",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "avg_launch_us": round(dec_ms * 1e3, 2),
                     "avg_launch_us_evented": round(dec_ev_ms * 1e3, 2)},
        "phase2_us": round(red_ms * 1e3, 2),
        "wall_ms_per_step": round(wall * 1e3 / K, 5),
    }
    if cold is not None:
        res["cold_cache"] = cold
    if graph is not None:
        res["graph_replay"] = graph
    if not args.no_read_stream:
        log("bench: read-stream legs")
        rs = read_stream(w, step, reps=20)
        res["read_stream"] = rs
        # phase 1 and the whole step against the same gather with no math
        res["pct_of_read_stream"] = round(100.0 * achieved / rs["paged_gather_gbs"], 1)
        res["step_pct_of_read_stream"] = round(100.0 * value / rs["paged_gather_gbs"], 1)
    if not args.no_cpu_baseline:
        log("bench: CPU oracle baseline")
        cb, parity = cpu_baseline(w, step.out, args.cpu_sample_seqs, args.cpu_seconds)
        res["cpu_baseline"] = cb
        res["parity_sample"] = parity
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
