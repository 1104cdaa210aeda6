"""Randomized tiny shapes (hypothesis), beside the fixed case lists.

CPU: the oracle's attention, split statistics and merge against numpy brute
force on random shapes of the [PAv2] phase-1 algorithm (module docstring):
block size, group size, head dims, ragged lengths (empty ones included) and
the partition size all drawn.

GPU: the HIP path through the C ABI against the oracle on random shapes
that both phase-1 kernel families and the latent-row kernel accept, with
the same bounds as the fixed cases. Examples are derandomized (the same
draws every run) and nothing is written to an example database.
"""
import math

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

from paged_attention_decode_tables_amd import workloads
import pins

CPU_SETTINGS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                        suppress_health_check=[HealthCheck.too_slow])
GPU_SETTINGS = settings(max_examples=24, deadline=None, derandomize=True, database=None,
                        suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])


def _lens(max_len, max_seqs):
    """1..max_seqs lengths in [0, max_len], at least one of them positive."""
    return st.lists(st.integers(0, max_len), min_size=1, max_size=max_seqs).filter(lambda v: max(v) > 0)


@CPU_SETTINGS
@given(seed=st.integers(0, 10 ** 6), lens=_lens(90, 4), bs=st.sampled_from([1, 2, 4, 8, 16]),
       hkv=st.integers(1, 2), group=st.integers(1, 4), d=st.sampled_from([4, 8, 16]),
       dv=st.sampled_from([4, 8, 12]), part=st.sampled_from([1, 3, 8, 64]))
def test_oracle_random_tiny_shapes(orc, seed, lens, bs, hkv, group, d, dv, part):
    w = workloads.custom(seed=seed, seq_lens=lens, num_heads=hkv * group, num_kv_heads=hkv, head_size=d,
                         v_head_size=dv, block_size=bs, dtype="f32", poison=True)
    args = (pins._np(w.query), pins._np(w.key_cache), pins._np(w.value_cache), w.block_tables.numpy(),
            w.seq_lens.numpy(), w.scale)
    want = pins.brute_attention(*args)
    got = orc.attention(*args)
    assert np.abs(got - want).max() < 1e-10
    n = -(-max(lens) // part)
    tmp, ml, es = orc.partials(*args, max_num_parts=n + 1, partition_size=part)
    split = pins._brute_partials(w, [part] * len(lens))
    for (s, h, p), (m, l, out) in split.items():
        assert abs(ml[s, h, p] - m) < 1e-10 and abs(es[s, h, p] / l - 1) < 1e-10
        assert np.abs(tmp[s, h, p] - out).max() < 1e-10
    merged = orc.reduce(tmp, ml, es, w.seq_lens.numpy(), partition_size=part)
    assert np.abs(merged - want).max() < 1e-10


@pytest.mark.gpu
@GPU_SETTINGS
@given(seed=st.integers(0, 10 ** 6), lens=_lens(1300, 4), dt=st.sampled_from(["f32", "f16", "bf16"]),
       d=st.sampled_from([64, 128, 256]), bs=st.sampled_from([1, 2, 8, 16, 32, 128]),
       hkv=st.integers(1, 2), group=st.sampled_from([1, 2, 3, 4, 8, 16]),
       part=st.sampled_from([64, 128, 512]), kernel=st.sampled_from(["auto", "valu"]))
def test_hip_random_shapes(orc, seed, lens, dt, d, bs, hkv, group, part, kernel):
    from gpu_util import check_output, check_partials, run_gpu, say
    say(f"random shape: dt={dt} D={d} bs={bs} Hkv={hkv} G={group} P={part} {kernel} lens={lens}")
    w = workloads.custom(seed=seed, seq_lens=lens, num_heads=hkv * group, num_kv_heads=hkv, head_size=d,
                         block_size=bs, dtype=dt, partition_size=part, poison=True)
    out, tmp, ml, es = run_gpu(w, partition_size=part, kernel=kernel)
    check_partials(w, orc, tmp, ml, es, partition_size=part, kernel=kernel)
    check_output(w, orc, out, kernel=kernel)


@pytest.mark.gpu
@settings(max_examples=10, deadline=None, derandomize=True, database=None,
          suppress_health_check=[HealthCheck.too_slow, HealthCheck.function_scoped_fixture])
@given(seed=st.integers(0, 10 ** 6), lens=_lens(1500, 6), heads=st.sampled_from([64, 128]),
       kv=st.sampled_from(["same", "fp8"]), workers=st.integers(0, 9))
def test_hip_random_latent_rows(orc, seed, lens, heads, kv, workers):
    """workers 0: fixed 512-token splits; otherwise balanced splits over that
    many token ranges."""
    from gpu_util import check_output, check_partials, run_gpu, say
    import test_gpu_parity as tp
    say(f"random latent rows: H={heads} kv={kv} workers={workers} lens={lens}")
    w = workloads.mla_custom(seed=seed, seq_lens=lens, num_heads=heads, kv_cache=kv, poison=True)
    if workers == 0:
        out, tmp, ml, es = run_gpu(w, partition_size=512)
        check_partials(w, orc, tmp, ml, es, partition_size=512)
    else:
        max_parts = max(2, math.ceil(max(lens) / 256))
        out, tmp, ml, es = tp.run_balanced(w, workers, max_parts)
        tp.check_balanced_pieces(w, orc, tmp, ml, es, workers, max_parts)
    check_output(w, orc, out)
