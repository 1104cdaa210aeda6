"""C-ABI checks that need no GPU: the library loads, exports every function
include/pagedattn.h declares, its argument blocks have the header's layout,
and invalid arguments are rejected on the host before any launch."""
import ctypes
import glob
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (load torch's HIP runtime first, as the product does)

from paged_attention_decode_tables_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedattn.h")


def declared_functions():
    """Functions declared in every public header (include/*.h)."""
    names = set()
    for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return api.load_library()


def test_header_declares_the_four_operations():
    names = declared_functions()
    for n in ("paged_attn_decode", "paged_attn_reduce", "build_page_indices", "num_kv_splits",
              "normal_decode_set_metadata", "prepare_swa_spec_page_table"):
        assert n in names
    assert len(names) >= 6, names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", api.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(lib, n)


def _c_layout(struct: str, fields):
    src = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){",
           f'printf("%zu\\n", sizeof({struct}));']
    src += [f'printf("%zu\\n", offsetof({struct}, {f}));' for f in fields]
    src += ["return 0;}"]
    d = os.path.join(ROOT, "_build")
    os.makedirs(d, exist_ok=True)
    c = os.path.join(d, f"layout_{struct}.c")
    exe = c[:-2]
    open(c, "w").write("\n".join(src))
    subprocess.run(["gcc", "-std=c99", c, "-o", exe], check=True)
    vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    return vals[0], vals[1:]


@pytest.mark.parametrize("cls,cname", [(api.DecodeArgs, "pa_decode_args"), (api.ReduceArgs, "pa_reduce_args"),
                                       (api.MetadataArgs, "pa_metadata_args")])
def test_argument_block_layout_matches_header(cls, cname):
    fields = [f for f, _ in cls._fields_]
    size, offs = _c_layout(cname, fields)
    assert ctypes.sizeof(cls) == size
    assert [getattr(cls, f).offset for f in fields] == offs


# ---------------------------------------------------------------------------
# host-side validation (dummy device addresses are never dereferenced: every
# case below must be rejected before a launch)
# ---------------------------------------------------------------------------
FAKE = 1 << 20  # 16-byte aligned stand-in address


def good_decode(dtype=api.PA_BF16, D=128, Dv=128, H=8, Hkv=2, bs=16, P=512):
    a = api.DecodeArgs()
    esz = 4 if dtype == api.PA_F32 else 2
    x = 16 // esz
    S, maxp = 2, 4
    a.tmp_output = FAKE
    a.tmp_stride_s, a.tmp_stride_h, a.tmp_stride_p, a.tmp_stride_d = H * maxp * Dv, maxp * Dv, Dv, 1
    a.exp_sums = a.max_logits = FAKE
    a.ml_stride_s, a.ml_stride_h, a.ml_stride_p = H * maxp, maxp, 1
    a.query = FAKE
    a.q_stride_s, a.q_stride_h, a.q_stride_d = H * D, D, 1
    a.key_cache = FAKE
    a.k_stride_b, a.k_stride_h, a.k_stride_dx, a.k_stride_bs, a.k_stride_x = Hkv * D * bs, D * bs, bs * x, x, 1
    a.value_cache = FAKE
    a.v_stride_b, a.v_stride_h, a.v_stride_d, a.v_stride_bs = Hkv * Dv * bs, Dv * bs, bs, 1
    a.block_tables = a.seq_lens = FAKE
    a.bt_stride_s, a.bt_stride_b = 128, 1
    a.scale = 0.1
    a.num_seqs, a.num_heads, a.num_kv_heads = S, H, Hkv
    a.head_size, a.v_head_size, a.block_size, a.x = D, Dv, bs, x
    a.partition_size, a.max_num_parts, a.max_seq_len = P, maxp, 2048
    a.dtype = dtype
    return a


def _mut(a, **kw):
    for k, v in kw.items():
        setattr(a, k, v)
    return a


DECODE_BAD = [
    ("dtype", dict(dtype=7), api.PA_EINVAL),
    ("heads", dict(num_heads=7), api.PA_EINVAL),
    ("kvheads0", dict(num_kv_heads=0), api.PA_EINVAL),
    ("bs_not_pow2", dict(block_size=12), api.PA_EINVAL),
    ("bs_too_big", dict(block_size=2048), api.PA_EINVAL),
    ("x_mismatch", dict(x=4, k_stride_bs=4, k_stride_dx=64), api.PA_ENOTSUP),
    ("partition_not_64", dict(partition_size=100), api.PA_EINVAL),
    ("too_few_parts", dict(max_seq_len=4096), api.PA_EINVAL),
    ("null_query", dict(query=None), api.PA_EINVAL),
    ("null_seq_lens", dict(seq_lens=None), api.PA_EINVAL),
    ("q_inner_stride", dict(q_stride_d=2), api.PA_ENOTSUP),
    ("k_inner_stride", dict(k_stride_bs=16), api.PA_ENOTSUP),
    ("v_inner_stride", dict(v_stride_d=128, v_stride_bs=16), api.PA_ENOTSUP),
    ("tmp_inner_stride", dict(tmp_stride_d=2), api.PA_ENOTSUP),
    ("head_size", dict(head_size=96, v_head_size=96), api.PA_ENOTSUP),
    ("misaligned_key", dict(key_cache=FAKE + 2), api.PA_ENOTSUP),
    ("misaligned_row", dict(k_stride_b=16 * 128 * 2 + 1), api.PA_ENOTSUP),
    ("max_parts0", dict(max_num_parts=0), api.PA_EINVAL),
    ("neg_seqs", dict(num_seqs=-1), api.PA_EINVAL),
    ("neg_num_group", dict(num_group=-1), api.PA_EINVAL),
    ("grid_rows", dict(num_group=1 << 27), api.PA_ENOTSUP),
    ("tmp_dtype_fp8", dict(tmp_dtype=api.PA_FP8_E4M3), api.PA_EINVAL),
    ("tmp_dtype_neg", dict(tmp_dtype=-1), api.PA_EINVAL),
    ("tmp_row_misaligned", dict(tmp_stride_p=130), api.PA_ENOTSUP),
    # 16-bit rows: a stride of 4 elements keeps them 8-byte aligned only
    ("tmp16_row_misaligned", dict(tmp_dtype=api.PA_BF16, tmp_stride_p=132), api.PA_ENOTSUP),
]


@pytest.mark.parametrize("name,change,code", DECODE_BAD, ids=[c[0] for c in DECODE_BAD])
def test_decode_rejects(lib, name, change, code):
    a = _mut(good_decode(), **change)
    assert lib.paged_attn_decode(ctypes.byref(a), None) == code
    assert lib.pa_last_error()


def test_decode_mfma_hint_rejected_where_it_does_not_apply(lib):
    a = _mut(good_decode(dtype=api.PA_F32, D=64, Dv=64), kernel_hint=api.PA_KERNEL["mfma"])
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_ENOTSUP
    a = _mut(good_decode(D=256, Dv=256), kernel_hint=api.PA_KERNEL["mfma"])  # head size 256
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_ENOTSUP
    a = _mut(good_decode(bs=4), kernel_hint=api.PA_KERNEL["mfma"])  # blocks of 4 tokens
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_ENOTSUP
    a = _mut(good_decode(H=16, Hkv=1), kernel_hint=api.PA_KERNEL["mfma"], num_group=2)  # 32 columns
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_ENOTSUP


def good_fp8(**kw):
    """A valid bf16-query problem over FP8 E4M3 caches (x = 16, byte strides)."""
    a = good_decode(**kw)
    D, Dv, Hkv, bs = a.head_size, a.v_head_size, a.num_kv_heads, a.block_size
    a.x = 16
    a.k_stride_b, a.k_stride_h, a.k_stride_dx, a.k_stride_bs, a.k_stride_x = Hkv * D * bs, D * bs, bs * 16, 16, 1
    a.kv_dtype = api.PA_FP8_E4M3
    a.k_scale, a.v_scale = 0.05, 0.1
    return a


FP8_BAD = [
    ("k_scale_zero", dict(k_scale=0.0), api.PA_EINVAL),
    ("v_scale_zero", dict(v_scale=0.0), api.PA_EINVAL),
    ("k_scale_inf", dict(k_scale=float("inf")), api.PA_EINVAL),
    ("v_scale_nan", dict(v_scale=float("nan")), api.PA_EINVAL),
    ("kv_dtype_unknown", dict(kv_dtype=9), api.PA_EINVAL),
    ("x_of_query_dtype", dict(x=8, k_stride_bs=8, k_stride_dx=16 * 8), api.PA_ENOTSUP),
    ("mfma_hint_f32_query", dict(kernel_hint=api.PA_KERNEL["mfma"], dtype=api.PA_F32,
                                 q_stride_s=8 * 128 * 2), api.PA_ENOTSUP),
    ("misaligned_block", dict(k_stride_b=2 * 128 * 16 + 8), api.PA_ENOTSUP),
]


@pytest.mark.parametrize("name,change,code", FP8_BAD, ids=[c[0] for c in FP8_BAD])
def test_decode_fp8_rejects(lib, name, change, code):
    a = _mut(good_fp8(), **change)
    assert lib.paged_attn_decode(ctypes.byref(a), None) == code
    assert lib.pa_last_error()


def test_decode_kv_dtype_must_be_query_dtype_or_fp8(lib):
    a = _mut(good_decode(), kv_dtype=api.PA_F16)  # bf16 query over f16 caches
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_EINVAL
    a = _mut(good_decode(), kv_dtype=api.PA_BF16, num_seqs=0)  # equal to dtype: accepted
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_OK
    a = _mut(good_fp8(), num_seqs=0)
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_OK


def test_decode_balanced_splits_need_the_mla_kernel(lib):
    """Balanced splits are built into the latent-row kernel only: 64 or 128
    heads over one latent row whose leading columns are the values. 16 heads
    over latent rows, and 128 heads whose values are a separate cache, are
    not that shape (fp8 codes or not)."""
    a = good_fp8(D=576, Dv=512, H=16, Hkv=1, bs=1)
    a.value_cache = a.key_cache
    a.v_stride_b, a.v_stride_h, a.v_stride_d = a.k_stride_b, a.k_stride_h, 1
    a.partition_size, a.num_workers, a.max_num_parts = 0, 256, 256
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_ENOTSUP
    assert "balanced" in lib.pa_last_error().decode()
    b = good_fp8(D=576, Dv=512, H=128, Hkv=1, bs=1)  # value cache not the key rows
    b.partition_size, b.num_workers, b.max_num_parts = 0, 256, 256
    assert lib.paged_attn_decode(ctypes.byref(b), None) == api.PA_ENOTSUP


def test_decode_empty_batch_is_a_noop(lib):
    a = _mut(good_decode(), num_seqs=0, query=None)
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_OK
    a = _mut(good_decode(), max_seq_len=0)
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_OK


def good_reduce():
    a = api.ReduceArgs()
    S, H, P, Dv = 2, 8, 4, 128
    a.output = FAKE
    a.out_stride_s, a.out_stride_h, a.out_stride_d = H * Dv, Dv, 1
    a.out_dtype = api.PA_BF16
    a.tmp_output = FAKE
    a.tmp_stride_s, a.tmp_stride_h, a.tmp_stride_p, a.tmp_stride_d = H * P * Dv, P * Dv, Dv, 1
    a.exp_sums = a.max_logits = FAKE
    a.ml_stride_s, a.ml_stride_h, a.ml_stride_p = H * P, P, 1
    a.seq_lens = FAKE
    a.num_seqs, a.num_heads, a.v_head_size = S, H, Dv
    a.partition_size, a.max_num_parts = 512, P
    return a


REDUCE_BAD = [
    ("out_dtype", dict(out_dtype=9), api.PA_EINVAL),
    ("heads0", dict(num_heads=0), api.PA_EINVAL),
    ("partition", dict(partition_size=32), api.PA_EINVAL),
    ("null_tmp", dict(tmp_output=None), api.PA_EINVAL),
    ("dv", dict(v_head_size=96), api.PA_ENOTSUP),
    ("inner", dict(out_stride_d=2), api.PA_ENOTSUP),
    ("tmp_align", dict(tmp_stride_p=130), api.PA_ENOTSUP),
    ("tmp16_align", dict(tmp_dtype=api.PA_BF16, tmp_stride_p=132), api.PA_ENOTSUP),
    ("neg_num_group", dict(num_group=-1), api.PA_EINVAL),
    ("tmp_dtype", dict(tmp_dtype=9), api.PA_EINVAL),
]


@pytest.mark.parametrize("name,change,code", REDUCE_BAD, ids=[c[0] for c in REDUCE_BAD])
def test_reduce_rejects(lib, name, change, code):
    a = _mut(good_reduce(), **change)
    assert lib.paged_attn_reduce(ctypes.byref(a), None) == code


def test_reduce_empty_batch_is_a_noop(lib):
    a = _mut(good_reduce(), num_seqs=0, output=None)
    assert lib.paged_attn_reduce(ctypes.byref(a), None) == api.PA_OK


def test_index_helpers_reject(lib):
    assert lib.build_page_indices(FAKE, FAKE, 8, 1, FAKE, -1, None) == api.PA_EINVAL
    assert lib.build_page_indices(None, FAKE, 8, 1, FAKE, 3, None) == api.PA_EINVAL
    assert lib.build_page_indices(None, None, 8, 1, None, 0, None) == api.PA_OK
    assert lib.num_kv_splits(FAKE, FAKE, 4, 1, 8, 1, 0, 256, None) == api.PA_EINVAL
    assert lib.num_kv_splits(FAKE, FAKE, 4, 0, 8, 1, 16, 256, None) == api.PA_EINVAL
    assert lib.num_kv_splits(FAKE, FAKE, 4, 1, 8, 1, 16, 0, None) == api.PA_EINVAL
    assert lib.num_kv_splits(None, None, 0, 1, 8, 1, 16, 256, None) == api.PA_OK
    # fewer query heads than kv heads: the heuristic's group size would be 0
    assert lib.num_kv_splits(FAKE, FAKE, 4, 1, 2, 4, 16, 256, None) == api.PA_EINVAL
    assert lib.paged_token_offsets(FAKE, 8, FAKE, 8, 1, None, FAKE, 2, 8, 3, 1, 1, None) == api.PA_EINVAL
    assert lib.paged_token_offsets(None, 8, FAKE, 8, 1, None, FAKE, 2, 8, 4, 1, 1, None) == api.PA_EINVAL


def good_metadata(B=4, pages=10, ps=16):
    a = api.MetadataArgs()
    a.cache_seqlens, a.cache_seqlens_stride = FAKE, 1
    a.cu_seqlens_k, a.cu_seqlens_k_stride = FAKE, 1
    a.page_table, a.page_table_stride0, a.page_table_stride1 = FAKE, pages, 1
    a.seq_lens, a.seq_lens_stride = FAKE, 1
    a.req_to_token, a.req_to_token_stride0, a.req_to_token_stride1 = FAKE, pages * ps, 1
    a.req_pool_indices, a.req_pool_indices_stride = FAKE, 1
    a.batch, a.max_seq_pages, a.page_size = B, pages, ps
    return a


@pytest.mark.parametrize("name,change", [
    ("page_size_not_pow2", dict(page_size=12)),
    ("page_size_zero", dict(page_size=0)),
    ("negative_batch", dict(batch=-1)),
    ("negative_pages", dict(max_seq_pages=-2)),
    ("reserved_set", dict(reserved=1)),
    ("no_cu", dict(cu_seqlens_k=None)),
    ("no_lengths_out", dict(cache_seqlens=None)),
    ("no_seq_lens", dict(seq_lens=None)),
    ("no_page_table", dict(page_table=None)),
    ("no_req_to_token", dict(req_to_token=None)),
    ("no_pool_indices", dict(req_pool_indices=None)),
])
def test_metadata_rejects(lib, name, change):
    a = _mut(good_metadata(), **change)
    assert lib.normal_decode_set_metadata(ctypes.byref(a), None) == api.PA_EINVAL
    assert lib.normal_decode_set_metadata(None, None) == api.PA_EINVAL


def test_spec_page_table_rejects(lib):
    f = lib.prepare_swa_spec_page_table
    assert f(FAKE, 8, 1, FAKE, 4, 1, FAKE, 4, 1, FAKE, FAKE, -1, 4, 4, 2, None) == api.PA_EINVAL
    assert f(FAKE, 8, 1, FAKE, 4, 1, FAKE, 4, 1, FAKE, FAKE, 3, -4, 4, 2, None) == api.PA_EINVAL
    assert f(FAKE, 8, 1, FAKE, 4, 1, FAKE, 4, 1, FAKE, FAKE, 3, 4, 4, 0, None) == api.PA_EINVAL
    assert f(None, 8, 1, FAKE, 4, 1, FAKE, 4, 1, FAKE, FAKE, 3, 4, 4, 2, None) == api.PA_EINVAL
    assert f(FAKE, 8, 1, None, 4, 1, FAKE, 4, 1, FAKE, FAKE, 3, 4, 4, 2, None) == api.PA_EINVAL
    assert f(FAKE, 8, 1, FAKE, 4, 1, FAKE, 4, 1, FAKE, None, 3, 4, 4, 2, None) == api.PA_EINVAL
    assert f(None, 8, 1, None, 4, 1, None, 4, 1, None, None, 0, 4, 4, 2, None) == api.PA_OK


def test_binding_raises_on_error():
    with pytest.raises(api.PagedAttnError) as e:
        api._check(api.PA_EINVAL)
    assert e.value.code == api.PA_EINVAL


# ---------------------------------------------------------------------------
# the Python binding checks what the C ABI cannot see (element types, shapes,
# contiguity of arrays read without strides, the device) before any call
# ---------------------------------------------------------------------------
def _decode_tensors(S=3, H=8, Hkv=2, D=128, bs=16, P=2, NB=10, dtype=torch.bfloat16):
    x = 16 // torch.tensor([], dtype=dtype).element_size()
    return dict(
        tmp_output=torch.zeros(S, H, P, D), exp_sums=torch.zeros(S, H, P),
        max_logits=torch.zeros(S, H, P), query=torch.zeros(S, H, D, dtype=dtype),
        key_cache=torch.zeros(NB, Hkv, D // x, bs, x, dtype=dtype),
        value_cache=torch.zeros(NB, Hkv, D, bs, dtype=dtype),
        block_tables=torch.zeros(S, 4, dtype=torch.int32),
        seq_lens=torch.ones(S, dtype=torch.int32), scale=0.1, max_seq_len=64)


def _bad_decode(**change):
    t = _decode_tensors()
    t.update(change)
    return t


@pytest.mark.parametrize("name,change,exc", [
    ("seq_lens_int64", dict(seq_lens=torch.ones(3, dtype=torch.int64)), TypeError),
    ("seq_lens_sliced", dict(seq_lens=torch.ones(6, dtype=torch.int32)[::2]), ValueError),
    ("workspace_int32", dict(tmp_output=torch.zeros(3, 8, 2, 128, dtype=torch.int32)), TypeError),
    ("workspace_short", dict(tmp_output=torch.zeros(3, 8, 2, 64)), ValueError),
    ("exp_sums_shape", dict(exp_sums=torch.zeros(3, 8, 1)), ValueError),
    ("max_logits_f16", dict(max_logits=torch.zeros(3, 8, 2, dtype=torch.float16)), TypeError),
    ("block_tables_int64", dict(block_tables=torch.zeros(3, 4, dtype=torch.int64)), TypeError),
    ("block_tables_1d", dict(block_tables=torch.zeros(12, dtype=torch.int32)), ValueError),
    ("query_rank", dict(query=torch.zeros(3, 8 * 128, dtype=torch.bfloat16)), ValueError),
    ("query_int", dict(query=torch.zeros(3, 8, 128, dtype=torch.int16)), TypeError),
    ("host_tensors", {}, ValueError),  # every shape right, but nothing is on a GPU
])
def test_binding_rejects_decode(name, change, exc):
    t = _bad_decode(**change)
    with pytest.raises(exc):
        api.paged_attn_decode(**t)


def test_binding_rejects_decode_options():
    with pytest.raises(TypeError):  # split counts as int64
        api.paged_attn_decode(**_decode_tensors(), num_splits=torch.ones(3, dtype=torch.int64))
    with pytest.raises(ValueError):  # one split count per query row
        api.paged_attn_decode(**_decode_tensors(), num_splits=torch.ones(4, dtype=torch.int32))
    t = _decode_tensors()
    t["block_tables"] = torch.zeros(12, dtype=torch.int32)
    with pytest.raises(ValueError):  # indptr of num_seqs + 1 entries
        api.paged_attn_decode(**t, kv_indptr=torch.zeros(3, dtype=torch.int32))


def test_binding_rejects_reduce():
    t = _decode_tensors()
    ok = dict(output=torch.zeros(3, 8, 128), tmp_output=t["tmp_output"], exp_sums=t["exp_sums"],
              max_logits=t["max_logits"], seq_lens=t["seq_lens"])
    for change, exc in ((dict(output=torch.zeros(3, 8, 64)), ValueError),
                        (dict(output=torch.zeros(3, 8, 128, dtype=torch.int32)), TypeError),
                        (dict(exp_sums=torch.zeros(3, 8, 2, dtype=torch.float64)), TypeError),
                        (dict(seq_lens=torch.ones(3, dtype=torch.int64)), TypeError),
                        (dict(tmp_output=torch.zeros(3, 8, 2, 128, dtype=torch.int16)), TypeError),
                        ({}, ValueError)):
        with pytest.raises(exc):
            api.paged_attn_reduce(**{**ok, **change})


def test_binding_rejects_index_helpers():
    bt = torch.zeros(4, 8, dtype=torch.int32)
    cu = torch.zeros(5, dtype=torch.int32)
    with pytest.raises(TypeError):
        api.build_page_indices(torch.zeros(32, dtype=torch.int64), bt, cu)
    with pytest.raises(ValueError):
        api.build_page_indices(torch.zeros(64, dtype=torch.int32)[::2], bt, cu)
    with pytest.raises(TypeError):
        api.build_page_indices(torch.zeros(32, dtype=torch.int32), bt, cu.long())
    with pytest.raises(ValueError):
        api.build_page_indices(torch.zeros(32, dtype=torch.int32), bt, cu)  # host tensors
    lens = torch.ones(4, dtype=torch.int32)
    with pytest.raises(TypeError):
        api.num_kv_splits(torch.zeros(4, dtype=torch.int32), lens.long(), 1, 8, 2, 16, 256)
    with pytest.raises(ValueError):  # one count per (sequence, group)
        api.num_kv_splits(torch.zeros(4, dtype=torch.int32), lens, 2, 8, 2, 16, 256)
    with pytest.raises(TypeError):
        api.paged_token_offsets(torch.zeros(4, 16, dtype=torch.int32), bt, lens, 8, 1, 1)
    with pytest.raises(ValueError):
        api.paged_token_offsets(torch.zeros(4, 16, dtype=torch.int64), bt, lens, 8, 1, 1)


def test_static_scratch_entry_rejects_on_the_host(lib):
    """paged_attn_decode_static checks its arguments before any device call:
    partials larger than the scratch buffer, caller workspaces given, and an
    empty batch (a no-op)."""
    lib.paged_attn_decode_static.argtypes = [ctypes.POINTER(api.DecodeArgs), ctypes.c_void_p,
                                             ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                             ctypes.c_void_p]
    a = good_decode()
    a.tmp_output = a.exp_sums = a.max_logits = None
    a.max_num_parts = 1 << 20  # 3 x 8 x 2^20 x 130 x 4 bytes
    assert lib.paged_attn_decode_static(ctypes.byref(a), FAKE, 1024, 128, api.PA_F32, None) == api.PA_EINVAL
    assert b"scratch buffer" in lib.pa_last_error()
    a = good_decode()  # workspaces given
    assert lib.paged_attn_decode_static(ctypes.byref(a), FAKE, 1024, 128, api.PA_F32, None) == api.PA_EINVAL
    a.tmp_output = a.exp_sums = a.max_logits = None
    a.num_seqs = 0
    assert lib.paged_attn_decode_static(ctypes.byref(a), None, 0, 0, api.PA_F32, None) == api.PA_OK
    assert lib.paged_attn_decode_static(None, None, 0, 0, api.PA_F32, None) == api.PA_EINVAL
    # 16-bit partials: sized at 2 bytes a value (+ 8 for the statistics)
    a = good_decode()
    a.tmp_output = a.exp_sums = a.max_logits = None
    a.max_num_parts, a.tmp_dtype = 1 << 20, api.PA_BF16
    assert lib.paged_attn_decode_static(ctypes.byref(a), FAKE, 1024, 128, api.PA_F32, None) == api.PA_EINVAL
    msg = lib.pa_last_error().decode()
    assert "x 2 + 8" in msg and str(a.num_seqs * a.num_heads * (1 << 20) * (128 * 2 + 8)) in msg, msg
    a.tmp_dtype = 7
    assert lib.paged_attn_decode_static(ctypes.byref(a), FAKE, 1024, 128, api.PA_F32, None) == api.PA_EINVAL


def test_read_probe_rejects_on_the_host(lib):
    f = lib.pa_read_probe
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p]
    assert f(FAKE, None, FAKE, 10, 1, 4096, 0, 4008, FAKE, 4, None) == api.PA_EINVAL  # run not 16k
    assert f(FAKE, None, FAKE, 10, 1, 4096, 0, 16384, FAKE, 4, None) == api.PA_EINVAL  # run > 8 KB
    assert f(FAKE, None, FAKE, 10, 0, 4096, 0, 4096, FAKE, 4, None) == api.PA_EINVAL  # no runs
    assert f(FAKE, None, FAKE, 10, 1, 4100, 0, 4096, FAKE, 4, None) == api.PA_EINVAL  # stride
    assert f(FAKE + 8, None, FAKE, 10, 1, 4096, 0, 4096, FAKE, 4, None) == api.PA_EINVAL  # alignment
    assert f(None, None, FAKE, 10, 1, 4096, 0, 4096, FAKE, 4, None) == api.PA_EINVAL  # no base
    assert f(FAKE, None, FAKE, 10, 1, 4096, 0, 4096, FAKE, 0, None) == api.PA_EINVAL  # no workgroups
    assert b"pa_read_probe" in lib.pa_last_error()


# ---------------------------------------------------------------------------
# paged_attn_decode_kernel: the kernel choice, host only (no GPU)
# ---------------------------------------------------------------------------
def _latent_args(H=128, dtype=api.PA_BF16, fp8=False):
    """Latent rows: D 576, Dv 512, page size 1, V the leading columns of K."""
    a = good_decode(dtype=dtype, D=576, Dv=512, H=H, Hkv=1, bs=1)
    if fp8:
        a.x, a.kv_dtype, a.k_scale, a.v_scale = 16, api.PA_FP8_E4M3, 0.05, 0.05
        a.k_stride_dx, a.k_stride_bs = 16, 16
    a.value_cache = a.key_cache
    a.v_stride_b, a.v_stride_h, a.v_stride_d, a.v_stride_bs = a.k_stride_b, a.k_stride_h, 1, 1
    return a


KERNEL_CHOICE = [
    ("mha_one_column", lambda: good_decode(H=8, Hkv=8), "valu"),
    ("mha_one_column_fp8", lambda: good_fp8(H=8, Hkv=8), "mfma"),
    ("mha_one_column_mfma_hint", lambda: _mut(good_decode(H=8, Hkv=8), kernel_hint=api.PA_KERNEL["mfma"]), "mfma"),
    ("gqa_8", lambda: good_decode(H=8, Hkv=1), "mfma"),
    ("gqa_8_valu_hint", lambda: _mut(good_decode(H=8, Hkv=1), kernel_hint=api.PA_KERNEL["valu"]), "valu"),
    ("gqa_32_columns", lambda: good_decode(H=32, Hkv=1), "valu"),
    ("mha_two_tokens", lambda: _mut(good_decode(H=8, Hkv=8), num_group=2), "mfma"),
    ("fp32", lambda: good_decode(dtype=api.PA_F32, D=64, Dv=64, H=8, Hkv=1), "valu"),
    ("head_256", lambda: good_decode(D=256, Dv=256, H=8, Hkv=1), "valu"),
    ("small_blocks", lambda: good_decode(H=8, Hkv=1, bs=4), "valu"),
    ("latent_rows", lambda: _latent_args(), "mla"),
    ("latent_rows_64", lambda: _latent_args(H=64), "mla"),
    ("latent_rows_f16", lambda: _latent_args(dtype=api.PA_F16), "mla"),
    ("latent_rows_fp8", lambda: _latent_args(fp8=True), "mla"),
    ("latent_rows_valu_hint", lambda: _mut(_latent_args(), kernel_hint=api.PA_KERNEL["valu"]), "valu"),
    ("latent_rows_32_heads", lambda: _latent_args(H=32), "valu"),
    ("latent_rows_not_aliased", lambda: _mut(_latent_args(), value_cache=FAKE + 4096), "valu"),
    ("empty_batch", lambda: _mut(good_decode(H=8, Hkv=1), num_seqs=0), "mfma"),
]


@pytest.mark.parametrize("name,make,kind", KERNEL_CHOICE, ids=[c[0] for c in KERNEL_CHOICE])
def test_decode_kernel_choice(lib, name, make, kind):
    rc = lib.paged_attn_decode_kernel(ctypes.byref(make()))
    assert rc > 0, lib.pa_last_error()
    assert api.KERNEL_NAMES[rc] == kind


def test_decode_kernel_choice_rejects_like_decode(lib):
    for name, change, code in DECODE_BAD:
        a = _mut(good_decode(), **change)
        assert lib.paged_attn_decode_kernel(ctypes.byref(a)) == code, name
    a = _mut(good_decode(), kernel_hint=7)
    assert lib.paged_attn_decode_kernel(ctypes.byref(a)) == api.PA_EINVAL
    assert lib.paged_attn_decode(ctypes.byref(a), None) == api.PA_EINVAL
