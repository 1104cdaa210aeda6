"""ctypes binding of libpagedattn.so (C ABI in include/pagedattn.h).

Argument marshalling only: each function reads shapes, strides, dtypes and
data pointers from torch tensors, fills the C argument block and calls the
library on the current (or given) HIP stream. All computation happens in the
library's HIP kernels. There is no fallback: if the library is missing the
first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libpagedattn.so"

PA_OK, PA_EINVAL, PA_ENOTSUP, PA_ELAUNCH = 0, -1, -2, -3
PA_F32, PA_F16, PA_BF16, PA_FP8_E4M3 = 0, 1, 2, 3
PA_KERNEL = {"auto": 0, "valu": 1, "mfma": 2}
KERNEL_NAMES = {1: "valu", 2: "mfma", 3: "mla"}  # paged_attn_decode_kernel results
_DTYPE = {torch.float32: PA_F32, torch.float16: PA_F16, torch.bfloat16: PA_BF16}
_FP8_CACHE = (torch.uint8, torch.float8_e4m3fn)  # cache tensors holding E4M3 codes
_CODE_NAMES = {PA_EINVAL: "PA_EINVAL", PA_ENOTSUP: "PA_ENOTSUP", PA_ELAUNCH: "PA_ELAUNCH"}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class PagedAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODE_NAMES.get(code, code)}: {msg}")
        self.code = code


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("tmp_output", _vp), ("tmp_stride_s", _i64), ("tmp_stride_h", _i64),
        ("tmp_stride_p", _i64), ("tmp_stride_d", _i64),
        ("exp_sums", _vp), ("max_logits", _vp),
        ("ml_stride_s", _i64), ("ml_stride_h", _i64), ("ml_stride_p", _i64),
        ("query", _vp), ("q_stride_s", _i64), ("q_stride_h", _i64), ("q_stride_d", _i64),
        ("key_cache", _vp), ("k_stride_b", _i64), ("k_stride_h", _i64), ("k_stride_dx", _i64),
        ("k_stride_bs", _i64), ("k_stride_x", _i64),
        ("value_cache", _vp), ("v_stride_b", _i64), ("v_stride_h", _i64), ("v_stride_d", _i64),
        ("v_stride_bs", _i64),
        ("block_tables", _vp), ("bt_stride_s", _i64), ("bt_stride_b", _i64),
        ("kv_indptr", _vp), ("seq_lens", _vp), ("num_splits", _vp),
        ("scale", ctypes.c_float),
        ("num_seqs", _i32), ("num_heads", _i32), ("num_kv_heads", _i32),
        ("head_size", _i32), ("v_head_size", _i32), ("block_size", _i32), ("x", _i32),
        ("partition_size", _i32), ("max_num_parts", _i32), ("max_seq_len", _i32),
        ("dtype", _i32), ("kernel_hint", _i32), ("num_workers", _i32),
        ("alibi_slopes", _vp), ("kv_dtype", _i32), ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float), ("num_group", _i32), ("tmp_dtype", _i32),
    ]


class ReduceArgs(ctypes.Structure):
    _fields_ = [
        ("output", _vp), ("out_stride_s", _i64), ("out_stride_h", _i64), ("out_stride_d", _i64),
        ("out_dtype", _i32),
        ("tmp_output", _vp), ("tmp_stride_s", _i64), ("tmp_stride_h", _i64),
        ("tmp_stride_p", _i64), ("tmp_stride_d", _i64),
        ("exp_sums", _vp), ("max_logits", _vp),
        ("ml_stride_s", _i64), ("ml_stride_h", _i64), ("ml_stride_p", _i64),
        ("seq_lens", _vp), ("num_splits", _vp),
        ("num_seqs", _i32), ("num_heads", _i32), ("v_head_size", _i32),
        ("partition_size", _i32), ("max_num_parts", _i32), ("num_group", _i32),
        ("tmp_dtype", _i32),
    ]


class MetadataArgs(ctypes.Structure):
    _fields_ = [
        ("cache_seqlens", _vp), ("cache_seqlens_stride", _i64),
        ("cu_seqlens_k", _vp), ("cu_seqlens_k_stride", _i64),
        ("page_table", _vp), ("page_table_stride0", _i64), ("page_table_stride1", _i64),
        ("swa_page_table", _vp), ("swa_page_table_stride0", _i64), ("swa_page_table_stride1", _i64),
        ("seq_lens", _vp), ("seq_lens_stride", _i64),
        ("req_to_token", _vp), ("req_to_token_stride0", _i64), ("req_to_token_stride1", _i64),
        ("req_pool_indices", _vp), ("req_pool_indices_stride", _i64),
        ("full_to_swa", _vp), ("full_to_swa_stride", _i64),
        ("batch", _i32), ("max_seq_pages", _i32), ("page_size", _i32), ("reserved", _i32),
        ("seq_len_delta", _i64),
    ]


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.environ.get("PAGEDATTN_LIB", os.path.join(_PKG, LIB_NAME))


def load_library() -> ctypes.CDLL:
    """Load libpagedattn.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m paged_attention_decode_tables_amd.build`")
    lib = ctypes.CDLL(path)
    lib.paged_attn_decode.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
    lib.paged_attn_decode_kernel.argtypes = [ctypes.POINTER(DecodeArgs)]
    lib.paged_attn_reduce.argtypes = [ctypes.POINTER(ReduceArgs), _vp]
    lib.paged_attn_decode_static.argtypes = [ctypes.POINTER(DecodeArgs), _vp, _i64, _i64, _i32, _vp]
    lib.build_page_indices.argtypes = [_vp, _vp, _i64, _i64, _vp, _i32, _vp]
    lib.num_kv_splits.argtypes = [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]
    lib.paged_token_offsets.argtypes = [_vp, _i64, _vp, _i64, _i64, _vp, _vp, _i32, _i32, _i32,
                                        _i64, _i64, _vp]
    lib.normal_decode_set_metadata.argtypes = [ctypes.POINTER(MetadataArgs), _vp]
    lib.prepare_swa_spec_page_table.argtypes = [_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64,
                                                _vp, _vp, _i32, _i32, _i32, _i32, _vp]
    lib.pa_read_probe.argtypes = [_vp, _vp, _vp, _i64, _i32, _i64, _i64, _i32, _vp, _i32, _vp]
    lib.pa_last_error.restype = ctypes.c_char_p
    lib.pa_last_error.argtypes = []
    _lib = lib
    return lib


def _check(rc: int):
    if rc != PA_OK:
        raise PagedAttnError(rc, load_library().pa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPE:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPE[t.dtype]


def _page_strides(block_tables: torch.Tensor, kv_indptr):
    if kv_indptr is not None or block_tables.dim() == 1:
        return 0, block_tables.stride(-1)
    return block_tables.stride(0), block_tables.stride(1)


def _need(t: Optional[torch.Tensor], name: str, dtype=None, ndim=None, shape=None,
          contiguous: bool = False, optional: bool = False):
    """Host-side checks the C ABI cannot make: element type, rank, shape and
    (for arrays the library indexes without strides) contiguity."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if dtype is not None:
        ok = t.dtype in dtype if isinstance(dtype, tuple) else t.dtype == dtype
        if not ok:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _same_gpu(stream, **tensors):
    """Every tensor must live on one GPU, the device of `stream` when it is a
    torch stream (the library hands their addresses to kernels on it)."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
    sdev = getattr(stream, "device", None)
    if dev is not None and sdev is not None and torch.device(sdev) != dev:
        raise ValueError(f"the tensors are on {dev}, the stream on {sdev}")


def _decode_args(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                 seq_lens, scale, max_seq_len, partition_size, num_splits, kv_indptr, kernel,
                 num_workers, alibi_slopes, k_scale, v_scale, num_group, stream,
                 max_num_parts=None) -> DecodeArgs:
    """Checked DecodeArgs for paged_attn_decode (workspaces given) or
    paged_attn_decode_static (workspaces None, max_num_parts given)."""
    _need(query, "query", tuple(_DTYPE), ndim=3)
    _need(key_cache, "key_cache", ndim=5)
    _need(value_cache, "value_cache", ndim=4)
    fp8 = key_cache.dtype in _FP8_CACHE
    if value_cache.dtype != key_cache.dtype or (not fp8 and key_cache.dtype != query.dtype):
        raise TypeError("key_cache and value_cache must share the query's dtype, or both be fp8 codes")
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.shape != (query.shape[1],) \
                or not alibi_slopes.is_contiguous():
            raise ValueError("alibi_slopes must be a contiguous fp32 tensor of shape [num_heads]")
    _need(seq_lens, "seq_lens", torch.int32, ndim=1, contiguous=True)
    R, H, D = query.shape
    S = seq_lens.shape[0]
    if num_group < 1 or R != S * num_group:
        raise ValueError(f"query has {R} rows, expected num_seqs * num_group = {S} * {num_group}")
    NB, Hkv, Dx, bs, x = key_cache.shape
    Dv = value_cache.shape[2]
    if max_num_parts is None:
        _need(tmp_output, "tmp_output", tuple(_DTYPE), ndim=4)
        P = tmp_output.shape[2]
        _need(tmp_output, "tmp_output", shape=(R, H, P, Dv))
        _need(exp_sums, "exp_sums", torch.float32, shape=(R, H, P))
        _need(max_logits, "max_logits", torch.float32, shape=(R, H, P))
    else:
        P = int(max_num_parts)
    _need(block_tables, "block_tables", torch.int32, ndim=1 if kv_indptr is not None else None)
    if kv_indptr is None and block_tables.dim() != 2:
        raise ValueError("block_tables must be [num_seqs, max_blocks] without kv_indptr")
    _need(kv_indptr, "kv_indptr", torch.int32, shape=(S + 1,), contiguous=True, optional=True)
    _need(num_splits, "num_splits", torch.int32, shape=(R,), contiguous=True, optional=True)
    _same_gpu(stream, tmp_output=tmp_output, exp_sums=exp_sums, max_logits=max_logits,
              query=query, key_cache=key_cache, value_cache=value_cache,
              block_tables=block_tables, seq_lens=seq_lens, kv_indptr=kv_indptr,
              num_splits=num_splits, alibi_slopes=alibi_slopes)
    a = DecodeArgs()
    if tmp_output is not None:
        a.tmp_output = _ptr(tmp_output)
        a.tmp_stride_s, a.tmp_stride_h, a.tmp_stride_p, a.tmp_stride_d = tmp_output.stride()
        a.tmp_dtype = _dtype(tmp_output)
        a.exp_sums = _ptr(exp_sums)
        a.max_logits = _ptr(max_logits)
        if exp_sums.stride() != max_logits.stride():
            raise ValueError("exp_sums and max_logits must share strides")
        a.ml_stride_s, a.ml_stride_h, a.ml_stride_p = exp_sums.stride()
    a.query = _ptr(query)
    a.q_stride_s, a.q_stride_h, a.q_stride_d = query.stride()
    a.key_cache = _ptr(key_cache)
    (a.k_stride_b, a.k_stride_h, a.k_stride_dx, a.k_stride_bs, a.k_stride_x) = key_cache.stride()
    a.value_cache = _ptr(value_cache)
    a.v_stride_b, a.v_stride_h, a.v_stride_d, a.v_stride_bs = value_cache.stride()
    a.block_tables = _ptr(block_tables)
    a.bt_stride_s, a.bt_stride_b = _page_strides(block_tables, kv_indptr)
    a.kv_indptr = _ptr(kv_indptr)
    a.seq_lens = _ptr(seq_lens)
    a.num_splits = _ptr(num_splits)
    a.scale = float(scale)
    a.num_seqs, a.num_heads, a.num_kv_heads = S, H, Hkv
    a.head_size, a.v_head_size, a.block_size, a.x = D, Dv, bs, x
    a.partition_size = partition_size
    a.max_num_parts = P
    a.max_seq_len = int(max_seq_len)
    a.dtype = _dtype(query)
    a.kernel_hint = PA_KERNEL[kernel]
    a.num_workers = num_workers
    a.alibi_slopes = _ptr(alibi_slopes)
    a.kv_dtype = PA_FP8_E4M3 if fp8 else 0
    a.k_scale, a.v_scale = float(k_scale), float(v_scale)
    a.num_group = num_group
    return a


def paged_attn_decode(tmp_output: torch.Tensor, exp_sums: torch.Tensor, max_logits: torch.Tensor,
                      query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                      block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                      max_seq_len: int, *, partition_size: int = 512,
                      num_splits: Optional[torch.Tensor] = None,
                      kv_indptr: Optional[torch.Tensor] = None, kernel: str = "auto",
                      num_workers: int = 0, alibi_slopes: Optional[torch.Tensor] = None,
                      k_scale: float = 1.0, v_scale: float = 1.0, num_group: int = 1,
                      stream=None) -> None:
    """Phase 1: per-split max logits, exp sums and normalised outputs.

    Shapes: tmp_output [S, H, P, Dv] fp32, f16 or bf16 (the split outputs
    are stored converted to its type); exp_sums / max_logits [S, H, P]
    fp32; query [S, H, D]; key_cache [NB, Hkv, D/x, bs, x]; value_cache
    [NB, Hkv, Dv, bs]; block_tables [S, max_blocks] int32 (or the flat page
    list when kv_indptr is given); seq_lens [S] int32. partition_size=0 with
    num_workers > 0 asks for balanced splits (equal token ranges).
    Caches of dtype uint8 or float8_e4m3fn hold FP8 E4M3 codes (x = 16),
    dequantized with k_scale / v_scale; alibi_slopes is an fp32 [H] tensor.
    num_group > 1: each sequence has num_group query tokens; query and the
    workspaces have num_seqs * num_group rows (row s * num_group + j) while
    seq_lens and the page lists stay per sequence.
    """
    lib = load_library()
    a = _decode_args(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                     seq_lens, scale, max_seq_len, partition_size, num_splits, kv_indptr, kernel,
                     num_workers, alibi_slopes, k_scale, v_scale, num_group, stream)
    _check(lib.paged_attn_decode(ctypes.byref(a), _stream(stream)))


def paged_attn_decode_kernel(tmp_output: torch.Tensor, exp_sums: torch.Tensor, max_logits: torch.Tensor,
                             query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                             block_tables: torch.Tensor, seq_lens: torch.Tensor, scale: float,
                             max_seq_len: int, *, partition_size: int = 512,
                             num_splits: Optional[torch.Tensor] = None,
                             kv_indptr: Optional[torch.Tensor] = None, kernel: str = "auto",
                             num_workers: int = 0, alibi_slopes: Optional[torch.Tensor] = None,
                             k_scale: float = 1.0, v_scale: float = 1.0, num_group: int = 1,
                             stream=None) -> str:
    """The phase-1 kernel paged_attn_decode would launch with these
    arguments ("valu", "mfma" or "mla"); nothing is launched."""
    lib = load_library()
    a = _decode_args(tmp_output, exp_sums, max_logits, query, key_cache, value_cache, block_tables,
                     seq_lens, scale, max_seq_len, partition_size, num_splits, kv_indptr, kernel,
                     num_workers, alibi_slopes, k_scale, v_scale, num_group, stream)
    rc = lib.paged_attn_decode_kernel(ctypes.byref(a))
    _check(min(rc, 0))
    return KERNEL_NAMES[rc]


def paged_attn_decode_static(output: torch.Tensor, query: torch.Tensor, key_cache: torch.Tensor,
                             value_cache: torch.Tensor, block_tables: torch.Tensor,
                             seq_lens: torch.Tensor, scale: float, max_seq_len: int, *,
                             max_num_parts: int, partition_size: int = 512,
                             num_splits: Optional[torch.Tensor] = None,
                             kv_indptr: Optional[torch.Tensor] = None, kernel: str = "auto",
                             num_workers: int = 0, alibi_slopes: Optional[torch.Tensor] = None,
                             k_scale: float = 1.0, v_scale: float = 1.0, num_group: int = 1,
                             tmp_dtype: torch.dtype = torch.float32, stream=None) -> None:
    """Phase 1 and phase 2 in one call with the split partials in the
    library's own device buffer (PA_STATIC_SCRATCH_BYTES per GPU), for
    callers that cannot allocate: output [S * num_group, H, Dv] receives the
    merged result. Arguments as for paged_attn_decode; max_num_parts sizes
    the partials, tmp_dtype is their element type. Overlapping calls on one
    GPU race on that buffer."""
    lib = load_library()
    a = _decode_args(None, None, None, query, key_cache, value_cache, block_tables, seq_lens, scale,
                     max_seq_len, partition_size, num_splits, kv_indptr, kernel, num_workers,
                     alibi_slopes, k_scale, v_scale, num_group, stream, max_num_parts=max_num_parts)
    if tmp_dtype not in _DTYPE:
        raise TypeError(f"tmp_dtype must be one of {tuple(_DTYPE)}, got {tmp_dtype}")
    a.tmp_dtype = _DTYPE[tmp_dtype]
    R, H, Dv = query.shape[0], query.shape[1], value_cache.shape[2]
    _need(output, "output", tuple(_DTYPE), shape=(R, H, Dv))
    if Dv > 1 and output.stride(2) != 1:
        raise ValueError("output rows must be contiguous (element stride 1)")
    _same_gpu(stream, output=output, query=query)
    _check(lib.paged_attn_decode_static(ctypes.byref(a), _ptr(output), output.stride(0),
                                        output.stride(1), _dtype(output), _stream(stream)))


def paged_attn_reduce(output: torch.Tensor, tmp_output: torch.Tensor, exp_sums: torch.Tensor,
                      max_logits: torch.Tensor, seq_lens: torch.Tensor, *,
                      partition_size: int = 512, num_splits: Optional[torch.Tensor] = None,
                      num_group: int = 1, stream=None) -> None:
    """Phase 2: log-sum-exp merge of the splits into output [S * num_group, H, Dv]."""
    lib = load_library()
    _need(tmp_output, "tmp_output", tuple(_DTYPE), ndim=4)
    _need(seq_lens, "seq_lens", torch.int32, ndim=1, contiguous=True)
    R, H, P, Dv = tmp_output.shape
    S = seq_lens.shape[0]
    if num_group < 1 or R != S * num_group:
        raise ValueError(f"tmp_output has {R} rows, expected num_seqs * num_group = {S} * {num_group}")
    _need(output, "output", tuple(_DTYPE), shape=(R, H, Dv))
    _need(exp_sums, "exp_sums", torch.float32, shape=(R, H, P))
    _need(max_logits, "max_logits", torch.float32, shape=(R, H, P))
    _need(num_splits, "num_splits", torch.int32, shape=(R,), contiguous=True, optional=True)
    _same_gpu(stream, output=output, tmp_output=tmp_output, exp_sums=exp_sums,
              max_logits=max_logits, seq_lens=seq_lens, num_splits=num_splits)
    a = ReduceArgs()
    a.output = _ptr(output)
    a.out_stride_s, a.out_stride_h, a.out_stride_d = output.stride()
    a.out_dtype = _dtype(output)
    a.tmp_output = _ptr(tmp_output)
    a.tmp_stride_s, a.tmp_stride_h, a.tmp_stride_p, a.tmp_stride_d = tmp_output.stride()
    a.tmp_dtype = _dtype(tmp_output)
    a.exp_sums = _ptr(exp_sums)
    a.max_logits = _ptr(max_logits)
    if exp_sums.stride() != max_logits.stride():
        raise ValueError("exp_sums and max_logits must share strides")
    a.ml_stride_s, a.ml_stride_h, a.ml_stride_p = exp_sums.stride()
    a.seq_lens = _ptr(seq_lens)
    a.num_splits = _ptr(num_splits)
    a.num_seqs, a.num_heads, a.v_head_size = S, H, Dv
    a.partition_size = partition_size
    a.max_num_parts = P
    a.num_group = num_group
    _check(lib.paged_attn_reduce(ctypes.byref(a), _stream(stream)))


def build_page_indices(page_indices: torch.Tensor, block_table: torch.Tensor,
                       cu_num_blocks: torch.Tensor, stream=None) -> None:
    """page_indices[cu[r] + i] = block_table[r, i] for i < cu[r+1] - cu[r]."""
    lib = load_library()
    _need(page_indices, "page_indices", torch.int32, ndim=1, contiguous=True)
    _need(block_table, "block_table", torch.int32, ndim=2)
    _need(cu_num_blocks, "cu_num_blocks", torch.int32, ndim=1, contiguous=True)
    if cu_num_blocks.shape[0] < 1:
        raise ValueError("cu_num_blocks must hold num_reqs + 1 >= 1 entries")
    _same_gpu(stream, page_indices=page_indices, block_table=block_table, cu_num_blocks=cu_num_blocks)
    num_reqs = cu_num_blocks.shape[0] - 1
    s0, s1 = block_table.stride()
    _check(lib.build_page_indices(_ptr(page_indices), _ptr(block_table), s0, s1,
                                  _ptr(cu_num_blocks), num_reqs, _stream(stream)))


def normal_decode_set_metadata(cache_seqlens: torch.Tensor, cu_seqlens_k: torch.Tensor,
                               page_table: torch.Tensor, req_to_token: torch.Tensor,
                               req_pool_indices: torch.Tensor, max_seq_pages: int,
                               seq_lens: torch.Tensor, seq_len_delta: int, page_size: int,
                               swa_page_table: Optional[torch.Tensor] = None,
                               full_to_swa: Optional[torch.Tensor] = None, stream=None) -> None:
    """Decode metadata in one launch (sglang metadata.py,
    normal_decode_set_metadata): cache_seqlens = int32(seq_lens + delta),
    cu_seqlens_k = their exclusive prefix sum, page_table[b, col] =
    req_to_token[req_pool_indices[b], col * page_size] // page_size, and the
    SWA table through full_to_swa when both SWA tensors are given. seq_lens
    and req_pool_indices are int64, the rest int32; any strides."""
    lib = load_library()
    for name, t, dt in (("cache_seqlens", cache_seqlens, torch.int32),
                        ("cu_seqlens_k", cu_seqlens_k, torch.int32),
                        ("page_table", page_table, torch.int32),
                        ("req_to_token", req_to_token, torch.int32),
                        ("req_pool_indices", req_pool_indices, torch.int64),
                        ("seq_lens", seq_lens, torch.int64),
                        ("swa_page_table", swa_page_table, torch.int32),
                        ("full_to_swa", full_to_swa, torch.int32)):
        if t is not None and t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
    _same_gpu(stream, cache_seqlens=cache_seqlens, cu_seqlens_k=cu_seqlens_k, page_table=page_table,
              req_to_token=req_to_token, req_pool_indices=req_pool_indices, seq_lens=seq_lens,
              swa_page_table=swa_page_table, full_to_swa=full_to_swa)
    B = seq_lens.shape[0]
    a = MetadataArgs()
    a.cache_seqlens, a.cache_seqlens_stride = _ptr(cache_seqlens), cache_seqlens.stride(0)
    a.cu_seqlens_k, a.cu_seqlens_k_stride = _ptr(cu_seqlens_k), cu_seqlens_k.stride(0)
    a.page_table = _ptr(page_table)
    a.page_table_stride0, a.page_table_stride1 = page_table.stride()
    if swa_page_table is not None:
        a.swa_page_table = _ptr(swa_page_table)
        a.swa_page_table_stride0, a.swa_page_table_stride1 = swa_page_table.stride()
    a.seq_lens, a.seq_lens_stride = _ptr(seq_lens), seq_lens.stride(0)
    a.req_to_token = _ptr(req_to_token)
    a.req_to_token_stride0, a.req_to_token_stride1 = req_to_token.stride()
    a.req_pool_indices, a.req_pool_indices_stride = _ptr(req_pool_indices), req_pool_indices.stride(0)
    if full_to_swa is not None:
        a.full_to_swa, a.full_to_swa_stride = _ptr(full_to_swa), full_to_swa.stride(0)
    a.batch, a.max_seq_pages, a.page_size = B, max_seq_pages, page_size
    a.seq_len_delta = seq_len_delta
    _check(lib.normal_decode_set_metadata(ctypes.byref(a), _stream(stream)))


def prepare_swa_spec_page_table(page_table_dst: torch.Tensor, page_table_a: torch.Tensor,
                                page_table_b: torch.Tensor, seq_len_a: torch.Tensor,
                                seq_len_b: torch.Tensor, speculative_num_draft_tokens: int,
                                stream=None) -> None:
    """Concatenate each request's page table with its draft rows' tables
    (sglang metadata.py, prepare_swa_spec_page_table_triton). All int32;
    page_table_dst is [bs * R, LEN_A + LEN_B]."""
    lib = load_library()
    for name, t in (("page_table_dst", page_table_dst), ("page_table_a", page_table_a),
                    ("page_table_b", page_table_b), ("seq_len_a", seq_len_a),
                    ("seq_len_b", seq_len_b)):
        if t.dtype != torch.int32:
            raise TypeError(f"{name} must be int32, got {t.dtype}")
    bs, R = seq_len_a.numel(), speculative_num_draft_tokens
    if seq_len_b.numel() != bs * R:
        raise ValueError("seq_len_b must hold bs * speculative_num_draft_tokens entries")
    if not (seq_len_a.is_contiguous() and seq_len_b.is_contiguous()):
        raise ValueError("seq_len_a and seq_len_b must be contiguous")
    _same_gpu(stream, page_table_dst=page_table_dst, page_table_a=page_table_a,
              page_table_b=page_table_b, seq_len_a=seq_len_a, seq_len_b=seq_len_b)
    LA, LB = page_table_a.shape[1], page_table_b.shape[1]
    if tuple(page_table_dst.shape) != (bs * R, LA + LB):
        raise ValueError(f"page_table_dst must be [{bs * R}, {LA + LB}]")
    _check(lib.prepare_swa_spec_page_table(
        _ptr(page_table_dst), *page_table_dst.stride(), _ptr(page_table_a), *page_table_a.stride(),
        _ptr(page_table_b), *page_table_b.stride(), _ptr(seq_len_a), _ptr(seq_len_b), bs, LA, LB, R,
        _stream(stream)))


def num_kv_splits(out: torch.Tensor, seq_lens: torch.Tensor, num_group: int, num_head: int,
                  num_kv_head: int, max_kv_splits: int, device_core_count: int,
                  stream=None) -> None:
    """Per-(seq, group) split counts from the sglang heuristic, on the device."""
    lib = load_library()
    _need(seq_lens, "seq_lens", torch.int32, ndim=1, contiguous=True)
    _need(out, "out", torch.int32, shape=(seq_lens.shape[0] * num_group,), contiguous=True)
    _same_gpu(stream, out=out, seq_lens=seq_lens)
    _check(lib.num_kv_splits(_ptr(out), _ptr(seq_lens), seq_lens.shape[0], num_group, num_head,
                             num_kv_head, max_kv_splits, device_core_count, _stream(stream)))


def paged_token_offsets(out: torch.Tensor, block_tables: torch.Tensor, seq_lens: torch.Tensor,
                        block_size: int, block_stride: int, slot_stride: int,
                        kv_indptr: Optional[torch.Tensor] = None, stream=None) -> None:
    """Test hook: out[s, t] = pages[t // bs] * block_stride + (t % bs) * slot_stride."""
    lib = load_library()
    _need(out, "out", torch.int64, ndim=2)
    if out.shape[1] > 1 and out.stride(1) != 1:
        raise ValueError("out rows must be contiguous (element stride 1)")
    S, max_len = out.shape
    _need(block_tables, "block_tables", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32, shape=(S,), contiguous=True)
    _need(kv_indptr, "kv_indptr", torch.int32, shape=(S + 1,), contiguous=True, optional=True)
    _same_gpu(stream, out=out, block_tables=block_tables, seq_lens=seq_lens, kv_indptr=kv_indptr)
    bs_s, bs_b = _page_strides(block_tables, kv_indptr)
    _check(lib.paged_token_offsets(_ptr(out), out.stride(0), _ptr(block_tables), bs_s, bs_b,
                                   _ptr(kv_indptr), _ptr(seq_lens), S, max_len, block_size,
                                   block_stride, slot_stride, _stream(stream)))


def read_probe(sink: torch.Tensor, base0: torch.Tensor, pages: torch.Tensor, runs_per_page: int,
               page_stride: int, run_stride: int, run_bytes: int,
               base1: Optional[torch.Tensor] = None, stream=None) -> None:
    """Plain read stream (measurement only, include/pagedattn_probe.h): reads
    run_bytes at base + pages[i] * page_stride + r * run_stride (bytes) for
    every page id, run r < runs_per_page and base in (base0, base1), folding
    the data into sink (uint32 [workgroups * 256 * 4]; workgroups = its
    length / 1024)."""
    lib = load_library()
    _need(pages, "pages", torch.int32, ndim=1, contiguous=True)
    _need(sink, "sink", (torch.int32, torch.uint32), ndim=1, contiguous=True)
    if sink.numel() % 1024:
        raise ValueError("sink must hold workgroups * 1024 uint32 entries")
    _same_gpu(stream, sink=sink, base0=base0, base1=base1, pages=pages)
    _check(lib.pa_read_probe(_ptr(base0), _ptr(base1), _ptr(pages), pages.numel(), runs_per_page,
                             page_stride, run_stride, run_bytes, _ptr(sink), sink.numel() // 1024,
                             _stream(stream)))
