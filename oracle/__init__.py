"""Plain CPU oracle for split-KV PagedAttention decode (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the GPU library
(``paged_attention_decode_tables_amd``) and never imports it; the GPU library
never imports this.

The arithmetic lives in ``oracle.c`` (plain C, fp64 accumulation); this module
only builds it with gcc, loads it with ctypes and converts numpy arrays.
Each function names the page passage it follows; see the header of
``oracle.c`` for the list of pages and the readings taken where they are
silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")


def lib_path(mutant: int = 0) -> str:
    name = "liboracle.so" if mutant == 0 else f"liboracle_mutant{mutant}.so"
    return os.path.join(_HERE, name)


def build(mutant: int = 0, openmp: bool = True) -> str:
    """Compile oracle.c with gcc (mutant > 0 builds a planted-mistake variant)."""
    out = lib_path(mutant)
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", _SRC, "-o", out + ".tmp", "-lm"]
    if openmp:
        cmd.insert(1, "-fopenmp")
    if mutant:
        cmd.insert(1, f"-DORACLE_MUTANT={mutant}")
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_I32P = ctypes.POINTER(ctypes.c_int32)
_I64P = ctypes.POINTER(ctypes.c_int64)
_F32P = ctypes.POINTER(ctypes.c_float)
_F64P = ctypes.POINTER(ctypes.c_double)
_U8P = ctypes.POINTER(ctypes.c_uint8)
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def _ptr(a: Optional[np.ndarray], ctype):
    if a is None:
        return ctypes.cast(None, ctype)
    return a.ctypes.data_as(ctype)


def _estrides(a: np.ndarray):
    return tuple(s // a.itemsize for s in a.strides)


class Oracle:
    """ctypes wrapper around one build of oracle.c."""

    def __init__(self, path: Optional[str] = None, mutant: int = 0):
        path = path or lib_path(mutant)
        if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
            build(mutant)
        self.lib = ctypes.CDLL(path)
        L = self.lib
        L.orc_token_offsets.argtypes = [_I64P, _I64, _I32P, _I64, _I64, _I32P, _I32P, _I32, _I32, _I64, _I64]
        L.orc_page_indices.argtypes = [_I32P, _I32P, _I64, _I64, _I32P, _I32]
        L.orc_num_kv_splits.argtypes = [_I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32]
        common = [_F32P, _I64, _I64, _F32P, _I64, _I64, _F32P, _I64, _I64,
                  _I32P, _I64, _I64, _I32P, _I32P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                  ctypes.c_double]
        L.orc_attention.argtypes = [_F64P] + common
        ext = [_F32P, _U8P, _U8P, ctypes.c_double, ctypes.c_double]
        L.orc_attention_v.argtypes = [_F64P] + common + ext
        L.orc_partials.argtypes = [_F64P, _F64P, _F64P] + common + [_I32P, _I32, _I32]
        L.orc_partials_v.argtypes = [_F64P, _F64P, _F64P] + common + [_I32P, _I32, _I32] + ext
        L.orc_reduce.argtypes = [_F64P, _F64P, _F64P, _F64P, _I32P, _I32P, _I32, _I32, _I32, _I32, _I32]
        L.orc_decode_metadata.argtypes = [_I32P, _I64, _I32P, _I64, _I32P, _I64, _I64,
                                          _I32P, _I64, _I64, _I64P, _I64, _I32P, _I64, _I64,
                                          _I64P, _I64, _I32P, _I64, _I32, _I32, _I32, _I64]
        L.orc_swa_spec_page_table.argtypes = [_I32P, _I64, _I64, _I32P, _I64, _I64, _I32P, _I64, _I64,
                                              _I32P, _I32P, _I32, _I32, _I32, _I32]
        self.mutant = L.orc_mutant_id()

    # -- integer helpers ----------------------------------------------------
    def token_offsets(self, pages, seq_lens, block_size, block_stride=1, slot_stride=1,
                      indptr=None, fill=-1):
        """[S, max_len] int64: offset of token t of sequence s (Triton issue
        2522, block-table example), -1 where t >= seq_len."""
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        S = seq_lens.shape[0]
        max_len = int(max(1, seq_lens.max(initial=0)))
        out = np.full((S, max_len), fill, dtype=np.int64)
        pages = np.asarray(pages, dtype=np.int32)
        if pages.ndim == 1:
            ps, pb = 0, _estrides(pages)[0]
        else:
            ps, pb = _estrides(pages)
        ip = None if indptr is None else np.ascontiguousarray(indptr, dtype=np.int32)
        rc = self.lib.orc_token_offsets(_ptr(out, _I64P), max_len, _ptr(pages, _I32P), ps, pb,
                                        _ptr(ip, _I32P), _ptr(seq_lens, _I32P), S, block_size,
                                        block_stride, slot_stride)
        assert rc == 0, rc
        return out

    def page_indices(self, block_table, cu_num_blocks, fill=-1):
        """Flat page list (vLLM PR 35765, _copy_page_indices_kernel)."""
        block_table = np.asarray(block_table, dtype=np.int32)
        cu = np.ascontiguousarray(cu_num_blocks, dtype=np.int32)
        nreq = cu.shape[0] - 1
        out = np.full((max(int(cu[-1]), 0) if nreq >= 0 else 0,), fill, dtype=np.int32)
        s0, s1 = _estrides(block_table) if block_table.ndim == 2 else (0, 1)
        rc = self.lib.orc_page_indices(_ptr(out, _I32P), _ptr(block_table, _I32P), s0, s1,
                                       _ptr(cu, _I32P), max(nreq, 0))
        assert rc == 0, rc
        return out

    def num_kv_splits(self, seq_lens, num_group, num_head, num_kv_head, max_kv_splits,
                      device_core_count):
        """Per-(seq, group) split counts (sglang metadata.py,
        get_num_kv_splits_triton)."""
        seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        out = np.zeros(seq_lens.shape[0] * num_group, dtype=np.int32)
        rc = self.lib.orc_num_kv_splits(_ptr(out, _I32P), _ptr(seq_lens, _I32P), seq_lens.shape[0],
                                        num_group, num_head, num_kv_head, max_kv_splits,
                                        device_core_count)
        if rc != 0:
            raise ValueError(f"orc_num_kv_splits: invalid arguments (rc={rc})")
        return out

    def decode_metadata(self, seq_lens, req_to_token, req_pool_indices, max_seq_pages,
                        page_size, seq_len_delta=0, full_to_swa=None):
        """Decode metadata (sglang metadata.py, normal_decode_set_metadata):
        returns (cache_seqlens [B] int32, cu_seqlens_k [B+1] int32,
        page_table [B, max_seq_pages] int32, swa_page_table or None). Inputs
        may be strided numpy views; seq_lens and req_pool_indices are int64,
        req_to_token and full_to_swa int32."""
        seq_lens = np.asarray(seq_lens)
        assert seq_lens.dtype == np.int64 and seq_lens.ndim == 1
        B = seq_lens.shape[0]
        rt = np.asarray(req_to_token)
        assert rt.dtype == np.int32 and rt.ndim == 2
        rpi = np.asarray(req_pool_indices)
        assert rpi.dtype == np.int64 and rpi.shape == (B,)
        cs = np.zeros(B, dtype=np.int32)
        cu = np.zeros(B + 1, dtype=np.int32)
        pt = np.full((B, max_seq_pages), -7, dtype=np.int32)
        swa = None
        f2s_stride = 0
        if full_to_swa is not None:
            full_to_swa = np.asarray(full_to_swa)
            assert full_to_swa.dtype == np.int32 and full_to_swa.ndim == 1
            f2s_stride = _estrides(full_to_swa)[0]
            swa = np.full((B, max_seq_pages), -7, dtype=np.int32)
        rc = self.lib.orc_decode_metadata(
            _ptr(cs, _I32P), 1, _ptr(cu, _I32P), 1, _ptr(pt, _I32P), max(max_seq_pages, 1), 1,
            _ptr(swa, _I32P), max(max_seq_pages, 1), 1,
            _ptr(seq_lens, _I64P), _estrides(seq_lens)[0],
            _ptr(rt, _I32P), *_estrides(rt), _ptr(rpi, _I64P), _estrides(rpi)[0],
            _ptr(full_to_swa, _I32P), f2s_stride, B, max_seq_pages, page_size, seq_len_delta)
        if rc != 0:
            raise ValueError(f"orc_decode_metadata: invalid arguments (rc={rc})")
        return cs, cu, pt, swa

    def swa_spec_page_table(self, page_table_a, page_table_b, seq_len_a, seq_len_b,
                            draft_tokens, fill=-1):
        """Speculative SWA page table (sglang metadata.py,
        prepare_swa_spec_page_table_triton): [bs * R, LEN_A + LEN_B] int32,
        `fill` where nothing is written. Inputs may be strided int32 views."""
        a = np.asarray(page_table_a)
        b = np.asarray(page_table_b)
        la = np.ascontiguousarray(seq_len_a, dtype=np.int32)
        lb = np.ascontiguousarray(seq_len_b, dtype=np.int32)
        assert a.dtype == np.int32 and b.dtype == np.int32 and a.ndim == 2 and b.ndim == 2
        bs = la.shape[0]
        assert lb.shape[0] == bs * draft_tokens
        out = np.full((bs * draft_tokens, a.shape[1] + b.shape[1]), fill, dtype=np.int32)
        rc = self.lib.orc_swa_spec_page_table(_ptr(out, _I32P), max(out.shape[1], 1), 1,
                                              _ptr(a, _I32P), *_estrides(a), _ptr(b, _I32P),
                                              *_estrides(b), _ptr(la, _I32P), _ptr(lb, _I32P), bs,
                                              a.shape[1], b.shape[1], draft_tokens)
        if rc != 0:
            raise ValueError(f"orc_swa_spec_page_table: invalid arguments (rc={rc})")
        return out

    # -- attention ----------------------------------------------------------
    def _problem(self, query, key_cache, value_cache, pages, seq_lens, scale, indptr):
        q = np.asarray(query, dtype=np.float32)
        kc = np.asarray(key_cache)
        vc = np.asarray(value_cache)
        fp8 = kc.dtype == np.uint8  # fp8 E4M3 codes (both caches)
        assert (vc.dtype == np.uint8) == fp8
        if not fp8:
            kc = kc.astype(np.float32, copy=False)
            vc = vc.astype(np.float32, copy=False)
        assert q.ndim == 3 and kc.ndim == 5 and vc.ndim == 4
        qs = _estrides(q)
        ks = _estrides(kc)
        vs = _estrides(vc)
        S, H, D = q.shape
        NB, Hkv, Dx, bs, x = kc.shape
        Dv = vc.shape[2]
        assert Dx * x == D and vc.shape[3] == bs
        # inner dims must be packed (the C code walks them directly)
        assert qs[2] == 1 and ks[2:] == (bs * x, x, 1) and vs[2:] == (bs, 1), (qs, ks, vs)
        pages = np.asarray(pages, dtype=np.int32)
        if indptr is not None:
            ip = np.ascontiguousarray(indptr, dtype=np.int32)
            ps, pb = 0, _estrides(pages)[0]
        else:
            ip = None
            ps, pb = _estrides(pages)
        seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
        args = [_ptr(q, _F32P), qs[0], qs[1], None if fp8 else _ptr(kc, _F32P), ks[0], ks[1],
                None if fp8 else _ptr(vc, _F32P), vs[0], vs[1], _ptr(pages, _I32P), ps, pb,
                _ptr(ip, _I32P), _ptr(seq, _I32P), S, H, Hkv, D, Dv, bs, x, float(scale)]
        keep = (q, kc, vc, pages, ip, seq)
        self._codes = (kc, vc) if fp8 else (None, None)
        return args, keep, (S, H, Dv)

    def _variant(self, alibi, k_scale, v_scale):
        """Extra arguments of the _v entry points, or None for the plain ones."""
        kc, vc = self._codes
        if alibi is None and kc is None:
            return None
        al = None if alibi is None else np.ascontiguousarray(alibi, dtype=np.float32)
        self._alibi = al
        return [_ptr(al, _F32P), None if kc is None else kc.ctypes.data_as(_U8P),
                None if vc is None else vc.ctypes.data_as(_U8P), float(k_scale), float(v_scale)]

    def attention(self, query, key_cache, value_cache, pages, seq_lens, scale, indptr=None,
                  alibi=None, k_scale=1.0, v_scale=1.0):
        """[S, H, Dv] float64 softmax attention of each query over its paged
        K/V rows (paged_attention_v2_triton.py, phase-1 docstring steps 1-4
        applied to the whole sequence). alibi: optional slopes [H]; uint8
        caches are fp8 E4M3 codes dequantized with k_scale / v_scale."""
        args, keep, (S, H, Dv) = self._problem(query, key_cache, value_cache, pages, seq_lens,
                                               scale, indptr)
        out = np.empty((S, H, Dv), dtype=np.float64)
        ext = self._variant(alibi, k_scale, v_scale)
        if ext is None:
            rc = self.lib.orc_attention(_ptr(out, _F64P), *args)
        else:
            rc = self.lib.orc_attention_v(_ptr(out, _F64P), *args, *ext)
        assert rc == 0, rc
        return out

    def partials(self, query, key_cache, value_cache, pages, seq_lens, scale, max_num_parts,
                 partition_size=512, num_splits=None, indptr=None, alibi=None, k_scale=1.0,
                 v_scale=1.0):
        """Phase-1 intermediates (tmp [S,H,P,Dv], max_logits, exp_sums
        [S,H,P]) in float64; tmp of empty partitions is NaN."""
        args, keep, (S, H, Dv) = self._problem(query, key_cache, value_cache, pages, seq_lens,
                                               scale, indptr)
        tmp = np.full((S, H, max_num_parts, Dv), np.nan, dtype=np.float64)
        ml = np.empty((S, H, max_num_parts), dtype=np.float64)
        es = np.empty((S, H, max_num_parts), dtype=np.float64)
        ns = None if num_splits is None else np.ascontiguousarray(num_splits, dtype=np.int32)
        ext = self._variant(alibi, k_scale, v_scale)
        if ext is None:
            rc = self.lib.orc_partials(_ptr(tmp, _F64P), _ptr(ml, _F64P), _ptr(es, _F64P), *args,
                                       _ptr(ns, _I32P), partition_size, max_num_parts)
        else:
            rc = self.lib.orc_partials_v(_ptr(tmp, _F64P), _ptr(ml, _F64P), _ptr(es, _F64P), *args,
                                         _ptr(ns, _I32P), partition_size, max_num_parts, *ext)
        assert rc == 0, rc
        return tmp, ml, es

    def reduce(self, tmp, max_logits, exp_sums, seq_lens, partition_size=512, num_splits=None):
        """Phase-2 log-sum-exp merge (paged_attention_v2_triton.py,
        _paged_attn_v2_reduce_kernel) -> [S, H, Dv] float64."""
        tmp = np.ascontiguousarray(tmp, dtype=np.float64)
        ml = np.ascontiguousarray(max_logits, dtype=np.float64)
        es = np.ascontiguousarray(exp_sums, dtype=np.float64)
        S, H, P, Dv = tmp.shape
        seq = np.ascontiguousarray(seq_lens, dtype=np.int32)
        ns = None if num_splits is None else np.ascontiguousarray(num_splits, dtype=np.int32)
        out = np.empty((S, H, Dv), dtype=np.float64)
        rc = self.lib.orc_reduce(_ptr(out, _F64P), _ptr(tmp, _F64P), _ptr(ml, _F64P),
                                 _ptr(es, _F64P), _ptr(seq, _I32P), _ptr(ns, _I32P),
                                 partition_size, S, H, Dv, P)
        assert rc == 0, rc
        return out


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The real (unmutated) oracle, built on first use."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
