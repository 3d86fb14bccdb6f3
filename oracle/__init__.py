"""CPU oracle for the sparse MLA hot path (ctypes wrapper over ``oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` are the only callers.  The product path
(``sparse_mla_attention_combine_amd``) never imports this package.

Every function takes and returns numpy arrays.  bf16 data travels as ``uint16``
bit patterns; FP8 codes and cache pages as ``uint8``.  Results of the attention
step are fp64.  The C source cites the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

LATENT, NOPE, ROPE, RECORD = 576, 512, 64, 648
# kv-cache dtypes: the packed FP8 record with UE8M0 block scales, plain bf16 records,
# plain E4M3 records with one per-tensor scale
KV_FP8_DS, KV_BF16, KV_FP8_E4M3 = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (plain C, fp64, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-pthread", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.oracle_e4m3_decode.argtypes, L.oracle_e4m3_decode.restype = [i32], dbl
        L.oracle_e4m3_encode.argtypes, L.oracle_e4m3_encode.restype = [dbl], i32
        L.oracle_bf16_from_double.argtypes, L.oracle_bf16_from_double.restype = [dbl], ctypes.c_uint16
        L.oracle_bf16_to_double.argtypes, L.oracle_bf16_to_double.restype = [ctypes.c_uint16], dbl
        L.oracle_ue8m0_exponent.argtypes, L.oracle_ue8m0_exponent.restype = [dbl], i32
        L.oracle_gather_dequant.argtypes = [vp, i32, i32, vp, i32, vp]
        L.oracle_gather_dequant_kv.argtypes = [vp, i32, i32, i32, dbl, vp, i32, vp]
        L.oracle_kv_record_bytes.argtypes, L.oracle_kv_record_bytes.restype = [i32], i32
        L.oracle_combine.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                     vp, i32, vp]
        L.oracle_combine_compressed.argtypes = [vp, i32, i32, vp, vp, vp, vp, i32, i32, i32, i32,
                                                i32, i32, i32, vp, i32, vp]
        L.oracle_gather_workspace.argtypes = [vp, i32, vp, i32, vp, i32, vp, i32, i32, vp, vp, i32,
                                              i32, i32, i32, vp, i32]
        L.oracle_indexer_topk.argtypes = [vp, i32, vp, vp, i32, i32, i32, i32, vp, i32, vp]
        L.oracle_kv_insert.argtypes = [vp, vp, vp, vp, vp, i32, vp, dbl, vp, i32, i32, i32, i32]
        L.oracle_kv_insert_kv.argtypes = [vp, vp, vp, vp, vp, i32, vp, dbl, vp, i32, i32, i32, dbl,
                                          i32, i32]
        L.oracle_sparse_mla.argtypes = [vp, vp, i32, i32, vp, i32, vp, vp, dbl, vp, vp, i32, i32,
                                        i32]
        L.oracle_sparse_mla_kv.argtypes = [vp, vp, i32, i32, i32, dbl, vp, i32, vp, vp, dbl, vp, vp,
                                           i32, i32, i32]
        for f in (L.oracle_gather_dequant, L.oracle_gather_dequant_kv, L.oracle_combine,
                  L.oracle_combine_compressed, L.oracle_gather_workspace, L.oracle_indexer_topk,
                  L.oracle_kv_insert, L.oracle_kv_insert_kv, L.oracle_sparse_mla,
                  L.oracle_sparse_mla_kv):
            f.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# ---- codecs -------------------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(x: float) -> int:
    return lib().oracle_e4m3_encode(float(x))


def bf16_from_double(x: float) -> int:
    return lib().oracle_bf16_from_double(float(x))


def bf16_to_double(b: int) -> float:
    return lib().oracle_bf16_to_double(int(b))


def ue8m0_exponent(amax: float) -> int:
    return lib().oracle_ue8m0_exponent(float(amax))


# ---- steps ----------------------------------------------------------------------------

def kv_record_bytes(kv_dtype: int = KV_FP8_DS) -> int:
    """Bytes of one slot's record in a cache of ``kv_dtype``."""
    return lib().oracle_kv_record_bytes(int(kv_dtype))


def gather_dequant(cache: np.ndarray, num_pages: int, page_size: int, slots: np.ndarray,
                   kv_dtype: int = KV_FP8_DS, kv_scale: float = 1.0) -> np.ndarray:
    """bf16 bits [n, 576] of the dequantised records of ``slots`` (zeros when invalid)."""
    slots = _c(slots, np.int32)
    out = np.zeros((slots.shape[0], LATENT), np.uint16)
    if kv_dtype == KV_FP8_DS:
        lib().oracle_gather_dequant(_ptr(cache), num_pages, page_size, _ptr(slots), slots.shape[0],
                                    _ptr(out))
    else:
        lib().oracle_gather_dequant_kv(_ptr(cache), num_pages, page_size, int(kv_dtype),
                                       float(kv_scale), _ptr(slots), slots.shape[0], _ptr(out))
    return out


def combine(topk, topk_lens, qsl, seq_lens, block_table, T, top_k, window, page_size,
            combined_stride, topk_width=None, fill=-7):
    """Combined index rows ``[T, combined_stride]`` and lengths ``[T]``.

    Rows of tokens no request covers keep the ``fill`` value (the step does not
    write them)."""
    topk = _c(topk, np.int32)
    tl = _c(topk_lens, np.int32)
    qsl = _c(qsl, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    bt = _c(block_table, np.int32)
    B = seq_lens.shape[0]
    out = np.full((T, combined_stride), fill, np.int32)
    lens = np.full((T,), fill, np.int32)
    width = topk.shape[1] if topk_width is None else topk_width
    lib().oracle_combine(_ptr(topk), topk.shape[1], width, _ptr(tl), _ptr(qsl), _ptr(seq_lens),
                         _ptr(bt), bt.shape[1], B, T, top_k, window, page_size, _ptr(out),
                         combined_stride, _ptr(lens))
    return out, lens


def combine_compressed(topk, topk_lens, qsl, seq_lens, gather_lens, T, top_k, ratio, window, M, N,
                       combined_stride, topk_width=None, fill=-7):
    """Combined rows ``[T, combined_stride]`` and lengths ``[T]`` in the workspace index
    space of the compressed-cache form (request b owns rows ``M*b .. M*b+M-1``)."""
    topk = _c(topk, np.int32)
    tl = _c(topk_lens, np.int32)
    qsl, seq_lens, gl = _c(qsl, np.int32), _c(seq_lens, np.int32), _c(gather_lens, np.int32)
    B = seq_lens.shape[0]
    out = np.full((T, combined_stride), fill, np.int32)
    lens = np.full((T,), fill, np.int32)
    width = topk.shape[1] if topk_width is None else topk_width
    lib().oracle_combine_compressed(_ptr(topk), topk.shape[1], width, _ptr(tl), _ptr(qsl),
                                    _ptr(seq_lens), _ptr(gl), B, T, top_k, ratio, window, M, N,
                                    _ptr(out), combined_stride, _ptr(lens))
    return out, lens


def gather_workspace(comp_cache, comp_num_pages, comp_bt, swa_cache, swa_num_pages, swa_bt,
                     page_size, seq_lens, gather_lens, ratio, M, N, ws_num_pages, ws=None):
    """The workspace cache (``ws_num_pages`` pages) those indices address."""
    comp_bt, swa_bt = _c(comp_bt, np.int32), _c(swa_bt, np.int32)
    seq_lens, gl = _c(seq_lens, np.int32), _c(gather_lens, np.int32)
    out = (np.full(ws_num_pages * page_size * RECORD, 0xA5, np.uint8) if ws is None
           else np.array(ws, np.uint8, copy=True))
    lib().oracle_gather_workspace(_ptr(_c(comp_cache, np.uint8)), comp_num_pages, _ptr(comp_bt),
                                  comp_bt.shape[1], _ptr(_c(swa_cache, np.uint8)), swa_num_pages,
                                  _ptr(swa_bt), swa_bt.shape[1], page_size, _ptr(seq_lens),
                                  _ptr(gl), seq_lens.shape[0], ratio, M, N, _ptr(out), ws_num_pages)
    return out


def indexer_topk(logits, qsl, seq_lens, T, ratio, top_k, topk_stride, fill=-7):
    """Top-k candidate ids ``[T, topk_stride]`` (ascending, -1 padded) and their counts
    ``[T]`` from per-token indexer logits ``[T, n]`` (fp32); rows of tokens no request
    covers keep ``fill``."""
    lg = _c(logits, np.float32)
    qsl, seq_lens = _c(qsl, np.int32), _c(seq_lens, np.int32)
    out = np.full((T, topk_stride), fill, np.int32)
    lens = np.full((T,), fill, np.int32)
    lib().oracle_indexer_topk(_ptr(lg), lg.shape[1], _ptr(qsl), _ptr(seq_lens), seq_lens.shape[0],
                              T, ratio, top_k, _ptr(out), topk_stride, _ptr(lens))
    return out, lens


def kv_insert(q_bits, kv_bits, positions, slot_mapping, cos_sin, weight_bits, eps, cache,
              num_pages, page_size, inplace=False, kv_dtype=KV_FP8_DS, kv_scale=1.0):
    """Returns (q_out_bits, cache_out); works on copies unless ``inplace`` (then q_bits and
    cache must be C-contiguous uint16 / uint8 arrays and are updated)."""
    if inplace:
        q, c = q_bits, cache
        assert q.dtype == np.uint16 and c.dtype == np.uint8
    else:
        q = np.array(q_bits, dtype=np.uint16, order="C", copy=True)
        c = np.array(cache, dtype=np.uint8, order="C", copy=True)
    kv = _c(kv_bits, np.uint16)
    pos = _c(positions, np.int64)
    sm = _c(slot_mapping, np.int64)
    cs = _c(cos_sin, np.float32)
    w = _c(weight_bits, np.uint16)
    T, H = q.shape[0], q.shape[1]
    if kv_dtype == KV_FP8_DS:
        lib().oracle_kv_insert(_ptr(q), _ptr(kv), _ptr(pos), _ptr(sm), _ptr(cs), cs.shape[0],
                               _ptr(w), float(eps), _ptr(c), num_pages, page_size, T, H)
    else:
        lib().oracle_kv_insert_kv(_ptr(q), _ptr(kv), _ptr(pos), _ptr(sm), _ptr(cs), cs.shape[0],
                                  _ptr(w), float(eps), _ptr(c), num_pages, page_size,
                                  int(kv_dtype), float(kv_scale), T, H)
    return q, c


def sparse_mla(q_bits, cache, num_pages, page_size, indices, lens, sinks, scale, nthreads=1,
               with_lse=True, kv_dtype=KV_FP8_DS, kv_scale=1.0):
    """fp64 outputs ``[T, H, 512]`` and lse ``[T, H]`` (or None)."""
    q = _c(q_bits, np.uint16)
    idx = _c(indices, np.int32)
    ln = _c(lens, np.int32)
    sk = _c(sinks, np.float32)
    T, H = q.shape[0], q.shape[1]
    out = np.zeros((T, H, NOPE), np.float64)
    lse = np.zeros((T, H), np.float64) if with_lse else None
    if kv_dtype == KV_FP8_DS:
        lib().oracle_sparse_mla(_ptr(q), _ptr(cache), num_pages, page_size, _ptr(idx),
                                idx.shape[1], _ptr(ln), _ptr(sk), float(scale), _ptr(out),
                                _ptr(lse), T, H, int(nthreads))
    else:
        lib().oracle_sparse_mla_kv(_ptr(q), _ptr(cache), num_pages, page_size, int(kv_dtype),
                                   float(kv_scale), _ptr(idx), idx.shape[1], _ptr(ln), _ptr(sk),
                                   float(scale), _ptr(out), _ptr(lse), T, H, int(nthreads))
    return out, lse
