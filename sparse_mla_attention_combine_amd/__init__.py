"""Python binding of libdsv4.so, the MI355X (gfx950) sparse MLA hot path.

Thin ctypes marshalling over the C ABI declared in ``include/dsv4.h``: each function
has the C entry point's name, takes torch tensors that already live on the GPU, passes
their device pointers and the current HIP stream, and raises on a non-zero status.
Every step of the path runs in the library's HIP kernels; there is no fallback.  If
the library has not been built the import fails (run
``python sparse_mla_attention_combine_amd/build.py``).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libdsv4.so")

LATENT_DIM, NOPE_DIM, ROPE_DIM, RECORD_BYTES, COMBINE_ALIGN = 576, 512, 64, 648, 128
# kv-cache dtypes (DSV4_KV_* of the C header): the packed FP8/UE8M0 record, bf16 records,
# E4M3 records with one per-tensor scale (kv_scale)
KV_FP8_DS_MLA, KV_BF16, KV_FP8_E4M3 = 0, 1, 2

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "`python sparse_mla_attention_combine_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _f32, _i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64

_lib.dsv4_status_str.argtypes, _lib.dsv4_status_str.restype = [_i32], ctypes.c_char_p
_lib.dsv4_last_error.argtypes, _lib.dsv4_last_error.restype = [], ctypes.c_char_p
_lib.dsv4_cache_page_bytes.argtypes = [_i32, _i32]
_lib.dsv4_cache_page_bytes.restype = ctypes.c_size_t
_lib.dsv4_kv_insert.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _vp, _i32, _i32, _i32,
                                _f32, _i32, _i32, _vp]
_lib.dsv4_combine_indices.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _vp, _i32, _vp, _vp]
_attn_head = [_vp, _vp, _i32, _i32, _i32, _f32, _vp, _i32, _vp, _vp, _f32, _vp, _vp, _i32, _i32]
_lib.dsv4_sparse_mla_decode.argtypes = _attn_head + [_vp, ctypes.c_size_t, _vp]
_lib.dsv4_sparse_mla_prefill.argtypes = _attn_head + [_vp, ctypes.c_size_t, _vp]
_lib.dsv4_sparse_mla_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
_lib.dsv4_sparse_mla_workspace_bytes.restype = ctypes.c_size_t
_lib.dsv4_gather_dequant.argtypes = [_vp, _i32, _i32, _i32, _f32, _vp, _i32, _vp, _vp]
_lib.dsv4_sparse_mla_split_workspace_bytes.argtypes = [_i32, _i32, _i32]
_lib.dsv4_sparse_mla_split_workspace_bytes.restype = ctypes.c_size_t
_lib.dsv4_sparse_mla_decode_split.argtypes = _attn_head + [_i32, _vp, ctypes.c_size_t, _vp]
_lib.dsv4_sparse_mla_decode_split_noalloc.argtypes = _attn_head + [_i32, _vp]
_lib.dsv4_combine_indices_compressed.argtypes = [_vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                                 _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp, _vp]
_lib.dsv4_sparse_mla_decode_topk.argtypes = [_vp, _vp, _i32, _i32, _i32, _f32, _vp, _i32, _i32,
                                             _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _f32,
                                             _vp, _vp, _i32, _i32, _vp]
_lib.dsv4_sparse_mla_decode_step.argtypes = [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _f32, _vp, _i32,
                                             _i32] + _lib.dsv4_sparse_mla_decode_topk.argtypes[4:]
_lib.dsv4_sparse_mla_decode_step_split.argtypes = (_lib.dsv4_sparse_mla_decode_step.argtypes[:-1]
                                                   + [_i32, _vp, ctypes.c_size_t, _vp])
_lib.dsv4_indexer_topk.argtypes = [_vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _i32, _vp,
                                   _vp]
_lib.dsv4_gather_workspace.argtypes = [_vp, _i32, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _vp,
                                       _i32, _i32, _i32, _i32, _vp, _i32, _vp]
_lib.dsv4_peak_mfma.argtypes = [_i32, _i32, _i32, _vp, ctypes.POINTER(ctypes.c_double), _vp]
_lib.dsv4_peak_stream.argtypes = [_vp, _vp, ctypes.c_size_t, _vp, _i32, _vp]
for _f in (_lib.dsv4_kv_insert, _lib.dsv4_combine_indices, _lib.dsv4_sparse_mla_decode,
           _lib.dsv4_sparse_mla_prefill, _lib.dsv4_gather_dequant, _lib.dsv4_sparse_mla_decode_split,
           _lib.dsv4_combine_indices_compressed, _lib.dsv4_gather_workspace,
           _lib.dsv4_indexer_topk, _lib.dsv4_sparse_mla_decode_topk,
           _lib.dsv4_sparse_mla_decode_step, _lib.dsv4_sparse_mla_decode_step_split,
           _lib.dsv4_sparse_mla_decode_split_noalloc, _lib.dsv4_peak_mfma, _lib.dsv4_peak_stream):
    _f.restype = _i32

EXPORTED = ["dsv4_status_str", "dsv4_last_error", "dsv4_cache_page_bytes", "dsv4_kv_insert",
            "dsv4_combine_indices", "dsv4_sparse_mla_decode", "dsv4_sparse_mla_prefill",
            "dsv4_gather_dequant", "dsv4_sparse_mla_split_workspace_bytes",
            "dsv4_sparse_mla_decode_split", "dsv4_combine_indices_compressed",
            "dsv4_gather_workspace", "dsv4_indexer_topk", "dsv4_sparse_mla_decode_topk",
            "dsv4_sparse_mla_decode_step", "dsv4_sparse_mla_decode_step_split",
            "dsv4_sparse_mla_workspace_bytes", "dsv4_sparse_mla_decode_split_noalloc",
            "dsv4_peak_mfma", "dsv4_peak_stream"]

NOALLOC_SCRATCH_BYTES = 32 << 20


class Dsv4Error(RuntimeError):
    def __init__(self, status: int, reason: str):
        super().__init__(f"{_lib.dsv4_status_str(status).decode()}: {reason}")
        self.status = status
        self.reason = reason


def library() -> ctypes.CDLL:
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise Dsv4Error(status, _lib.dsv4_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise TypeError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise TypeError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _want(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def cache_page_bytes(page_size: int = 64, kv_dtype: int = KV_FP8_DS_MLA) -> int:
    return int(_lib.dsv4_cache_page_bytes(page_size, kv_dtype))


def new_cache(num_pages: int, page_size: int = 64, device="cuda",
              kv_dtype: int = KV_FP8_DS_MLA) -> torch.Tensor:
    """Zero-filled uint8 cache of ``num_pages`` pages (caller-owned device memory)."""
    return torch.zeros(num_pages * cache_page_bytes(page_size, kv_dtype), dtype=torch.uint8,
                       device=device)


def _num_pages(kv_cache, page_size, kv_dtype):
    pb = cache_page_bytes(page_size, kv_dtype)
    return kv_cache.numel() // pb if pb else 0


def dsv4_kv_insert(q, kv, positions, slot_mapping, cos_sin, q_norm_weight, eps, kv_cache,
                   page_size=64, stream=None, kv_dtype=KV_FP8_DS_MLA, kv_scale=1.0):
    """q bf16 [T, H, 576] (in place), kv bf16 [T, 576], positions/slot_mapping int64 [T],
    cos_sin fp32 [max_pos, 64], q_norm_weight bf16 [576], kv_cache uint8 pages of
    kv_dtype (kv_scale: the per-tensor scale of a KV_FP8_E4M3 cache)."""
    _want(q, torch.bfloat16, "q"), _want(kv, torch.bfloat16, "kv")
    _want(positions, torch.int64, "positions"), _want(slot_mapping, torch.int64, "slot_mapping")
    _want(cos_sin, torch.float32, "cos_sin"), _want(q_norm_weight, torch.bfloat16, "q_norm_weight")
    _want(kv_cache, torch.uint8, "kv_cache")
    T, H = (q.shape[0], q.shape[1]) if q is not None else (kv.shape[0], 0)
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    _check(_lib.dsv4_kv_insert(_ptr(q) if H else None, _ptr(kv), _ptr(positions),
                               _ptr(slot_mapping), _ptr(cos_sin), cos_sin.shape[0],
                               _ptr(q_norm_weight) if H else None, float(eps), _ptr(kv_cache),
                               num_pages, page_size, int(kv_dtype), float(kv_scale), T, H,
                               _stream(stream)))
    return q


def dsv4_combine_indices(topk, topk_lens, query_start_loc, seq_lens, block_table, top_k, window,
                         combined, combined_lens, page_size=64, topk_width=None, stream=None):
    """topk int32 [T, width], topk_lens int32 [T] or None, query_start_loc int32 [B+1],
    seq_lens int32 [B], block_table int32 [B, pages]; writes combined int32
    [T, stride] and combined_lens int32 [T]."""
    for t, n in ((topk, "topk"), (topk_lens, "topk_lens"), (query_start_loc, "query_start_loc"),
                 (seq_lens, "seq_lens"), (block_table, "block_table"), (combined, "combined"),
                 (combined_lens, "combined_lens")):
        _want(t, torch.int32, n)
    T = combined.shape[0]
    B = seq_lens.shape[0]
    width = topk.shape[1] if topk_width is None else topk_width
    _check(_lib.dsv4_combine_indices(_ptr(topk), topk.shape[1], width, _ptr(topk_lens),
                                     _ptr(query_start_loc), _ptr(seq_lens), _ptr(block_table),
                                     block_table.shape[1], B, T, top_k, window, page_size,
                                     _ptr(combined), combined.shape[1], _ptr(combined_lens),
                                     _stream(stream)))


def dsv4_combine_indices_compressed(topk, topk_lens, query_start_loc, seq_lens, gather_lens,
                                    top_k, compress_ratio, window, M, N, combined, combined_lens,
                                    topk_width=None, stream=None):
    """Compressed-cache form of the combine: writes combined int32 [T, stride] (indices
    into a per-request workspace of M rows: N compressed entries, then gathered raw
    tokens) and combined_lens int32 [T]."""
    for t, n in ((topk, "topk"), (topk_lens, "topk_lens"), (query_start_loc, "query_start_loc"),
                 (seq_lens, "seq_lens"), (gather_lens, "gather_lens"), (combined, "combined"),
                 (combined_lens, "combined_lens")):
        _want(t, torch.int32, n)
    T, B = combined.shape[0], seq_lens.shape[0]
    width = topk.shape[1] if topk_width is None else topk_width
    _check(_lib.dsv4_combine_indices_compressed(
        _ptr(topk), topk.shape[1], width, _ptr(topk_lens), _ptr(query_start_loc), _ptr(seq_lens),
        _ptr(gather_lens), B, T, top_k, compress_ratio, window, M, N, _ptr(combined),
        combined.shape[1], _ptr(combined_lens), _stream(stream)))


def dsv4_indexer_topk(logits, query_start_loc, seq_lens, top_k, topk, topk_lens, compress_ratio=1,
                      stream=None):
    """logits fp32 [T, n] per-token indexer scores -> topk int32 [T, stride] (the top_k
    largest causal candidates, ascending ids, -1 padded) and topk_lens int32 [T]."""
    _want(logits, torch.float32, "logits")
    for t, n in ((query_start_loc, "query_start_loc"), (seq_lens, "seq_lens"), (topk, "topk"),
                 (topk_lens, "topk_lens")):
        _want(t, torch.int32, n)
    _check(_lib.dsv4_indexer_topk(_ptr(logits), logits.shape[1], _ptr(query_start_loc),
                                  _ptr(seq_lens), seq_lens.shape[0], topk.shape[0], compress_ratio,
                                  top_k, _ptr(topk), topk.shape[1], _ptr(topk_lens),
                                  _stream(stream)))


def dsv4_gather_workspace(comp_cache, comp_block_table, swa_cache, swa_block_table, seq_lens,
                          gather_lens, compress_ratio, M, N, ws_cache, page_size=64, stream=None):
    """Fills ws_cache (uint8 pages) with the workspace rows the compressed-form indices
    address: compressed entries through comp_block_table, raw tokens through
    swa_block_table (int32 [B, stride] each)."""
    for t, n in ((comp_cache, "comp_cache"), (swa_cache, "swa_cache"), (ws_cache, "ws_cache")):
        _want(t, torch.uint8, n)
    for t, n in ((comp_block_table, "comp_block_table"), (swa_block_table, "swa_block_table"),
                 (seq_lens, "seq_lens"), (gather_lens, "gather_lens")):
        _want(t, torch.int32, n)
    pb = cache_page_bytes(page_size)
    _check(_lib.dsv4_gather_workspace(
        _ptr(comp_cache), comp_cache.numel() // pb, _ptr(comp_block_table), comp_block_table.shape[1],
        _ptr(swa_cache), swa_cache.numel() // pb, _ptr(swa_block_table), swa_block_table.shape[1],
        page_size, _ptr(seq_lens), _ptr(gather_lens), seq_lens.shape[0], compress_ratio, M, N,
        _ptr(ws_cache), ws_cache.numel() // pb, _stream(stream)))
    return ws_cache


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _attention(fn, q, kv_cache, indices, lens, sinks, softmax_scale, out, lse, page_size,
               workspace, stream, kv_dtype, kv_scale):
    _want(q, torch.bfloat16, "q"), _want(kv_cache, torch.uint8, "kv_cache")
    _want(indices, torch.int32, "indices"), _want(lens, torch.int32, "lens")
    _want(sinks, torch.float32, "sinks"), _want(out, torch.bfloat16, "out")
    _want(lse, torch.float32, "lse")
    T, H = q.shape[0], q.shape[1]
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    _check(fn(_ptr(q), _ptr(kv_cache), num_pages, page_size, int(kv_dtype), float(kv_scale),
              _ptr(indices), indices.shape[1],
              _ptr(lens), _ptr(sinks), float(softmax_scale), _ptr(out), _ptr(lse), T, H,
              _ptr(workspace), _nbytes(workspace), _stream(stream)))
    return out


def workspace_bytes(T, H, width, prefill=False):
    """Device workspace bytes dsv4_sparse_mla_decode (or _prefill) may use."""
    return int(_lib.dsv4_sparse_mla_workspace_bytes(T, H, width, int(bool(prefill))))


def dsv4_sparse_mla_decode(q, kv_cache, indices, lens, sinks, softmax_scale, out, lse=None,
                           page_size=64, workspace=None, stream=None, kv_dtype=KV_FP8_DS_MLA,
                           kv_scale=1.0):
    """q bf16 [T, H, 576], indices int32 [T, stride] physical slots, lens int32 [T],
    sinks fp32 [H] or None -> out bf16 [T, H, 512] (and lse fp32 [T, H] if given).
    workspace: None, or a device tensor of at least workspace_bytes(T, H, stride) bytes
    (lets a small batch run its rows in pieces)."""
    return _attention(_lib.dsv4_sparse_mla_decode, q, kv_cache, indices, lens, sinks,
                      softmax_scale, out, lse, page_size, workspace, stream, kv_dtype, kv_scale)


def dsv4_sparse_mla_prefill(q, kv_cache, indices, lens, sinks, softmax_scale, out, lse=None,
                            page_size=64, workspace=None, stream=None, kv_dtype=KV_FP8_DS_MLA,
                            kv_scale=1.0):
    """Same contract as dsv4_sparse_mla_decode, scheduled for many query tokens."""
    return _attention(_lib.dsv4_sparse_mla_prefill, q, kv_cache, indices, lens, sinks,
                      softmax_scale, out, lse, page_size, workspace, stream, kv_dtype, kv_scale)


def dsv4_sparse_mla_decode_topk(q, kv_cache, topk, topk_lens, query_start_loc, seq_lens,
                                block_table, top_k, window, sinks, softmax_scale, out, lse=None,
                                page_size=64, topk_width=None, stream=None,
                                kv_dtype=KV_FP8_DS_MLA, kv_scale=1.0):
    """dsv4_combine_indices + dsv4_sparse_mla_decode in one launch (the combined rows are
    built in LDS): q bf16 [T, H, 576], topk int32 [T, width], topk_lens int32 [T] or None,
    query_start_loc int32 [B+1], seq_lens int32 [B], block_table int32 [B, pages] ->
    out bf16 [T, H, 512] (and lse fp32 [T, H] if given)."""
    _want(q, torch.bfloat16, "q"), _want(kv_cache, torch.uint8, "kv_cache")
    for t, n in ((topk, "topk"), (topk_lens, "topk_lens"), (query_start_loc, "query_start_loc"),
                 (seq_lens, "seq_lens"), (block_table, "block_table")):
        _want(t, torch.int32, n)
    _want(sinks, torch.float32, "sinks"), _want(out, torch.bfloat16, "out")
    _want(lse, torch.float32, "lse")
    T, H = q.shape[0], q.shape[1]
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    width = topk.shape[1] if topk_width is None else topk_width
    _check(_lib.dsv4_sparse_mla_decode_topk(
        _ptr(q), _ptr(kv_cache), num_pages, page_size, int(kv_dtype), float(kv_scale), _ptr(topk),
        topk.shape[1], width,
        _ptr(topk_lens), _ptr(query_start_loc), _ptr(seq_lens), _ptr(block_table),
        block_table.shape[1], seq_lens.shape[0], top_k, window, _ptr(sinks), float(softmax_scale),
        _ptr(out), _ptr(lse), T, H, _stream(stream)))
    return out


def dsv4_sparse_mla_decode_step(q, kv, positions, slot_mapping, cos_sin, q_norm_weight, eps,
                                kv_cache, topk, topk_lens, query_start_loc, seq_lens, block_table,
                                top_k, window, sinks, softmax_scale, out, lse=None, page_size=64,
                                topk_width=None, splits=1, workspace=None, stream=None,
                                kv_dtype=KV_FP8_DS_MLA, kv_scale=1.0):
    """dsv4_kv_insert + dsv4_sparse_mla_decode_topk in one launch: the arguments of the
    two (q normalised in place, the new kv rows inserted into kv_cache) -> out bf16
    [T, H, 512] (and lse fp32 [T, H] if given).  splits > 1: rows cut into pieces merged
    by their lse (dsv4_sparse_mla_decode_step_split), with a device workspace of at least
    split_workspace_bytes(T, H, splits) bytes."""
    _want(q, torch.bfloat16, "q"), _want(kv, torch.bfloat16, "kv")
    _want(positions, torch.int64, "positions"), _want(slot_mapping, torch.int64, "slot_mapping")
    _want(cos_sin, torch.float32, "cos_sin"), _want(q_norm_weight, torch.bfloat16, "q_norm_weight")
    _want(kv_cache, torch.uint8, "kv_cache")
    for t, n in ((topk, "topk"), (topk_lens, "topk_lens"), (query_start_loc, "query_start_loc"),
                 (seq_lens, "seq_lens"), (block_table, "block_table")):
        _want(t, torch.int32, n)
    _want(sinks, torch.float32, "sinks"), _want(out, torch.bfloat16, "out")
    _want(lse, torch.float32, "lse")
    T, H = q.shape[0], q.shape[1]
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    width = topk.shape[1] if topk_width is None else topk_width
    args = (_ptr(q), _ptr(kv), _ptr(positions), _ptr(slot_mapping), _ptr(cos_sin),
            cos_sin.shape[0], _ptr(q_norm_weight), float(eps), _ptr(kv_cache), num_pages,
            page_size, int(kv_dtype), float(kv_scale), _ptr(topk), topk.shape[1], width, _ptr(topk_lens), _ptr(query_start_loc),
            _ptr(seq_lens), _ptr(block_table), block_table.shape[1], seq_lens.shape[0], top_k,
            window, _ptr(sinks), float(softmax_scale), _ptr(out), _ptr(lse), T, H)
    if splits == 1:
        _check(_lib.dsv4_sparse_mla_decode_step(*args, _stream(stream)))
    else:
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(_lib.dsv4_sparse_mla_decode_step_split(*args, splits, _ptr(workspace), ws_bytes,
                                                      _stream(stream)))
    return out


def split_workspace_bytes(T, H, splits):
    """Device workspace bytes dsv4_sparse_mla_decode_split needs."""
    return int(_lib.dsv4_sparse_mla_split_workspace_bytes(T, H, splits))


def dsv4_sparse_mla_decode_split(q, kv_cache, indices, lens, sinks, softmax_scale, out, splits,
                                 workspace, lse=None, page_size=64, stream=None,
                                 kv_dtype=KV_FP8_DS_MLA, kv_scale=1.0):
    """dsv4_sparse_mla_decode with each token's row cut into `splits` pieces merged by
    their lse; workspace: a caller-owned device tensor of at least
    split_workspace_bytes(T, H, splits) bytes (16-byte aligned)."""
    _want(q, torch.bfloat16, "q"), _want(kv_cache, torch.uint8, "kv_cache")
    _want(indices, torch.int32, "indices"), _want(lens, torch.int32, "lens")
    _want(sinks, torch.float32, "sinks"), _want(out, torch.bfloat16, "out")
    _want(lse, torch.float32, "lse")
    T, H = q.shape[0], q.shape[1]
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.dsv4_sparse_mla_decode_split(
        _ptr(q), _ptr(kv_cache), num_pages, page_size, int(kv_dtype), float(kv_scale), _ptr(indices), indices.shape[1], _ptr(lens),
        _ptr(sinks), float(softmax_scale), _ptr(out), _ptr(lse), T, H, int(splits), _ptr(workspace),
        ws_bytes, _stream(stream)))
    return out


def dsv4_sparse_mla_decode_split_noalloc(q, kv_cache, indices, lens, sinks, softmax_scale, out,
                                         splits, lse=None, page_size=64, stream=None,
                                         kv_dtype=KV_FP8_DS_MLA, kv_scale=1.0):
    """dsv4_sparse_mla_decode_split with its workspace in the library's static per-GPU
    scratch array (no allocation; split_workspace_bytes(T, H, splits) must fit
    NOALLOC_SCRATCH_BYTES).  Calls that overlap on one GPU race."""
    _want(q, torch.bfloat16, "q"), _want(kv_cache, torch.uint8, "kv_cache")
    _want(indices, torch.int32, "indices"), _want(lens, torch.int32, "lens")
    _want(sinks, torch.float32, "sinks"), _want(out, torch.bfloat16, "out")
    _want(lse, torch.float32, "lse")
    T, H = q.shape[0], q.shape[1]
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    _check(_lib.dsv4_sparse_mla_decode_split_noalloc(
        _ptr(q), _ptr(kv_cache), num_pages, page_size, int(kv_dtype), float(kv_scale), _ptr(indices), indices.shape[1], _ptr(lens),
        _ptr(sinks), float(softmax_scale), _ptr(out), _ptr(lse), T, H, int(splits),
        _stream(stream)))
    return out


def dsv4_gather_dequant(kv_cache, slots, out, page_size=64, stream=None, kv_dtype=KV_FP8_DS_MLA,
                        kv_scale=1.0):
    """slots int32 [n] -> out bf16 [n, 576] (dequantised rows; zeros for invalid slots)."""
    _want(kv_cache, torch.uint8, "kv_cache"), _want(slots, torch.int32, "slots")
    _want(out, torch.bfloat16, "out")
    num_pages = _num_pages(kv_cache, page_size, kv_dtype)
    _check(_lib.dsv4_gather_dequant(_ptr(kv_cache), num_pages, page_size, int(kv_dtype),
                                    float(kv_scale), _ptr(slots), slots.shape[0], _ptr(out),
                                    _stream(stream)))
    return out


def dsv4_peak_mfma(shape, iters, sink, stream=None):
    """Matrix-core probe: sink fp32 [workgroups * 256] (workgroups = sink.numel() // 256);
    shape 0 = 32x32x16, 1 = 16x16x32 bf16 MFMAs.  Returns the launch's dense FLOPs."""
    _want(sink, torch.float32, "sink")
    flops = ctypes.c_double(0.0)
    _check(_lib.dsv4_peak_mfma(int(shape), sink.numel() // 256, int(iters), _ptr(sink),
                               ctypes.byref(flops), _stream(stream)))
    return flops.value


def dsv4_peak_stream(src, sink, dst=None, stream=None):
    """HBM probe: reads src (its bytes) and, if dst is given, copies it there; sink int32
    [workgroups * 256] receives each thread's xor of what it read (read-only)."""
    _want(sink, torch.int32, "sink")
    n = _nbytes(src)
    if dst is not None and _nbytes(dst) < n:
        raise ValueError("dst is smaller than src")
    _check(_lib.dsv4_peak_stream(_ptr(src), None if dst is None else _ptr(dst), n, _ptr(sink),
                                 sink.numel() // 256, _stream(stream)))
