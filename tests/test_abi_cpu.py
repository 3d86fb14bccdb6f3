"""The C-ABI library loads, exports every symbol include/dsv4.h declares, and rejects
bad arguments on the host (these calls return before any HIP call, so they run
without a GPU)."""
import ctypes
import os
import re

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dsv4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsv4_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(dsv4):
    lib = dsv4.library()
    names = declared_functions()
    assert {"dsv4_kv_insert", "dsv4_combine_indices", "dsv4_sparse_mla_decode",
            "dsv4_sparse_mla_prefill", "dsv4_gather_dequant"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dsv4.EXPORTED)


def test_status_strings_and_page_bytes(dsv4):
    lib = dsv4.library()
    assert lib.dsv4_status_str(0) == b"DSV4_OK"
    assert lib.dsv4_status_str(4) == b"DSV4_ERR_UNSUPPORTED"
    assert lib.dsv4_cache_page_bytes(64, 0) == 64 * 648
    assert lib.dsv4_cache_page_bytes(32, 1) == 32 * 1152
    assert lib.dsv4_cache_page_bytes(256, 2) == 256 * 576
    assert lib.dsv4_cache_page_bytes(0, 0) == 0
    assert lib.dsv4_cache_page_bytes(64, 3) == 0


def _fake(n=1 << 20):
    """A host buffer only used as a non-NULL, aligned address (never dereferenced:
    every call below fails validation before any launch)."""
    buf = (ctypes.c_uint8 * (n + 64))()
    addr = ctypes.addressof(buf)
    return buf, ctypes.c_void_p((addr + 63) // 64 * 64)


def test_attention_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()
    args = dict(q=p, cache=p, num_pages=4, page_size=64, kvd=0, kvs=1.0, idx=p, stride=128,
                lens=p, sinks=None, scale=0.04, out=p, lse=None, T=2, H=16)

    def call(fn, **kw):
        a = dict(args, ws=None, wsb=0, **kw)
        return fn(a["q"], a["cache"], a["num_pages"], a["page_size"], a["kvd"], a["kvs"],
                  a["idx"], a["stride"], a["lens"], a["sinks"], a["scale"], a["out"], a["lse"],
                  a["T"], a["H"], a["ws"], a["wsb"], None)

    for fn in (lib.dsv4_sparse_mla_decode, lib.dsv4_sparse_mla_prefill):
        assert call(fn, H=24) == 4 and b"H = 24" in lib.dsv4_last_error()
        for bad in (16, 48, 128, 0, -64):
            assert call(fn, page_size=bad) == 4
        assert call(fn, q=None) == 1
        assert call(fn, lens=None) == 1
        assert call(fn, T=-1) == 2
        assert call(fn, num_pages=-3) == 2
        assert call(fn, out=ctypes.c_void_p(p.value + 2)) == 3
        assert call(fn, T=0, q=None) == 0 and lib.dsv4_last_error() == b""
        # cache dtypes: unknown -> unsupported; the fp8 cache's scale must be in range
        assert call(fn, kvd=3) == 4 and b"kv_dtype" in lib.dsv4_last_error()
        assert call(fn, kvd=-1) == 4
        for bad in (0.0, -1.0, float("nan"), float("inf"), 2.0 ** -70, 2.0 ** 70):
            assert call(fn, kvd=2, kvs=bad) == 2 and b"kv_scale" in lib.dsv4_last_error()
        assert call(fn, kvd=1, kvs=0.0, T=0, q=None) == 0   # the scale is the fp8 cache's only
        assert call(fn, kvd=2, kvs=0.5, T=0, q=None) == 0


def test_attention_workspace_contract(dsv4):
    """dsv4_sparse_mla_workspace_bytes: 0 for a batch that fills the GPU and for prefill,
    the split workspace of the chosen piece count otherwise; the decode / prefill reject
    a short, misaligned or inconsistent workspace before launching anything."""
    lib = dsv4.library()
    wsb = lib.dsv4_sparse_mla_workspace_bytes
    split = lib.dsv4_sparse_mla_split_workspace_bytes
    assert wsb(64, 128, 2176, 0) == 0              # 256 workgroups: no split
    assert wsb(8192, 64, 2176, 1) == 0             # prefill: never
    assert wsb(8, 128, 2176, 1) == 0
    assert wsb(8, 128, 2176, 0) == split(8, 128, 8)  # 32 workgroups -> 8 pieces
    assert wsb(32, 128, 2176, 0) == split(32, 128, 2)
    assert wsb(8, 128, 600, 0) == split(8, 128, 2)   # pieces of >= 256 entries
    assert wsb(8, 128, 255, 0) == 0
    assert wsb(2, 16, 4096, 0) == split(2, 16, 8)
    assert wsb(-1, 128, 2176, 0) == 0 and wsb(8, 24, 2176, 0) == 0 and wsb(8, 128, -1, 0) == 0
    keep, p = _fake()
    need = wsb(2, 16, 4096, 0)

    def call(fn, **kw):
        a = dict(q=p, cache=p, num_pages=4, page_size=64, idx=p, stride=4096, lens=p, sinks=None,
                 scale=0.04, out=p, lse=None, T=2, H=16, ws=p, wsb=need)
        a.update(kw)
        return fn(a["q"], a["cache"], a["num_pages"], a["page_size"], 0, 1.0, a["idx"],
                  a["stride"], a["lens"], a["sinks"], a["scale"], a["out"], a["lse"], a["T"],
                  a["H"], a["ws"], a["wsb"], None)

    for fn in (lib.dsv4_sparse_mla_decode, lib.dsv4_sparse_mla_prefill):
        assert call(fn, T=0, q=None) == 0
        assert call(fn, ws=None, wsb=16) == 5 and b"NULL" in lib.dsv4_last_error()
        assert call(fn, ws=ctypes.c_void_p(p.value + 8), T=0) == 5
    assert call(lib.dsv4_sparse_mla_decode, wsb=need - 1) == 5  # fails before any launch
    assert b"hold" in lib.dsv4_last_error()
    assert call(lib.dsv4_sparse_mla_prefill, wsb=0, T=0) == 0   # prefill needs none
    assert call(lib.dsv4_sparse_mla_decode, H=24) == 4


def test_noalloc_split_decode_validation(dsv4):
    """The entry point without a workspace argument refuses a size past its static array
    (32 MiB) and a bad piece count before launching anything."""
    lib = dsv4.library()
    keep, p = _fake()

    def call(**kw):
        a = dict(T=2, H=16, splits=4, stride=128, kvd=0, kvs=1.0)
        a.update(kw)
        return lib.dsv4_sparse_mla_decode_split_noalloc(
            p, p, 4, 64, a["kvd"], a["kvs"], p, a["stride"], p, None, 0.04, p, None, a["T"],
            a["H"], a["splits"], None)

    assert dsv4.NOALLOC_SCRATCH_BYTES == 32 << 20
    assert lib.dsv4_sparse_mla_split_workspace_bytes(64, 128, 8) > dsv4.NOALLOC_SCRATCH_BYTES
    assert call(T=64, H=128, splits=8) == 5 and b"static scratch" in lib.dsv4_last_error()
    assert call(splits=0) == 2 and call(splits=65) == 2
    assert call(H=24) == 4
    assert call(kvd=5) == 4 and call(kvd=2, kvs=-2.0) == 2
    assert call(T=0) == 0


def test_split_decode_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()
    need = lib.dsv4_sparse_mla_split_workspace_bytes(2, 16, 4)
    assert need == 2 * 4 * 16 * 514 * 4
    assert lib.dsv4_sparse_mla_split_workspace_bytes(-1, 16, 4) == 0

    def call(**kw):
        a = dict(q=p, cache=p, num_pages=4, page_size=64, idx=p, stride=128, lens=p, sinks=None,
                 scale=0.04, out=p, lse=None, T=2, H=16, splits=4, ws=p, wsb=need, kvd=0, kvs=1.0)
        a.update(kw)
        return lib.dsv4_sparse_mla_decode_split(a["q"], a["cache"], a["num_pages"], a["page_size"],
                                                a["kvd"], a["kvs"],
                                                a["idx"], a["stride"], a["lens"], a["sinks"],
                                                a["scale"], a["out"], a["lse"], a["T"], a["H"],
                                                a["splits"], a["ws"], a["wsb"], None)

    assert call(splits=0) == 2 and b"splits 0" in lib.dsv4_last_error()
    assert call(splits=65) == 2
    assert call(ws=None) == 5 and b"workspace" in lib.dsv4_last_error()
    assert call(wsb=need - 4) == 5
    assert call(ws=ctypes.c_void_p(p.value + 4)) == 5
    assert call(H=24) == 4
    assert call(q=None) == 1
    assert call(kvd=7) == 4 and call(kvd=2, kvs=float("nan")) == 2
    assert call(T=0, q=None) == 0
    assert lib.dsv4_status_str(5) == b"DSV4_ERR_WORKSPACE"


def test_combine_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()

    def call(**kw):
        a = dict(topk=p, ts=2048, tw=2048, tl=None, qsl=p, sl=p, bt=p, bts=512, B=64, T=64,
                 top_k=2048, window=128, P=64, comb=p, cs=2176, cl=p)
        a.update(kw)
        return lib.dsv4_combine_indices(a["topk"], a["ts"], a["tw"], a["tl"], a["qsl"], a["sl"],
                                        a["bt"], a["bts"], a["B"], a["T"], a["top_k"], a["window"],
                                        a["P"], a["comb"], a["cs"], a["cl"], None)

    assert call(cs=2100) == 2 and b"2176" in lib.dsv4_last_error()
    assert call(top_k=4096) == 2
    assert call(P=128) == 4
    assert call(qsl=None) == 1
    assert call(ts=100, tw=2048) == 2
    assert call(T=0) == 0


def test_compressed_combine_and_workspace_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()

    def comb(**kw):
        a = dict(topk=p, ts=512, tw=512, tl=None, qsl=p, sl=p, gl=p, B=4, T=4, top_k=512, r=4,
                 window=128, M=4096, N=2048, comb=p, cs=640, cl=p)
        a.update(kw)
        return lib.dsv4_combine_indices_compressed(
            a["topk"], a["ts"], a["tw"], a["tl"], a["qsl"], a["sl"], a["gl"], a["B"], a["T"],
            a["top_k"], a["r"], a["window"], a["M"], a["N"], a["comb"], a["cs"], a["cl"], None)

    assert comb(r=0) == 2 and b"compress_ratio" in lib.dsv4_last_error()
    assert comb(N=5000) == 2
    assert comb(N=-1) == 2
    assert comb(B=1 << 20, M=1 << 12) == 2
    assert comb(cs=600) == 2
    assert comb(top_k=600) == 2
    assert comb(gl=None) == 1
    assert comb(comb=ctypes.c_void_p(p.value + 2)) == 3
    assert comb(T=0) == 0

    def ws(**kw):
        a = dict(cc=p, cn=4, cbt=p, cbs=8, sc=p, sn=4, sbt=p, sbs=8, P=64, sl=p, gl=p, B=2, r=4,
                 M=300, N=100, ws=p, wn=10)
        a.update(kw)
        return lib.dsv4_gather_workspace(a["cc"], a["cn"], a["cbt"], a["cbs"], a["sc"], a["sn"],
                                         a["sbt"], a["sbs"], a["P"], a["sl"], a["gl"], a["B"], a["r"],
                                         a["M"], a["N"], a["ws"], a["wn"], None)

    assert ws(P=128) == 4
    assert ws(r=0) == 2
    assert ws(N=301) == 2
    assert ws(cn=-1) == 2
    assert ws(sl=None) == 1
    assert ws(ws=None) == 1
    assert ws(ws=ctypes.c_void_p(p.value + 8)) == 3
    assert ws(B=0) == 0 and ws(wn=0) == 0


def test_indexer_topk_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()

    def call(**kw):
        a = dict(lg=p, ls=4096, qsl=p, sl=p, B=2, T=2, r=1, k=2048, out=p, os=2048, ol=p)
        a.update(kw)
        return lib.dsv4_indexer_topk(a["lg"], a["ls"], a["qsl"], a["sl"], a["B"], a["T"], a["r"],
                                     a["k"], a["out"], a["os"], a["ol"], None)

    assert call(r=0) == 2
    assert call(os=100) == 2 and b"topk_stride" in lib.dsv4_last_error()
    assert call(k=-1) == 2
    assert call(qsl=None) == 1
    assert call(lg=None) == 1
    assert call(out=ctypes.c_void_p(p.value + 2)) == 3
    assert call(T=0) == 0


def test_decode_topk_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()

    def call(**kw):
        a = dict(q=p, cache=p, npg=4, P=64, topk=p, ts=2048, tw=2048, tl=None, qsl=p, sl=p, bt=p,
                 bts=8, B=2, top_k=2048, window=128, sinks=None, scale=0.04, out=p, lse=None, T=2,
                 H=128, kvd=0, kvs=1.0)
        a.update(kw)
        return lib.dsv4_sparse_mla_decode_topk(
            a["q"], a["cache"], a["npg"], a["P"], a["kvd"], a["kvs"], a["topk"], a["ts"], a["tw"], a["tl"], a["qsl"],
            a["sl"], a["bt"], a["bts"], a["B"], a["top_k"], a["window"], a["sinks"], a["scale"],
            a["out"], a["lse"], a["T"], a["H"], None)

    assert call(window=2049) == 4 and b"4096" in lib.dsv4_last_error()
    assert call(H=24) == 4
    assert call(P=48) == 4
    assert call(top_k=3000) == 2
    assert call(qsl=None) == 1
    assert call(out=ctypes.c_void_p(p.value + 2)) == 3
    assert call(kvd=3) == 4 and call(kvd=2, kvs=0.0) == 2
    assert call(T=0) == 0


def test_decode_step_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()

    def call(**kw):
        a = dict(q=p, kv=p, pos=p, sm=p, cs=p, maxp=100, w=p, eps=1e-6, cache=p, npg=4, P=64,
                 topk=p, ts=2048, tw=2048, tl=None, qsl=p, sl=p, bt=p, bts=8, B=2, top_k=2048,
                 window=128, sinks=None, scale=0.04, out=p, lse=None, T=2, H=128, kvd=0, kvs=1.0)
        a.update(kw)
        return lib.dsv4_sparse_mla_decode_step(
            a["q"], a["kv"], a["pos"], a["sm"], a["cs"], a["maxp"], a["w"], a["eps"], a["cache"],
            a["npg"], a["P"], a["kvd"], a["kvs"], a["topk"], a["ts"], a["tw"], a["tl"], a["qsl"], a["sl"], a["bt"],
            a["bts"], a["B"], a["top_k"], a["window"], a["sinks"], a["scale"], a["out"], a["lse"],
            a["T"], a["H"], None)

    assert call(window=2049) == 4 and b"4096" in lib.dsv4_last_error()
    assert call(H=24) == 4
    assert call(P=48) == 4
    assert call(top_k=3000) == 2
    assert call(maxp=-1) == 2
    assert call(eps=-1.0) == 2
    assert call(kv=None) == 1
    assert call(w=None) == 1
    assert call(cs=None) == 1
    assert call(q=ctypes.c_void_p(p.value + 8)) == 3
    assert call(pos=ctypes.c_void_p(p.value + 4)) == 3
    assert call(kvd=3) == 4 and call(kvd=2, kvs=float("inf")) == 2
    assert call(T=0) == 0


def test_decode_step_split_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()
    need = lib.dsv4_sparse_mla_split_workspace_bytes(2, 128, 4)

    def call(**kw):
        a = dict(S=4, ws=p, wsb=need, T=2, H=128, window=128, P=64)
        a.update(kw)
        return lib.dsv4_sparse_mla_decode_step_split(
            p, p, p, p, p, 100, p, 1e-6, p, 4, a["P"], 0, 1.0, p, 2048, 2048, None, p, p, p, 8, 2, 2048,
            a["window"], None, 0.04, p, None, a["T"], a["H"], a["S"], a["ws"], a["wsb"], None)

    assert call(S=0) == 4 and call(S=65) == 4
    assert call(wsb=need - 1) == 5
    assert call(ws=None) == 5
    assert call(ws=ctypes.c_void_p(p.value + 8)) == 5
    assert call(window=2049) == 4
    assert call(H=24) == 4
    assert call(P=48) == 4
    assert call(T=0) == 0
    # B = 2 requests: more than 64 query tokens per request on average is refused (the
    # step re-quantises a request's new rows in every workgroup of its tokens)
    assert call(T=129) == 4 and b"query tokens per request" in lib.dsv4_last_error()
    assert call(T=128) == 5  # within the bound: the workspace check comes next


def test_insert_and_gather_validation(dsv4):
    lib = dsv4.library()
    keep, p = _fake()

    def ins(**kw):
        a = dict(q=p, kv=p, pos=p, sm=p, cs=p, maxp=100, w=p, eps=1e-6, cache=p, npg=4, P=64, T=4,
                 H=8, kvd=0, kvs=1.0)
        a.update(kw)
        return lib.dsv4_kv_insert(a["q"], a["kv"], a["pos"], a["sm"], a["cs"], a["maxp"], a["w"],
                                  a["eps"], a["cache"], a["npg"], a["P"], a["kvd"], a["kvs"],
                                  a["T"], a["H"], None)

    assert ins(H=129) == 2
    assert ins(P=16) == 4
    assert ins(kv=None) == 1
    assert ins(q=None) == 1
    assert ins(q=None, w=None, H=0, kv=None) == 1
    assert ins(eps=-1.0) == 2
    assert ins(q=ctypes.c_void_p(p.value + 8)) == 3
    assert ins(kvd=4) == 4 and ins(kvd=2, kvs=0.0) == 2 and b"kv_scale" in lib.dsv4_last_error()
    assert ins(T=0) == 0 and ins(T=0, kvd=1) == 0
    assert lib.dsv4_gather_dequant(p, 4, 64, 0, 1.0, None, 5, p, None) == 1
    assert lib.dsv4_gather_dequant(p, 4, 64, 0, 1.0, p, -1, p, None) == 2
    assert lib.dsv4_gather_dequant(p, 4, 48, 0, 1.0, p, 5, p, None) == 4
    assert lib.dsv4_gather_dequant(p, 4, 64, 9, 1.0, p, 5, p, None) == 4
    assert lib.dsv4_gather_dequant(p, 4, 64, 2, -1.0, p, 5, p, None) == 2
    assert lib.dsv4_gather_dequant(p, 4, 64, 0, 1.0, p, 0, p, None) == 0


def test_binding_rejects_host_tensors(dsv4):
    import pytest
    import torch
    q = torch.zeros(1, 16, 576, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        dsv4.dsv4_sparse_mla_decode(q, torch.zeros(64 * 648, dtype=torch.uint8),
                                    torch.zeros(1, 128, dtype=torch.int32),
                                    torch.zeros(1, dtype=torch.int32), None, 0.04,
                                    torch.zeros(1, 16, 512, dtype=torch.bfloat16))


def test_peak_probe_validation(dsv4):
    """The measurement probes check shape, sizes, pointers and alignment on the host."""
    lib = dsv4.library()
    keep, p = _fake()
    fl = ctypes.c_double(0.0)
    lib.dsv4_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.dsv4_peak_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    assert lib.dsv4_peak_mfma(2, 4, 10, p, ctypes.byref(fl), None) == 4  # UNSUPPORTED
    assert lib.dsv4_peak_mfma(0, 0, 10, p, ctypes.byref(fl), None) == 2  # SHAPE
    assert lib.dsv4_peak_mfma(1, 4, 0, p, ctypes.byref(fl), None) == 2
    assert lib.dsv4_peak_mfma(0, 4, 10, None, ctypes.byref(fl), None) == 1  # NULL
    assert lib.dsv4_peak_mfma(0, 4, 10, p, None, None) == 1
    assert lib.dsv4_peak_mfma(0, 4, 10, ctypes.c_void_p(p.value + 2), ctypes.byref(fl), None) == 3
    assert lib.dsv4_peak_stream(p, None, 17, p, 4, None) == 2
    assert lib.dsv4_peak_stream(p, None, 1024, p, 0, None) == 2
    assert lib.dsv4_peak_stream(None, None, 1024, p, 4, None) == 1
    assert lib.dsv4_peak_stream(p, None, 1024, None, 4, None) == 1
    assert lib.dsv4_peak_stream(ctypes.c_void_p(p.value + 8), None, 1024, p, 4, None) == 3
    assert lib.dsv4_peak_stream(p, ctypes.c_void_p(p.value + 4), 1024, p, 4, None) == 3
