"""GPU parity of the whole decode step in one launch (dsv4_sparse_mla_decode_step): its
q, cache bytes, output and lse are bit-identical to dsv4_kv_insert followed by
dsv4_sparse_mla_decode_topk on random multi-token requests (more new tokens per request
than a workgroup has waves, windows over the new rows, holes, tokens of no request,
skipped positions) at every head-group shape and page sizes 32, 64 and 256, with the new rows'
slots holding garbage beforehand; on the full benchmark workload and under HIP-graph
replay; and equal to the oracle's insert -> combine -> attention chain within the
attention bar on a small case."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import attention_workload, bf16_normal, rope_table
from tests.gpu_helpers import (assert_attention_close, bits_to_f64, dev, dev_bf16, host_bits,
                               log, oracle_cache)

pytestmark = pytest.mark.gpu


def _same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _kv(c):
    return dict(kv_dtype=c.get("kvd", 0), kv_scale=c.get("kvs", 1.0))


def _run_two(dsv4, c, q0, cache0):
    q, cache = q0.clone(), cache0.clone()
    T, H = q.shape[0], q.shape[1]
    dsv4.dsv4_kv_insert(q, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6, cache,
                        page_size=c["P"], **_kv(c))
    out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_topk(q, cache, c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"],
                                     c["top_k"], c["window"], c["sinks"], c["scale"], out, lse,
                                     page_size=c["P"], **_kv(c))
    return q, cache, out, lse


def _run_step(dsv4, c, q0, cache0, out=None, lse=None):
    q, cache = q0.clone(), cache0.clone()
    T, H = q.shape[0], q.shape[1]
    if out is None:
        out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_step(q, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6,
                                     cache, c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"],
                                     c["top_k"], c["window"], c["sinks"], c["scale"], out, lse,
                                     page_size=c["P"], **_kv(c))
    return q, cache, out, lse


def _random_case(rng, P, H, qmax, B=None, top_k=None, window=None, max_len=2500,
                 full_rows=False, kv_dtype=0, kv_scale=1.0):
    B = int(rng.integers(1, 5)) if B is None else B
    top_k = int(rng.choice([16, 300, 2048])) if top_k is None else top_k
    window = int(rng.choice([0, 1, 4, 128])) if window is None else window
    qlens = rng.integers(1, qmax + 1, size=B)
    lo_len = max_len - 200 if full_rows else 0
    seq_lens = np.array([int(rng.integers(max(ql, lo_len), max_len)) for ql in qlens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32) + int(rng.integers(0, 2))
    T = int(qsl[-1] - qsl[0]) + 2  # the last two tokens belong to no request
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    npg = sum(pages) + 1           # the last page: slots of the tokens of no request
    perm = rng.permutation(npg - 1)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    if pages[0] > 1:
        bt[0, 0] = -1  # a hole in the table (a new token under it gets no slot)
    # the new tokens' positions and slots, as the block tables give them
    pos = np.zeros(T, np.int64)
    slots = np.zeros(T, np.int64)
    for b in range(B):
        for i in range(int(qlens[b])):
            t = int(qsl[b] - qsl[0]) + i
            p = int(seq_lens[b]) - int(qlens[b]) + i
            pos[t] = p
            pg = int(bt[b, p // P])
            slots[t] = pg * P + p % P if pg >= 0 else -1
    pos[T - 2], slots[T - 2] = 7, (npg - 1) * P + 3
    pos[T - 1], slots[T - 1] = -1, (npg - 1) * P + 4  # skipped: q and cache untouched
    # garbage everywhere, then the context rows (positions before the new tokens)
    cache = rng.integers(0, 256, size=npg * P * oracle.kv_record_bytes(kv_dtype), dtype=np.uint8)
    ctx_b = np.concatenate([np.full(L - ql, b) for b, (L, ql) in enumerate(zip(seq_lens, qlens))])
    ctx_p = np.concatenate([np.arange(L - ql) for L, ql in zip(seq_lens, qlens)]).astype(np.int64)
    keep = bt[ctx_b, ctx_p // P] >= 0
    ctx_s = bt[ctx_b[keep], ctx_p[keep] // P].astype(np.int64) * P + ctx_p[keep] % P
    cos_sin = rope_table(max_len + 100)
    oracle.kv_insert(np.zeros((ctx_s.size, 0, 576), np.uint16),
                     bf16_normal(rng, (ctx_s.size, 576)), ctx_p[keep], ctx_s, cos_sin,
                     np.zeros(576, np.uint16), 1e-6, cache, npg, P, inplace=True,
                     kv_dtype=kv_dtype, kv_scale=kv_scale)
    if full_rows:  # distinct valid picks: every row as long as top_k allows
        topk = np.stack([rng.permutation(max_len - 200 - 1)[:top_k] for _ in range(T)]).astype(np.int32)
    else:
        topk = rng.integers(-3, max_len + 100, size=(T, top_k)).astype(np.int32)
    # fewer picks than the cap in some rows: the causal prefix of the top-k
    tl = (rng.integers(0, top_k + 2, size=T).astype(np.int32)
          if rng.integers(0, 2) and not full_rows else None)
    sinks = rng.standard_normal(H).astype(np.float32) if rng.integers(0, 2) else None
    h = dict(P=P, top_k=top_k, window=window, B=B, T=T, npg=npg, kv=bf16_normal(rng, (T, 576)),
             pos=pos, slots=slots, cos_sin=cos_sin, w=bf16_normal(rng, (576,), mean=1.0, std=0.1),
             topk=topk, tl=tl, qsl=qsl, sl=seq_lens, bt=bt, sinks=sinks,
             q=bf16_normal(rng, (T, H, 576)), cache=cache)
    h.update(kvd=kv_dtype, kvs=kv_scale)
    c = dict(P=P, top_k=top_k, window=window, scale=1 / 24, B=B, T=T, kv=dev_bf16(h["kv"]),
             kvd=kv_dtype, kvs=kv_scale,
             pos=dev(pos), slots=dev(slots), cos_sin=dev(cos_sin, np.float32), w=dev_bf16(h["w"]),
             topk=dev(topk), tl=None if tl is None else dev(tl), qsl=dev(qsl), sl=dev(seq_lens),
             bt=dev(bt), sinks=None if sinks is None else dev(sinks))
    return c, dev_bf16(h["q"]), dev(cache), h


@pytest.mark.parametrize("seed", range(10))
def test_decode_step_equals_insert_then_decode_topk(dsv4, seed):
    rng = np.random.default_rng(3000 + seed)
    P = [64, 32, 256][seed % 3]
    H = [128, 16, 64, 32][seed % 4]
    qmax = [1, 3, 7, 12][seed % 4]
    c, q0, cache0, _ = _random_case(rng, P, H, qmax)
    log(f"decode_step seed={seed} P={P} H={H} B={c['B']} T={c['T']} top_k={c['top_k']} "
        f"window={c['window']} qmax={qmax}")
    qa, ca, oa, la = _run_two(dsv4, c, q0, cache0)
    qb, cb, ob, lb = _run_step(dsv4, c, q0, cache0)
    torch.cuda.synchronize()
    assert _same(qa, qb), "q"
    assert torch.equal(ca, cb), "cache"
    assert _same(oa, ob) and _same(la, lb), "out / lse"
    assert _same(qb[-1], q0[-1])  # skipped position: q untouched


def _bench_case(dsv4, seed=11):
    wl = attention_workload(2, seed=seed, instances=1)
    it = wl["instances"][0]
    cache = dsv4.new_cache(wl["num_pages"])
    cos_sin = dev(wl["cos_sin"], np.float32)
    dsv4.dsv4_kv_insert(None, dev_bf16(wl["ctx_kv"]), dev(wl["ctx_pos"], np.int64),
                        dev(wl["ctx_slot"], np.int64), cos_sin, None, wl["eps"], cache)
    T = wl["T"]
    # one new token per request at position seq_len - 1 (the decode step)
    pos = wl["seq_lens"].astype(np.int64) - 1
    slots = wl["block_table"][np.arange(T), pos // 64].astype(np.int64) * 64 + pos % 64
    rng = np.random.default_rng(seed)
    c = dict(P=64, top_k=wl["top_k"], window=wl["window"], scale=wl["softmax_scale"],
             kv=dev_bf16(bf16_normal(rng, (T, 576))), pos=dev(pos), slots=dev(slots),
             cos_sin=cos_sin, w=dev_bf16(wl["q_norm_weight"]), topk=dev(it["topk"]),
             tl=dev(it["topk_lens"]), qsl=dev(wl["qsl"]), sl=dev(wl["seq_lens"]),
             bt=dev(wl["block_table"]), sinks=dev(it["sinks"]))
    return c, dev_bf16(it["q"]), cache


def test_decode_step_benchmark_workload_and_graph(dsv4):
    c, q0, cache0 = _bench_case(dsv4)
    log(f"decode_step benchmark workload T={q0.shape[0]} H={q0.shape[1]}")
    qa, ca, oa, la = _run_two(dsv4, c, q0, cache0)
    qb, cb, ob, lb = _run_step(dsv4, c, q0, cache0)
    torch.cuda.synchronize()
    assert _same(qa, qb) and torch.equal(ca, cb) and _same(oa, ob) and _same(la, lb)
    # graph replays: q is restored eagerly before each (the step normalises it in place);
    # re-inserting the same rows rewrites the same cache bytes
    q, cache = q0.clone(), cache0.clone()
    out = torch.empty_like(ob)
    lse = torch.empty_like(lb)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        dsv4.dsv4_sparse_mla_decode_step(q, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"],
                                         1e-6, cache, c["topk"], c["tl"], c["qsl"], c["sl"],
                                         c["bt"], c["top_k"], c["window"], c["sinks"], c["scale"],
                                         out, lse)
    for r in range(3):
        q.copy_(q0)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(q, qb) and torch.equal(cache, cb), r
        assert _same(out, ob) and _same(lse, lb), r


def test_decode_step_against_oracle(dsv4):
    """Several new tokens per request, a window over them, sinks: the step on the GPU
    against the oracle's insert, combine and attention in sequence."""
    rng = np.random.default_rng(44)
    while True:
        c, q0, cache0, h = _random_case(rng, 64, 32, 5, B=3, top_k=64, window=16)
        if h["sinks"] is not None and h["tl"] is not None:
            break
    T, P = h["T"], h["P"]
    q_ref, cache_ref = oracle.kv_insert(h["q"], h["kv"], h["pos"], h["slots"], h["cos_sin"],
                                        h["w"], 1e-6, h["cache"], h["npg"], P)
    W = (h["top_k"] + h["window"] + 127) // 128 * 128
    ref_idx, ref_lens = oracle.combine(h["topk"], h["tl"], h["qsl"], h["sl"], h["bt"], T,
                                       h["top_k"], h["window"], P, W)
    # tokens of no request attend to nothing (the combine leaves their rows untouched)
    base = int(h["qsl"][0])
    inreq = np.arange(T) < int(h["qsl"][-1]) - base
    ref_lens = np.where(inreq, ref_lens, 0).astype(np.int32)
    ref, rlse = oracle.sparse_mla(q_ref, cache_ref, h["npg"], P, ref_idx, ref_lens, h["sinks"],
                                  1 / 24, nthreads=8)
    log(f"decode_step vs oracle T={T} H=32 qlens={np.diff(h['qsl']).tolist()}")
    q, cache, out, lse = _run_step(dsv4, c, q0, cache0)
    torch.cuda.synchronize()
    # the new rows' nope codes and scales are exact; q within a bf16 rounding (plus the
    # rotation's fp32 rounding), which the attention bar absorbs
    pg_g = cache.cpu().numpy().reshape(h["npg"], -1)
    pg_r = cache_ref.reshape(h["npg"], -1)
    assert np.array_equal(pg_g[:, :P * 512], pg_r[:, :P * 512])
    assert np.array_equal(pg_g[:, P * 640:], pg_r[:, P * 640:])
    # one bf16 ulp of the oracle value (<= 2^-7 |r|) plus the fp32 rotation's rounding
    g, r = bits_to_f64(host_bits(q)), bits_to_f64(q_ref)
    ratio = np.abs(g - r) / (2.0 ** -7 * np.abs(r) + 2.0 ** -16)
    log(f"  q: exact fraction {np.mean(g == r):.6f}, worst |diff| / bound {ratio.max():.3f}")
    assert np.all(ratio <= 1.0)
    assert_attention_close(host_bits(out), ref, "decode_step vs oracle")
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= 2e-3


def test_decode_step_longest_row(dsv4):
    """The longest combined row the one-launch forms take (top_k + window = 4096 entries,
    the whole LDS index block): both fused entry points against insert + combine +
    decode."""
    rng = np.random.default_rng(3100)
    P, H = 64, 128
    c, q0, cache0, h = _random_case(rng, P, H, 2, B=3, top_k=3968, window=128, max_len=4600,
                                    full_rows=True)
    log(f"decode_step longest row: T={c['T']} top_k=3968 window=128")
    qa, ca, oa, la = _run_two(dsv4, c, q0, cache0)
    qb, cb, ob, lb = _run_step(dsv4, c, q0, cache0)
    # the three-launch reference: insert, combine into rows of 4096, decode
    q3, c3 = q0.clone(), cache0.clone()
    T = c["T"]
    dsv4.dsv4_kv_insert(q3, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6, c3,
                        page_size=P)
    comb = torch.full((T, 4096), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(T, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"], c["top_k"],
                              c["window"], comb, lens, page_size=P)
    o3 = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    l3 = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode(q3, c3, comb, lens, c["sinks"], c["scale"], o3, l3, page_size=P)
    torch.cuda.synchronize()
    assert int(lens.max()) == 4096  # rows of the full length occur
    assert _same(qa, qb) and torch.equal(ca, cb) and _same(oa, ob) and _same(la, lb)
    # rows of tokens of no request are empty in the fused forms; compare the request rows
    nreq = int(h["qsl"][-1] - h["qsl"][0])
    assert _same(ob[:nreq], o3[:nreq]) and _same(lb[:nreq], l3[:nreq])


@pytest.mark.parametrize("seed", range(6))
def test_decode_step_split_equals_insert_combine_split(dsv4, seed):
    """The split form of the one-launch step against insert, combine (rows of width
    round_up(top_k + window, 128)) and the split decode with the same number of pieces:
    out and lse bit for bit; q and the cache bytes as the unsplit step leaves them."""
    rng = np.random.default_rng(3200 + seed)
    P = [64, 32, 256][seed % 3]
    H = [128, 16, 64][seed % 3]
    splits = [2, 3, 8][seed % 3]
    c, q0, cache0, h = _random_case(rng, P, H, [1, 5][seed % 2])
    T = c["T"]
    W = (c["top_k"] + c["window"] + 127) // 128 * 128
    log(f"decode_step split seed={seed} P={P} H={H} T={T} top_k={c['top_k']} "
        f"window={c['window']} splits={splits}")
    ws = torch.empty(dsv4.split_workspace_bytes(T, H, splits), dtype=torch.uint8, device="cuda")
    # reference chain
    q3, c3 = q0.clone(), cache0.clone()
    dsv4.dsv4_kv_insert(q3, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6, c3,
                        page_size=P)
    comb = torch.full((T, W), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(T, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"], c["top_k"],
                              c["window"], comb, lens, page_size=P)
    o3 = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    l3 = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_split(q3, c3, comb, lens, c["sinks"], c["scale"], o3, splits, ws,
                                      lse=l3, page_size=P)
    torch.cuda.synchronize()
    o3, l3 = o3.clone(), l3.clone()
    # the split step
    q, cache = q0.clone(), cache0.clone()
    out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_step(q, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6,
                                     cache, c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"],
                                     c["top_k"], c["window"], c["sinks"], c["scale"], out, lse,
                                     page_size=P, splits=splits, workspace=ws)
    torch.cuda.synchronize()
    assert _same(q, q3) and torch.equal(cache, c3)
    assert _same(out, o3) and _same(lse, l3)


@pytest.mark.parametrize("splits", [3, 5])
def test_decode_step_split_many_rounds(dsv4, splits):
    """The split step on the benchmark batch (64 tokens x 4 head groups x `splits` pieces =
    768 / 1280 workgroups, several dispatch rounds, so the pieces of one row start at
    different times): q, cache bytes, out and lse bit for bit equal to insert, combine
    and the split decode.  Every piece reads the raw q rows; a piece that read rows a
    sibling had already normalised would normalise them twice and differ here."""
    c, q0, cache0 = _bench_case(dsv4, seed=12)
    T, H, P = q0.shape[0], q0.shape[1], 64
    W = (c["top_k"] + c["window"] + 127) // 128 * 128
    log(f"decode_step split many rounds: T={T} H={H} splits={splits} "
        f"workgroups={T * (H // 32) * splits}")
    ws = torch.empty(dsv4.split_workspace_bytes(T, H, splits), dtype=torch.uint8, device="cuda")
    q3, c3 = q0.clone(), cache0.clone()
    dsv4.dsv4_kv_insert(q3, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6, c3,
                        page_size=P)
    comb = torch.full((T, W), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(T, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"], c["top_k"],
                              c["window"], comb, lens, page_size=P)
    o3 = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    l3 = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_split(q3, c3, comb, lens, c["sinks"], c["scale"], o3, splits, ws,
                                      lse=l3, page_size=P)
    torch.cuda.synchronize()
    o3, l3 = o3.clone(), l3.clone()
    for rep in range(2):
        q, cache = q0.clone(), cache0.clone()
        out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
        dsv4.dsv4_sparse_mla_decode_step(q, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"],
                                         1e-6, cache, c["topk"], c["tl"], c["qsl"], c["sl"],
                                         c["bt"], c["top_k"], c["window"], c["sinks"], c["scale"],
                                         out, lse, page_size=P, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert _same(q, q3), ("q", rep)
        assert torch.equal(cache, c3), ("cache", rep)
        assert _same(out, o3) and _same(lse, l3), ("out / lse", rep)
