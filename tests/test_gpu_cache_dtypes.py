"""GPU parity of the bf16 and per-tensor fp8 kv caches (one record of the 576 values per
slot) against the oracle, at page sizes 32 and 64 (the two the pages list for these
dtypes) and a fp8 scale that is a power of two and one that is not:

* insert: bf16 value dims bit for bit, fp8 value codes bit for bit (both sides decide a
  code on the same fp32 quotient); the rotated rope dims within the rotation bar of the
  packed cache's test (bf16), or one E4M3 step of it (fp8: a rope value one bf16 ulp
  apart may round to the neighbouring code); q within the rotation bar; skipped slots and
  positions leave the cache untouched;
* gather hook: bit for bit (bf16 copies; fp8 code x s rounded once to bf16);
* decode, prefill and split decode at H = 16 / 64 / 128 on ragged rows with -1 holes,
  out-of-range and duplicated slots and a row longer than one 4096-entry index block:
  the attention bar of the packed cache (1e-2 max, 1e-3 mean, lse 2e-3);
* the benchmark decode batch (64 tokens x 128 heads, rows of ~1700 slots) in both
  dtypes, every token against the oracle, lse within 1e-4;
* the one-launch step (and its split form) bit for bit equal to insert + fused
  decode (insert + combine + split decode), and against the oracle's insert -> combine
  -> attention chain."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import attention_workload, bf16_normal, rope_table
from tests.gpu_helpers import (assert_attention_close, bits_to_f64, dev, dev_bf16, host_bits,
                               log, oracle_cache, within_rotation_bound)
from tests.test_gpu_decode_step import _random_case, _run_step, _run_two, _same

pytestmark = pytest.mark.gpu
# (kv_dtype, kv_scale): bf16; fp8 with a power-of-two scale; fp8 with a general scale
DTYPES = [(1, 1.0), (2, 0.0625), (2, 0.0371)]
IDS = ["bf16", "fp8-s2^-4", "fp8-s0.0371"]


def _rb(kvd):
    return oracle.kv_record_bytes(kvd)


def _e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()


@pytest.mark.parametrize("P", [32, 64])
@pytest.mark.parametrize("kvd,kvs", DTYPES, ids=IDS)
def test_insert(dsv4, P, kvd, kvs):
    rng = np.random.default_rng(700 + 10 * kvd + P)
    num_pages, T, H = 9, 200, 4
    q = bf16_normal(rng, (T, H, 576))
    kv = bf16_normal(rng, (T, 576))
    kv[:10] = bf16_normal(rng, (10, 576), std=1e-3)       # fp8 subnormals
    kv[10:20] = bf16_normal(rng, (10, 576), std=60.0)     # beyond 448 * s: saturation
    pos = rng.integers(0, 700, T)
    slot_mapping = rng.permutation(num_pages * P)[:T].astype(np.int64)
    slot_mapping[5] = -1
    slot_mapping[6] = num_pages * P
    pos[7] = 700  # out of range: the token is left untouched
    weight = bf16_normal(rng, (576,), mean=1.0, std=0.1)
    cos_sin = rope_table(700)
    rb = _rb(kvd)
    cache0 = rng.integers(0, 256, size=num_pages * P * rb, dtype=np.uint8)
    log(f"insert kv_dtype={kvd} kv_scale={kvs} P={P} T={T} H={H}")
    q_ref, c_ref = oracle.kv_insert(q, kv, pos, slot_mapping, cos_sin, weight, 1e-6, cache0,
                                    num_pages, P, kv_dtype=kvd, kv_scale=kvs)
    qd, cache = dev_bf16(q), dev(cache0)
    dsv4.dsv4_kv_insert(qd, dev_bf16(kv), dev(pos, np.int64), dev(slot_mapping, np.int64),
                        dev(cos_sin, np.float32), dev_bf16(weight), 1e-6, cache, page_size=P,
                        kv_dtype=kvd, kv_scale=kvs)
    torch.cuda.synchronize()
    ok, exact, worst = within_rotation_bound(host_bits(qd), q_ref, 64)
    log(f"  q within bound={ok} exact frac={exact:.6f} worst/bound={worst:.3f}")
    assert ok
    g = cache.cpu().numpy().reshape(-1, rb)
    r = c_ref.reshape(-1, rb)
    if kvd == 1:
        assert np.array_equal(g[:, :1024], r[:, :1024])
        rg = np.ascontiguousarray(g[:, 1024:]).view(np.uint16)
        rr = np.ascontiguousarray(r[:, 1024:]).view(np.uint16)
        ok, exact, worst = within_rotation_bound(rg, rr, 64)
        log(f"  rope within bound={ok} exact frac={exact:.6f} worst/bound={worst:.3f}")
        assert ok
    else:
        assert np.array_equal(g[:, :512], r[:, :512])
        same = g[:, 512:] == r[:, 512:]
        vg, vr = _e4m3(g[:, 512:]), _e4m3(r[:, 512:])
        step = np.exp2(np.floor(np.log2(np.maximum(np.abs(vr), 2.0 ** -6))) - 3)  # e4m3 spacing
        with np.errstate(invalid="ignore"):
            near = np.abs(vg - vr) <= step
        log(f"  rope codes exact frac={np.mean(same):.6f}")
        assert np.all(same | near) and np.mean(same) > 0.99


@pytest.mark.parametrize("kvd,kvs", DTYPES, ids=IDS)
def test_gather(dsv4, kvd, kvs):
    rng = np.random.default_rng(800 + kvd)
    P, num_pages = 32, 6
    n_slots = num_pages * P
    if kvd == 1:
        cache = bf16_normal(rng, (n_slots, 576), std=3.0).view(np.uint8).reshape(-1)
    else:
        cache = rng.integers(0, 256, size=n_slots * 576, dtype=np.uint8)
        cache[(cache & 0x7F) == 0x7F] = 0x35  # no NaN codes
    query = np.concatenate([rng.permutation(n_slots)[:150], [-1, -7, n_slots, n_slots + 99]])
    ref = oracle.gather_dequant(cache, num_pages, P, query.astype(np.int32), kv_dtype=kvd,
                                kv_scale=kvs)
    out = torch.full((query.size, 576), 5.0, dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_gather_dequant(dev(cache), dev(query, np.int32), out, page_size=P, kv_dtype=kvd,
                             kv_scale=kvs)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref)


def _cache(rng, kvd, kvs, P, num_pages, n_rows):
    slots = rng.choice(num_pages * P, size=n_rows, replace=False).astype(np.int64)
    kv = bf16_normal(rng, (n_rows, 576))
    cache = np.zeros(num_pages * P * _rb(kvd), np.uint8)
    _, cache = oracle.kv_insert(np.zeros((n_rows, 0, 576), np.uint16), kv,
                                rng.integers(0, 1000, n_rows), slots, rope_table(1000),
                                np.zeros(576, np.uint16), 1e-6, cache, num_pages, P,
                                kv_dtype=kvd, kv_scale=kvs)
    return cache, slots


@pytest.mark.parametrize("H", [16, 64, 128])
@pytest.mark.parametrize("kvd,kvs", DTYPES, ids=IDS)
def test_attention(dsv4, H, kvd, kvs):
    rng = np.random.default_rng(900 + H + 10 * kvd)
    P = 32 if H == 64 else 64
    num_pages = 160
    cache, slots = _cache(rng, kvd, kvs, P, num_pages, 4500)
    lens_list = [0, 1, 63, 65, 200, 777, 4200]
    T, stride = len(lens_list), 4224
    idx = np.full((T, stride), 999999, np.int32)
    for t, L in enumerate(lens_list):
        row = rng.choice(slots, size=L, replace=True)
        row[rng.random(L) < 0.08] = -1
        oor = rng.random(L) < 0.02
        row[oor] = num_pages * P + rng.integers(0, 50, oor.sum())
        idx[t, :L] = row
    lens = np.array(lens_list, np.int32)
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    scale = 1.0 / 24
    ref, rlse = oracle.sparse_mla(q, cache, num_pages, P, idx, lens, sinks, scale, nthreads=8,
                                  kv_dtype=kvd, kv_scale=kvs)
    cache_dev = dev(cache)
    for mode in ("decode", "prefill", "split"):
        log(f"attention {mode} kv_dtype={kvd} kv_scale={kvs} H={H} P={P} T={T}")
        out = torch.full((T, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
        kw = dict(lse=lse, page_size=P, kv_dtype=kvd, kv_scale=kvs)
        args = (dev_bf16(q), cache_dev, dev(idx), dev(lens), dev(sinks), scale, out)
        if mode == "split":
            ws = torch.empty(dsv4.split_workspace_bytes(T, H, 3), dtype=torch.uint8, device="cuda")
            dsv4.dsv4_sparse_mla_decode_split(*args, 3, ws, **kw)
        else:
            fn = dsv4.dsv4_sparse_mla_decode if mode == "decode" else dsv4.dsv4_sparse_mla_prefill
            fn(*args, **kw)
        torch.cuda.synchronize()
        assert_attention_close(host_bits(out), ref, f"{mode} {kvd}")
        gl = lse.cpu().numpy()
        fin = np.isfinite(rlse)
        assert np.array_equal(fin, np.isfinite(gl))
        assert np.max(np.abs(gl[fin] - rlse[fin])) <= 2e-3


@pytest.mark.parametrize("kvd,kvs", DTYPES[:2], ids=IDS[:2])
def test_benchmark_decode_batch(dsv4, kvd, kvs):
    wl = attention_workload(2)
    it = wl["instances"][0]
    log(f"benchmark decode batch kv_dtype={kvd}: T={wl['T']} H={wl['H']} "
        f"ctx rows={wl['ctx_kv'].shape[0]}")
    cache = oracle_cache(wl, kv_dtype=kvd, kv_scale=kvs)
    idx, lens = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                               wl["block_table"], wl["T"], wl["top_k"], wl["window"], 64, wl["W"])
    T, H = wl["T"], wl["H"]
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode(dev_bf16(it["q"]), dev(cache), dev(idx), dev(lens),
                                dev(it["sinks"]), wl["softmax_scale"], out, lse, kv_dtype=kvd,
                                kv_scale=kvs)
    torch.cuda.synchronize()
    ref, rlse = oracle.sparse_mla(it["q"], cache, wl["num_pages"], 64, idx, lens, it["sinks"],
                                  wl["softmax_scale"], nthreads=16, kv_dtype=kvd, kv_scale=kvs)
    assert_attention_close(host_bits(out), ref, f"benchmark batch {kvd}")
    lerr = float(np.max(np.abs(lse.cpu().numpy() - rlse)))
    log(f"  lse max err {lerr:.2e}")
    assert lerr <= 1e-4


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("kvd,kvs", DTYPES, ids=IDS)
def test_step_equals_insert_then_decode(dsv4, seed, kvd, kvs):
    rng = np.random.default_rng(4000 + seed + 10 * kvd)
    P = [64, 32][seed % 2]
    H = [128, 16, 64, 32][seed % 4]
    c, q0, cache0, h = _random_case(rng, P, H, [1, 4][seed % 2], kv_dtype=kvd, kv_scale=kvs)
    log(f"step kv_dtype={kvd} seed={seed} P={P} H={H} T={c['T']} top_k={c['top_k']} "
        f"window={c['window']}")
    qa, ca, oa, la = _run_two(dsv4, c, q0, cache0)
    qb, cb, ob, lb = _run_step(dsv4, c, q0, cache0)
    torch.cuda.synchronize()
    assert _same(qa, qb) and torch.equal(ca, cb) and _same(oa, ob) and _same(la, lb)
    # the split step against insert + combine + split decode, bit for bit
    T, splits = c["T"], 3
    W = (c["top_k"] + c["window"] + 127) // 128 * 128
    ws = torch.empty(dsv4.split_workspace_bytes(T, H, splits), dtype=torch.uint8, device="cuda")
    kw = dict(page_size=P, kv_dtype=kvd, kv_scale=kvs)
    q3, c3 = q0.clone(), cache0.clone()
    dsv4.dsv4_kv_insert(q3, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6, c3, **kw)
    comb = torch.full((T, W), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros(T, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"], c["top_k"],
                              c["window"], comb, lens, page_size=P)
    o3 = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    l3 = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_split(q3, c3, comb, lens, c["sinks"], c["scale"], o3, splits, ws,
                                      lse=l3, **kw)
    q, cache = q0.clone(), cache0.clone()
    out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_step(q, c["kv"], c["pos"], c["slots"], c["cos_sin"], c["w"], 1e-6,
                                     cache, c["topk"], c["tl"], c["qsl"], c["sl"], c["bt"],
                                     c["top_k"], c["window"], c["sinks"], c["scale"], out, lse,
                                     splits=splits, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert _same(q, q3) and torch.equal(cache, c3) and torch.equal(cache, cb)
    assert _same(out, o3) and _same(lse, l3)


@pytest.mark.parametrize("kvd,kvs", DTYPES, ids=IDS)
def test_step_against_oracle(dsv4, kvd, kvs):
    """Several new tokens per request, a window over them, sinks: the one-launch step
    against the oracle's insert, combine and attention in sequence."""
    rng = np.random.default_rng(45 + kvd)
    while True:
        c, q0, cache0, h = _random_case(rng, 64, 32, 5, B=3, top_k=64, window=16, kv_dtype=kvd,
                                        kv_scale=kvs)
        if h["sinks"] is not None and h["tl"] is not None:
            break
    T, P = h["T"], h["P"]
    q_ref, cache_ref = oracle.kv_insert(h["q"], h["kv"], h["pos"], h["slots"], h["cos_sin"],
                                        h["w"], 1e-6, h["cache"], h["npg"], P, kv_dtype=kvd,
                                        kv_scale=kvs)
    W = (h["top_k"] + h["window"] + 127) // 128 * 128
    ref_idx, ref_lens = oracle.combine(h["topk"], h["tl"], h["qsl"], h["sl"], h["bt"], T,
                                       h["top_k"], h["window"], P, W)
    inreq = np.arange(T) < int(h["qsl"][-1]) - int(h["qsl"][0])
    ref_lens = np.where(inreq, ref_lens, 0).astype(np.int32)
    ref, rlse = oracle.sparse_mla(q_ref, cache_ref, h["npg"], P, ref_idx, ref_lens, h["sinks"],
                                  1 / 24, nthreads=8, kv_dtype=kvd, kv_scale=kvs)
    log(f"step vs oracle kv_dtype={kvd} T={T} H=32 qlens={np.diff(h['qsl']).tolist()}")
    q, cache, out, lse = _run_step(dsv4, c, q0, cache0)
    torch.cuda.synchronize()
    rb = _rb(kvd)
    g = cache.cpu().numpy().reshape(-1, rb)
    r = cache_ref.reshape(-1, rb)
    assert np.array_equal(g[:, :512 * (2 if kvd == 1 else 1)], r[:, :512 * (2 if kvd == 1 else 1)])
    gq, rq = bits_to_f64(host_bits(q)), bits_to_f64(q_ref)
    assert np.all(np.abs(gq - rq) <= 2.0 ** -7 * np.abs(rq) + 2.0 ** -16)
    assert_attention_close(host_bits(out), ref, f"step vs oracle {kvd}")
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= 2e-3
