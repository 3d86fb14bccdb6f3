"""GPU parity of the integer and byte steps: index combining, gather/dequantise, and the
fused insert.  Bar: bit-exact against the oracle for indices, lengths, FP8 codes and
scale bytes; bf16 values computed in fp32 on the GPU (rotated rope dims, normalised q)
within one bf16 ulp of the oracle's fp64-then-rounded values."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import attention_workload, bf16_normal, insert_workload, rope_table
from tests.gpu_helpers import dev, dev_bf16, host_bits, log, within_rotation_bound

pytestmark = pytest.mark.gpu
P = 64


def _gpu_combine(dsv4, topk, tl, qsl, sl, bt, T, top_k, window, W, topk_width=None, fill=-7):
    comb = torch.full((T, W), fill, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), fill, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(dev(topk, np.int32), None if tl is None else dev(tl, np.int32),
                              dev(qsl, np.int32), dev(sl, np.int32), dev(bt, np.int32), top_k,
                              window, comb, lens, topk_width=topk_width)
    torch.cuda.synchronize()
    return comb.cpu().numpy(), lens.cpu().numpy()


@pytest.mark.parametrize("seed", range(6))
def test_combine_random_small(dsv4, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 6))
    top_k = int(rng.choice([8, 64, 300]))
    window = int(rng.choice([0, 1, 128]))
    width = top_k + int(rng.integers(0, 5))
    qlens = rng.integers(1, 6, size=B)
    seq_lens = np.array([int(rng.integers(ql, 900)) for ql in qlens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32) + int(rng.integers(0, 4))
    T = int(qsl[-1] - qsl[0]) + 2  # two rows no request owns
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    perm = rng.permutation(sum(pages) + 3)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    topk = rng.integers(-5, 1000, size=(T, width)).astype(np.int32)
    tl = rng.integers(-2, top_k + 3, size=T).astype(np.int32) if seed % 2 else None
    W = (top_k + window + 127) // 128 * 128 + 128 * int(seed % 3 == 0)
    log(f"combine seed={seed} B={B} T={T} top_k={top_k} window={window} W={W}")
    ref, rlen = oracle.combine(topk, tl, qsl, seq_lens, bt, T, top_k, window, P, W,
                               topk_width=width - 1)
    got, glen = _gpu_combine(dsv4, topk, tl, qsl, seq_lens, bt, T, top_k, window, W, topk_width=width - 1)
    assert np.array_equal(got, ref) and np.array_equal(glen, rlen)


@pytest.mark.parametrize("cfg", [0, 2, 3, 4])
def test_combine_workloads_full_size(dsv4, cfg):
    wl = attention_workload(cfg, context_kv="none" if cfg != 0 else "all", ctx_tokens=[])
    it = wl["instances"][0]
    log(f"combine cfg={cfg} T={wl['T']} W={wl['W']}")
    ref, rlen = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                               wl["block_table"], wl["T"], wl["top_k"], wl["window"], P, wl["W"])
    got, glen = _gpu_combine(dsv4, it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                             wl["block_table"], wl["T"], wl["top_k"], wl["window"], wl["W"])
    assert np.array_equal(glen, rlen)
    assert np.array_equal(got, ref)


def test_gather_dequant_bit_exact(dsv4):
    rng = np.random.default_rng(11)
    num_pages = 40
    cache = np.zeros(num_pages * P * 648, np.uint8)
    n_ins = 1500
    slots = rng.choice(num_pages * P, size=n_ins, replace=False).astype(np.int64)
    kv = bf16_normal(rng, (n_ins, 576))
    kv[:300] = bf16_normal(rng, (300, 576), std=1e-3)
    kv[300:600] = bf16_normal(rng, (300, 576), std=300.0)
    q0 = np.zeros((n_ins, 0, 576), np.uint16)
    _, cache = oracle.kv_insert(q0, kv, rng.integers(0, 100, n_ins), slots, rope_table(100),
                                np.zeros(576, np.uint16), 1e-6, cache, num_pages, P)
    # two pages of raw random bytes: every non-NaN code, scale bytes 90..160
    pages = cache.reshape(num_pages, -1)
    for pg in (3, 17):
        raw = rng.integers(0, 256, size=P * 512, dtype=np.uint8)
        raw[(raw & 0x7F) == 0x7F] = 0x05
        pages[pg, :P * 512] = raw
        pages[pg, P * 640:] = rng.integers(90, 161, size=P * 8, dtype=np.uint8)
    query = np.concatenate([rng.permutation(num_pages * P)[:2000], [-1, -100, num_pages * P, 2**30]])
    query = query.astype(np.int32)
    ref = oracle.gather_dequant(cache, num_pages, P, query)
    out = torch.empty(query.size, 576, dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_gather_dequant(dev(cache), dev(query), out)
    torch.cuda.synchronize()
    got = host_bits(out)
    assert np.array_equal(got, ref)


def _insert_gpu(dsv4, wl, cache0, q=None):
    q = wl["q"] if q is None else q
    qd = dev_bf16(q) if q.shape[1] else None
    cache = dev(cache0)
    dsv4.dsv4_kv_insert(qd, dev_bf16(wl["kv"]), dev(wl["positions"], np.int64),
                        dev(wl["slot_mapping"], np.int64), dev(wl["cos_sin"], np.float32),
                        dev_bf16(wl["q_norm_weight"]), wl["eps"], cache)
    torch.cuda.synchronize()
    return (host_bits(qd) if qd is not None else None), cache.cpu().numpy()


def _compare_insert(q_gpu, cache_gpu, q_ref, cache_ref, num_pages):
    pg_g = cache_gpu.reshape(num_pages, -1)
    pg_r = cache_ref.reshape(num_pages, -1)
    nope_eq = np.array_equal(pg_g[:, :P * 512], pg_r[:, :P * 512])
    scale_eq = np.array_equal(pg_g[:, P * 640:], pg_r[:, P * 640:])
    rope_g = np.ascontiguousarray(pg_g[:, P * 512:P * 640]).view(np.uint16).reshape(-1, 64)
    rope_r = np.ascontiguousarray(pg_r[:, P * 512:P * 640]).view(np.uint16).reshape(-1, 64)
    rok, rexact, rworst = within_rotation_bound(rope_g, rope_r, 64)
    log(f"  cache nope bit-exact={nope_eq} scales bit-exact={scale_eq} rope within bound={rok} "
        f"exact frac={rexact:.6f} worst/bound={rworst:.3f}")
    assert nope_eq and scale_eq and rok
    if q_gpu is not None:
        qok, qexact, qworst = within_rotation_bound(q_gpu, q_ref, 64)
        log(f"  q within bound={qok} exact frac={qexact:.6f} worst/bound={qworst:.3f}")
        assert qok


def test_insert_full_size(dsv4):
    wl = insert_workload()
    log(f"insert T={wl['T']} H={wl['H']} pages={wl['num_pages']}")
    cache0 = np.zeros(wl["num_pages"] * P * 648, np.uint8)
    q_ref, c_ref = oracle.kv_insert(wl["q"], wl["kv"], wl["positions"], wl["slot_mapping"],
                                    wl["cos_sin"], wl["q_norm_weight"], wl["eps"], cache0,
                                    wl["num_pages"], P)
    q_gpu, c_gpu = _insert_gpu(dsv4, wl, cache0)
    _compare_insert(q_gpu, c_gpu, q_ref, c_ref, wl["num_pages"])


def test_insert_edge_cases_and_codec_sweep(dsv4):
    """Skipped tokens, tiny/huge magnitudes, and blocks that sweep every finite bf16
    value below the block maximum for several scale exponents (exhaustive codec check)."""
    rng = np.random.default_rng(5)
    bits = np.arange(65536, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    vals = f[np.isfinite(f) & (np.abs(f) <= 1.0) & (np.abs(f) > 0)]
    rows = []
    for e in (-120, -20, -7, 0, 5, 100):  # block max 448 * 2^e, then values scaled by 2^e*448
        scaled = (vals.astype(np.float64) * 448.0 * 2.0 ** e).astype(np.float32)
        scaled = scaled[np.isfinite(scaled)]
        per = 63
        nb = int(np.ceil(scaled.size / per))
        blk = np.zeros((nb, 64), np.float32)
        flat = np.zeros(nb * per, np.float32)
        flat[:scaled.size] = scaled
        blk[:, 1:] = flat.reshape(nb, per)
        blk[:, 0] = np.float32(448.0 * 2.0 ** e)
        rows.append(blk.reshape(-1))
    allv = np.concatenate(rows)
    ntok = int(np.ceil(allv.size / 512))
    nope = np.zeros(ntok * 512, np.float32)
    nope[:allv.size] = allv
    import torch as _t
    nope_bits = _t.from_numpy(nope).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16)
    T = ntok + 6
    kv = bf16_normal(rng, (T, 576))
    kv[:ntok, :512] = nope_bits.reshape(ntok, 512)
    kv[ntok] = 0  # all-zero row
    kv[ntok + 1, :512] = bf16_normal(rng, (512,), std=1e-30)  # fp32-subnormal-scale amax
    num_pages = int(np.ceil(T / P)) + 2
    H = 3
    wl = dict(q=bf16_normal(rng, (T, H, 576)), kv=kv, positions=rng.integers(0, 500, T),
              slot_mapping=rng.permutation(num_pages * P)[:T].astype(np.int64),
              cos_sin=rope_table(500), q_norm_weight=bf16_normal(rng, (576,), mean=1.0, std=0.1),
              eps=1e-6)
    wl["positions"][ntok + 2] = 500      # out of range -> token untouched
    wl["positions"][ntok + 3] = -4       # out of range -> token untouched
    wl["slot_mapping"][ntok + 4] = -1    # no cache write, q still processed
    wl["slot_mapping"][ntok + 5] = num_pages * P  # out of range slot
    log(f"insert sweep T={T} pages={num_pages}")
    cache0 = rng.integers(0, 256, size=num_pages * P * 648, dtype=np.uint8)
    q_ref, c_ref = oracle.kv_insert(wl["q"], wl["kv"], wl["positions"], wl["slot_mapping"],
                                    wl["cos_sin"], wl["q_norm_weight"], wl["eps"], cache0,
                                    num_pages, P)
    q_gpu, c_gpu = _insert_gpu(dsv4, wl, cache0)
    _compare_insert(q_gpu, c_gpu, q_ref, c_ref, num_pages)
    assert np.array_equal(q_gpu[ntok + 2:ntok + 4], wl["q"][ntok + 2:ntok + 4])
    # cache-only insert (no q heads)
    wl0 = dict(wl, q=np.zeros((T, 0, 576), np.uint16))
    _, c_gpu0 = _insert_gpu(dsv4, wl0, cache0)
    assert np.array_equal(c_gpu0, c_gpu)


def test_insert_without_rope_rows_touches_nothing(dsv4):
    """max_pos = 0 (a rope table of no rows) leaves every position out of range: q and the
    cache keep their bytes and the table is never read (called through the C-ABI with a
    valid table pointer and max_pos 0)."""
    import ctypes
    rng = np.random.default_rng(6)
    T, H, num_pages = 9, 2, 2
    q0 = bf16_normal(rng, (T, H, 576))
    cache0 = rng.integers(0, 256, size=num_pages * P * 648, dtype=np.uint8)
    qd, cache = dev_bf16(q0), dev(cache0)
    kv = dev_bf16(bf16_normal(rng, (T, 576)))
    pos, slots = dev(np.zeros(T, np.int64)), dev(np.arange(T, dtype=np.int64))
    table = torch.zeros(4, 64, dtype=torch.float32, device="cuda")
    w = dev_bf16(bf16_normal(rng, (576,)))
    vp = ctypes.c_void_p
    st = dsv4.library().dsv4_kv_insert(vp(qd.data_ptr()), vp(kv.data_ptr()), vp(pos.data_ptr()),
                                       vp(slots.data_ptr()), vp(table.data_ptr()), 0,
                                       vp(w.data_ptr()), ctypes.c_float(1e-6),
                                       vp(cache.data_ptr()), num_pages, P, 0, ctypes.c_float(1.0),
                                       T, H, None)
    torch.cuda.synchronize()
    assert st == 0
    assert np.array_equal(host_bits(qd), q0) and np.array_equal(cache.cpu().numpy(), cache0)
