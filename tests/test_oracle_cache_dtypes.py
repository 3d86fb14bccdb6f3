"""Pins of the oracle's bf16 and per-tensor fp8 kv-cache dtypes (records of the 576
latent values back to back, slot s at byte s * record_bytes).

(i)   bf16 insert: the nope half of a record is the input row's bits, the rope half the
      complex-product rotation rounded to bf16 (within half an ulp of the exact value);
      q is the same as with the packed cache; skipped slots and positions leave the
      cache untouched.
(ii)  fp8 insert: every code is torch's float8_e4m3fn rounding of the fp32 quotient
      z / s clamped to +-448, z being the bf16 row (rope rotated); covers saturation,
      subnormals and signed zeros.
(iii) gather: bf16 records come back bit for bit; fp8 records as torch's e4m3 decode
      times s, rounded once to bf16 (s chosen so that the product is exact in fp32);
      invalid slots give zero rows.
(iv)  attention equals fp64 dense softmax attention (torch) over rows decoded by torch,
      and an fp8 cache of scale s gives s * out and the same lse as scale 1 with the
      softmax scale multiplied by s.
(v)   the three readers agree bit for bit on values all three formats hold exactly.
"""
import numpy as np
import pytest
import torch

from synth_inputs import bf16_bits, bf16_normal, rope_table
from tests.oracle_refs import bits_to_f64, dense_attention

LATENT, NOPE = 576, 512


def _rotate(y, cs_row):
    c = cs_row[:32].astype(np.float64)
    s = cs_row[32:].astype(np.float64)
    z = (y[..., 512::2] + 1j * y[..., 513::2]) * (c + 1j * s)
    out = y.copy()
    out[..., 512::2] = z.real
    out[..., 513::2] = z.imag
    return out


def _ulp_bf16(x):
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _records(cache, kv_dtype, orc):
    rb = orc.kv_record_bytes(kv_dtype)
    return cache.reshape(-1, rb)


def _insert_case(orc, seed, P, kv_dtype, kv_scale=1.0, T=12, H=3, num_pages=3, max_pos=3000):
    rng = np.random.default_rng(seed)
    q = bf16_normal(rng, (T, H, 576))
    kv = bf16_normal(rng, (T, 576), std=1.0)
    kv[1] *= 0  # zeros, signed below
    kv[1, ::2] = bf16_bits(np.full(288, -0.0, np.float32))
    kv[2] = bf16_normal(rng, (576,), std=1e-4)    # fp8 subnormals at s ~ 1e-2
    kv[3] = bf16_normal(rng, (576,), std=300.0 * max(1.0, kv_scale))  # beyond 448 * s
    pos = rng.integers(0, max_pos, size=T).astype(np.int64)
    slots = rng.choice(num_pages * P, size=T, replace=False).astype(np.int64)
    slots[4] = -1
    slots[5] = num_pages * P
    pos[6] = max_pos  # position out of range: token untouched
    w = bf16_normal(rng, (576,), mean=1.0, std=0.1)
    cs = rope_table(max_pos)
    rb = orc.kv_record_bytes(kv_dtype)
    cache0 = rng.integers(0, 256, size=num_pages * P * rb, dtype=np.uint8)
    qo, cache = orc.kv_insert(q, kv, pos, slots, cs, w, 1e-6, cache0, num_pages, P,
                              kv_dtype=kv_dtype, kv_scale=kv_scale)
    return dict(q=q, kv=kv, pos=pos, slots=slots, w=w, cs=cs, cache0=cache0, qo=qo, cache=cache,
                num_pages=num_pages, max_pos=max_pos)


def _written(r, num_slots):
    return [(t, int(s)) for t, s in enumerate(r["slots"])
            if 0 <= s < num_slots and 0 <= r["pos"][t] < r["max_pos"]]


@pytest.mark.parametrize("P", [32, 64])
def test_bf16_insert_record(orc, P):
    for seed in range(3):
        r = _insert_case(orc, 10 + seed, P, orc.KV_BF16)
        rec = _records(r["cache"], orc.KV_BF16, orc)
        rec0 = _records(r["cache0"], orc.KV_BF16, orc)
        done = _written(r, r["num_pages"] * P)
        for t, s in done:
            vals = rec[s].view(np.uint16)
            assert np.array_equal(vals[:NOPE], r["kv"][t, :NOPE])
            y = _rotate(bits_to_f64(r["kv"][t]), r["cs"][r["pos"][t]])[NOPE:]
            got = bits_to_f64(vals[NOPE:])
            assert np.all(np.abs(got - y) <= 0.5 * _ulp_bf16(y) * (1 + 1e-9) + 1e-300)
        untouched = np.setdiff1d(np.arange(rec.shape[0]), [s for _, s in done])
        assert np.array_equal(rec[untouched], rec0[untouched])
        # q does not depend on the cache dtype
        q_ds, _ = orc.kv_insert(r["q"], r["kv"], r["pos"], r["slots"], r["cs"], r["w"], 1e-6,
                                np.zeros(r["num_pages"] * P * 648, np.uint8), r["num_pages"], P)
        assert np.array_equal(r["qo"], q_ds)


@pytest.mark.parametrize("P,kv_scale", [(32, 0.0137), (64, 2.5), (64, 1.0)])
def test_fp8_insert_record(orc, P, kv_scale):
    s32 = float(np.float32(kv_scale))
    for seed in range(3):
        r = _insert_case(orc, 20 + seed, P, orc.KV_FP8_E4M3, kv_scale=s32)
        # z: the bf16 row with its rope dims rotated, from the bf16-dtype insert (pinned above)
        rb = _insert_case(orc, 20 + seed, P, orc.KV_BF16, kv_scale=s32)  # same inputs
        rec = _records(r["cache"], orc.KV_FP8_E4M3, orc)
        rec0 = _records(r["cache0"], orc.KV_FP8_E4M3, orc)
        zrec = _records(rb["cache"], orc.KV_BF16, orc)
        done = _written(r, r["num_pages"] * P)
        sat = 0
        for t, s in done:
            z = bits_to_f64(zrec[s].view(np.uint16))
            quo = (z / s32).astype(np.float32)
            sat += int(np.sum(np.abs(quo) > 448))
            ref = torch.from_numpy(np.clip(quo, -448, 448)).to(torch.float8_e4m3fn)
            assert np.array_equal(rec[s], ref.view(torch.uint8).numpy()), (seed, t)
        assert sat > 0  # the row of std 300 saturates at every scale used here
        untouched = np.setdiff1d(np.arange(rec.shape[0]), [s for _, s in done])
        assert np.array_equal(rec[untouched], rec0[untouched])
        assert np.array_equal(r["qo"], rb["qo"])


def test_gather_bf16_and_fp8(orc):
    rng = np.random.default_rng(5)
    P, num_pages = 32, 4
    n_slots = num_pages * P
    # bf16: random finite bits
    cache = bf16_normal(rng, (n_slots, LATENT), std=4.0).view(np.uint8).reshape(-1)
    query = np.concatenate([rng.permutation(n_slots)[:40], [-1, -9, n_slots, 10**6]])
    got = orc.gather_dequant(cache, num_pages, P, query, kv_dtype=orc.KV_BF16)
    recs = cache.view(np.uint16).reshape(n_slots, LATENT)
    assert np.array_equal(got[:40], recs[query[:40]])
    assert np.all(got[40:] == 0)
    # fp8: any non-NaN code; s with 16 significant bits (code * s exact in fp32)
    codes = rng.integers(0, 256, size=n_slots * LATENT, dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    s = float(np.ldexp(np.round(np.ldexp(0.0371, 20)), -20))
    got = bits_to_f64(orc.gather_dequant(codes, num_pages, P, query, kv_dtype=orc.KV_FP8_E4M3,
                                         kv_scale=s))
    dec = torch.from_numpy(codes.reshape(n_slots, LATENT)[query[:40]].copy()).view(
        torch.float8_e4m3fn).to(torch.float64) * s
    ref = dec.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got[:40], ref)
    assert np.all(got[40:] == 0)


def _decode_rows(orc, cache, kv_dtype, kv_scale, slots):
    n = orc.kv_record_bytes(kv_dtype)
    recs = cache.reshape(-1, n)[slots]
    if kv_dtype == orc.KV_BF16:
        return bits_to_f64(recs.view(np.uint16))
    return torch.from_numpy(recs.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * kv_scale


@pytest.mark.parametrize("kv_dtype,kv_scale", [(1, 1.0), (2, 0.021), (2, 3.0)])
def test_attention_dense(orc, kv_dtype, kv_scale):
    rng = np.random.default_rng(40 + kv_dtype)
    P, num_pages, ctx, H = 64, 5, 150, 8
    slots = rng.choice(num_pages * P, size=ctx, replace=False).astype(np.int64)
    kv = bf16_normal(rng, (ctx, LATENT), std=1.0 if kv_dtype == 1 else 0.3)
    rb = orc.kv_record_bytes(kv_dtype)
    cache = np.zeros(num_pages * P * rb, np.uint8)
    _, cache = orc.kv_insert(np.zeros((ctx, 0, LATENT), np.uint16), kv,
                             rng.integers(0, 900, ctx), slots, rope_table(900),
                             np.zeros(LATENT, np.uint16), 1e-6, cache, num_pages, P,
                             kv_dtype=kv_dtype, kv_scale=kv_scale)
    q = bf16_normal(rng, (2, H, LATENT))
    z = rng.standard_normal(H).astype(np.float32)
    idx = np.full((2, ctx + 6), -1, np.int32)
    idx[0, :ctx] = slots
    idx[1, :ctx] = rng.permutation(slots)
    idx[1, ctx] = num_pages * P  # out of range: skipped
    lens = np.array([ctx, ctx + 3], np.int32)
    scale = 1.0 / np.sqrt(LATENT)
    out, lse = orc.sparse_mla(q, cache, num_pages, P, idx, lens, z, scale, kv_dtype=kv_dtype,
                              kv_scale=kv_scale)
    K = _decode_rows(orc, cache, kv_dtype, kv_scale, slots)
    for t in range(2):
        ro, rl = dense_attention(q[t], K, scale, z)
        assert np.max(np.abs(out[t] - ro)) < 1e-12
        assert np.max(np.abs(lse[t] - rl)) < 1e-12
    if kv_dtype == 2:
        out1, lse1 = orc.sparse_mla(q, cache, num_pages, P, idx, lens, z, scale * kv_scale,
                                    kv_dtype=kv_dtype, kv_scale=1.0)
        assert np.max(np.abs(out - kv_scale * out1)) < 1e-12 * max(1.0, kv_scale)
        assert np.max(np.abs(lse - lse1)) < 1e-12


def test_readers_agree_on_exact_values(orc):
    """Rows of E4M3 values times 2^k are held exactly by all three formats (packed: codes +
    scale byte k + 127 per block, rope as bf16; bf16; fp8 with s = 2^k and rope codes), so
    gather and attention agree bit for bit."""
    rng = np.random.default_rng(77)
    P, num_pages, n, H = 32, 3, 70, 4
    k = -3
    codes = rng.integers(0, 256, size=(n, LATENT), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x2C
    vals = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * 2.0 ** k
    slots = rng.choice(num_pages * P, size=n, replace=False)
    ds = np.zeros(num_pages * P * 648, np.uint8).reshape(num_pages, -1)
    bf = np.zeros((num_pages * P, LATENT), np.uint16)
    f8 = np.zeros((num_pages * P, LATENT), np.uint8)
    for i, s in enumerate(slots):
        pg, off = divmod(int(s), P)
        ds[pg, off * 512:(off + 1) * 512] = codes[i, :NOPE]
        rope16 = bf16_bits(vals[i, NOPE:].astype(np.float32))
        ds[pg, P * 512 + off * 128:P * 512 + (off + 1) * 128] = rope16.view(np.uint8)
        ds[pg, P * 640 + off * 8:P * 640 + (off + 1) * 8] = 127 + k
        bf[s] = bf16_bits(vals[i].astype(np.float32))
        f8[s] = codes[i]
    caches = [(orc.KV_FP8_DS, ds.reshape(-1), 1.0), (orc.KV_BF16, bf.view(np.uint8).reshape(-1), 1.0),
              (orc.KV_FP8_E4M3, f8.reshape(-1), 2.0 ** k)]
    query = np.concatenate([slots, [-1]]).astype(np.int32)
    g = [orc.gather_dequant(c, num_pages, P, query, kv_dtype=d, kv_scale=sc) for d, c, sc in caches]
    assert np.array_equal(g[0], g[1]) and np.array_equal(g[0], g[2])
    assert np.array_equal(bits_to_f64(g[0][:n]), vals)
    q = bf16_normal(rng, (3, H, LATENT))
    idx = np.stack([rng.permutation(slots) for _ in range(3)]).astype(np.int32)
    lens = np.array([n, n // 2, 0], np.int32)
    res = [orc.sparse_mla(q, c, num_pages, P, idx, lens, None, 0.05, kv_dtype=d, kv_scale=sc)
           for d, c, sc in caches]
    for o, l in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(l, res[0][1])
