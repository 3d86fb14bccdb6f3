"""Pins of the oracle's fused insert step.

q path: compared with torch.nn.functional.rms_norm (fp64) followed by a rotation of
each GPT-J pair written as a complex product (numpy complex128), then bf16 rounding;
closed form for a constant vector (y = sign(c) * w / sqrt(1 + eps / c^2)).
kv path: each nope block's scale byte satisfies the UE8M0 definition by brute force,
each code is torch's float8_e4m3fn rounding of k * 2^-e (exact product), the stored
rope values equal the complex-product rotation rounded to bf16, and slot -1 or an
out-of-range position leaves the cache untouched.
"""
import numpy as np
import torch
import torch.nn.functional as F

from synth_inputs import bf16_bits, bf16_normal, rope_table
from tests.oracle_refs import bits_to_f64, cache_fields

P = 64


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


def _run(orc, seed, T=6, H=4, num_pages=4, max_pos=5000):
    rng = np.random.default_rng(seed)
    q = bf16_normal(rng, (T, H, 576))
    kv = bf16_normal(rng, (T, 576), std=float(rng.choice([0.01, 1.0, 30.0])))
    pos = rng.integers(0, max_pos, size=T).astype(np.int64)
    pos[0] = 0
    slots = rng.choice(num_pages * P, size=T, replace=False).astype(np.int64)
    w = bf16_normal(rng, (576,), mean=1.0, std=0.1)
    cs = rope_table(max_pos)
    cache0 = rng.integers(0, 256, size=num_pages * P * 648, dtype=np.uint8)
    qo, cache = orc.kv_insert(q, kv, pos, slots, cs, w, 1e-6, cache0, num_pages, P)
    return dict(q=q, kv=kv, pos=pos, slots=slots, w=w, cs=cs, cache0=cache0, qo=qo, cache=cache,
                T=T, H=H, num_pages=num_pages)


def test_q_rmsnorm_rope_matches_library(orc):
    for seed in range(4):
        r = _run(orc, seed)
        x = torch.from_numpy(bits_to_f64(r["q"]))
        w = torch.from_numpy(bits_to_f64(r["w"]))
        y = F.rms_norm(x, (576,), w, 1e-6).numpy()
        for t in range(r["T"]):
            y[t] = _rotate(y[t], r["cs"][r["pos"][t]])
        got = bits_to_f64(r["qo"])
        assert np.all(np.abs(got - y) <= 0.5 * _ulp_bf16(y) * (1 + 1e-9) + 1e-300)


def test_q_constant_vector_closed_form(orc):
    for c in [0.5, -3.0, 1e-3, 100.0]:
        q = np.full((1, 2, 576), bf16_bits(np.array([c], np.float32))[0], np.uint16)
        w = bf16_normal(np.random.default_rng(1), (576,), mean=1.0, std=0.1)
        cache = np.zeros(P * 648, np.uint8)
        cb = bits_to_f64(q[0, 0, :1])[0]
        qo, _ = orc.kv_insert(q, np.zeros((1, 576), np.uint16), np.zeros(1, np.int64),
                              np.array([-1], np.int64), rope_table(2), w, 1e-6, cache, 1, P)
        ref = np.sign(cb) * bits_to_f64(w) / np.sqrt(1 + 1e-6 / cb ** 2)  # position 0: no rotation
        got = bits_to_f64(qo[0, 1])
        assert np.all(np.abs(got - ref) <= 0.5 * _ulp_bf16(ref) * (1 + 1e-9))


def test_kv_quantisation_and_rope(orc):
    e4m3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for seed in range(4):
        r = _run(orc, 10 + seed)
        nope, rope, scale = cache_fields(r["cache"], r["num_pages"], P)
        k = bits_to_f64(r["kv"])
        for t in range(r["T"]):
            s = int(r["slots"][t])
            pg, off = s // P, s % P
            for blk in range(8):
                kb = k[t, blk * 64:(blk + 1) * 64]
                amax = np.max(np.abs(kb))
                e = int(scale[pg, off, blk]) - 127
                if amax == 0:
                    assert e == -127
                else:
                    assert amax <= 448 * 2.0 ** e and amax > 448 * 2.0 ** (e - 1)
                scaled = np.ldexp(kb, -e)  # exact
                ref = torch.from_numpy(scaled.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                assert np.array_equal(nope[pg, off, blk * 64:(blk + 1) * 64], ref)
                dec = e4m3[nope[pg, off, blk * 64:(blk + 1) * 64]] * 2.0 ** e
                assert np.all(np.abs(dec - kb) <= 2.0 ** -4 * np.abs(kb) + 2.0 ** (e - 10))
            rot = _rotate(k[t:t + 1], r["cs"][r["pos"][t]])[0, 512:]
            got = bits_to_f64(np.ascontiguousarray(rope[pg, off]).view(np.uint16))
            assert np.all(np.abs(got - rot) <= 0.5 * _ulp_bf16(rot) * (1 + 1e-9) + 1e-300)


def test_skips_leave_memory_untouched(orc):
    rng = np.random.default_rng(3)
    T, H, num_pages = 4, 2, 2
    q = bf16_normal(rng, (T, H, 576))
    kv = bf16_normal(rng, (T, 576))
    pos = np.array([1, 7000, -1, 3], np.int64)           # tokens 1, 2: position out of range
    slots = np.array([5, 6, 7, -1], np.int64)             # token 3: no cache write
    cache0 = rng.integers(0, 256, size=num_pages * P * 648, dtype=np.uint8)
    qo, cache = orc.kv_insert(q, kv, pos, slots, rope_table(100), bf16_normal(rng, (576,)), 1e-6,
                              cache0, num_pages, P)
    assert np.array_equal(qo[1:3], q[1:3]) and not np.array_equal(qo[3], q[3])
    changed = np.nonzero(cache != cache0)[0]
    nope, rope, scale = cache_fields(cache, num_pages, P)
    n0, r0, s0 = cache_fields(cache0, num_pages, P)
    diff_slots = set()
    for arr, arr0 in ((nope, n0), (rope, r0), (scale, s0)):
        d = np.nonzero(np.any(arr.reshape(num_pages * P, -1) != arr0.reshape(num_pages * P, -1), axis=1))[0]
        diff_slots |= set(int(x) for x in d)
    assert diff_slots <= {5} and len(changed) > 0
