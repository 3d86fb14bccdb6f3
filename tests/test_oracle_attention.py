"""Pins of the oracle's attention and dequant-gather steps.

(i)  gather/dequant equals torch's E4M3 decode times 2^(byte-127), rounded to bf16;
     negative and out-of-range slots give zero rows.
(ii) dense equality: listing every valid slot of a tiny context equals fp64 dense
     softmax attention computed with torch.softmax / matmul (sinks as an extra logit).
(iii) permutation invariance of the index list; (iv) -1 entries and entries past the
     row length contribute nothing (bit-identical); (v) the sink closed form
     out_sink = out * S / (S + e^z) and z -> -inf equals no sink; (vi) one slot -> its
     value row exactly; identical keys -> mean of the values; a duplicated entry
     doubles its weight.
"""
import math

import numpy as np
import pytest

from synth_inputs import bf16_normal, rope_table
from tests.oracle_refs import bits_to_f64, dense_attention, torch_dequant

P = 64


def make_cache(orc, rng, num_pages, n_rows, slots=None, scale_kv=1.0):
    """Cache whose rows at `slots` hold N(0, scale) latents inserted by the oracle."""
    if slots is None:
        slots = rng.choice(num_pages * P, size=n_rows, replace=False)
    kv = bf16_normal(rng, (len(slots), 576), std=scale_kv)
    cache = np.zeros(num_pages * P * 648, np.uint8)
    q0 = np.zeros((len(slots), 0, 576), np.uint16)
    pos = rng.integers(0, 1000, size=len(slots))
    _, cache = orc.kv_insert(q0, kv, pos, np.asarray(slots, np.int64), rope_table(1000),
                             np.zeros(576, np.uint16), 1e-6, cache, num_pages, P)
    return cache, np.asarray(slots, np.int64)


def test_gather_dequant_matches_torch_decode(orc):
    rng = np.random.default_rng(0)
    num_pages = 3
    cache, slots = make_cache(orc, rng, num_pages, 100, scale_kv=3.0)
    # also raw random bytes (any non-NaN code, realistic scale bytes) in one page
    pages = cache.reshape(num_pages, -1)
    raw = rng.integers(0, 256, size=P * 512, dtype=np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x11
    pages[2, :P * 512] = raw
    pages[2, P * 640:] = rng.integers(100, 140, size=P * 8, dtype=np.uint8)
    query = np.concatenate([slots[:50], np.arange(2 * P, 3 * P), [-1, -5, num_pages * P, 10**6]])
    got = bits_to_f64(orc.gather_dequant(cache, num_pages, P, query))
    ref = torch_dequant(cache, num_pages, P, query)
    assert np.array_equal(got, ref)
    assert np.all(got[-4:] == 0)


def _setup(orc, seed, H=16, ctx=200, num_pages=6, sinks=True):
    rng = np.random.default_rng(seed)
    cache, slots = make_cache(orc, rng, num_pages, ctx)
    q = bf16_normal(rng, (1, H, 576))
    z = rng.standard_normal(H).astype(np.float32) if sinks else None
    return rng, cache, slots, q, z, num_pages


@pytest.mark.parametrize("sinks", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_dense_equality(orc, seed, sinks):
    rng, cache, slots, q, z, npg = _setup(orc, seed, sinks=sinks)
    scale = 1.0 / 24.0
    idx = slots[None, :].astype(np.int32)
    out, lse = orc.sparse_mla(q, cache, npg, P, idx, np.array([idx.shape[1]]), z, scale)
    K = torch_dequant(cache, npg, P, slots)
    ro, rl = dense_attention(q[0], K, scale, z)
    assert np.max(np.abs(out[0] - ro)) < 1e-12
    assert np.max(np.abs(lse[0] - rl)) < 1e-12
    # peaked logits as well (q x 8): one wrong or missing slot moves outputs a lot
    qp = bf16_normal(np.random.default_rng(seed + 50), (1, 16, 576), std=8.0)
    out, lse = orc.sparse_mla(qp, cache, npg, P, idx, np.array([idx.shape[1]]), z, scale)
    ro, rl = dense_attention(qp[0], K, scale, z)
    assert np.max(np.abs(out[0] - ro)) < 1e-12 and np.max(np.abs(lse[0] - rl)) < 1e-11


def test_permutation_and_padding(orc):
    rng, cache, slots, q, z, npg = _setup(orc, 3)
    n = slots.size
    idx = slots[None, :].astype(np.int32)
    base, blse = orc.sparse_mla(q, cache, npg, P, idx, np.array([n]), z, 0.04)
    perm = rng.permutation(n)
    o2, l2 = orc.sparse_mla(q, cache, npg, P, idx[:, perm], np.array([n]), z, 0.04)
    assert np.max(np.abs(o2 - base)) < 1e-13 and np.max(np.abs(l2 - blse)) < 1e-12
    # -1 holes, out-of-range slots, and garbage past the length: bit-identical result
    m = n + 30
    filler = rng.choice(m, size=30, replace=False)
    mask = np.zeros(m, bool)
    mask[filler] = True
    vals = np.empty(m, np.int64)
    vals[~mask] = slots
    vals[mask] = -1
    vals[filler[:5]] = npg * P + np.arange(5)
    row = np.full((1, m + 10), 12345, np.int32)
    row[0, :m] = vals
    o3, l3 = orc.sparse_mla(q, cache, npg, P, row, np.array([m]), z, 0.04)
    assert np.array_equal(o3, base) and np.array_equal(l3, blse)


def test_sink_closed_form(orc):
    rng, cache, slots, q, _, npg = _setup(orc, 4, sinks=False)
    idx = slots[None, :64].astype(np.int32)
    L = np.array([64])
    o0, l0 = orc.sparse_mla(q, cache, npg, P, idx, L, None, 0.05)
    z = rng.standard_normal(16).astype(np.float32)
    o1, l1 = orc.sparse_mla(q, cache, npg, P, idx, L, z, 0.05)
    S = np.exp(l0[0])  # sum of exp(s_j)
    factor = S / (S + np.exp(z.astype(np.float64)))
    assert np.max(np.abs(o1[0] - o0[0] * factor[:, None])) < 1e-13
    assert np.max(np.abs(l1[0] - np.log(S + np.exp(z.astype(np.float64))))) < 1e-12
    zneg = np.full(16, -np.inf, np.float32)
    o2, l2 = orc.sparse_mla(q, cache, npg, P, idx, L, zneg, 0.05)
    assert np.array_equal(o2, o0) and np.array_equal(l2, l0)


def test_special_cases(orc):
    rng, cache, slots, q, _, npg = _setup(orc, 5, sinks=False)
    K = torch_dequant(cache, npg, P, slots)
    # one slot -> its value row exactly
    o, l = orc.sparse_mla(q, cache, npg, P, slots[None, 7:8].astype(np.int32), np.array([1]), None, 0.1)
    assert np.array_equal(o[0], np.broadcast_to(K[7, :512], (16, 512)))
    # the same slot listed n times -> still its value row; lse grows by ln n
    o2, l2 = orc.sparse_mla(q, cache, npg, P, np.full((1, 5), slots[7], np.int32), np.array([5]), None, 0.1)
    assert np.max(np.abs(o2 - o)) < 1e-15 and np.max(np.abs(l2 - l - math.log(5))) < 1e-12
    # a duplicated entry doubles its weight
    a, b = slots[3], slots[9]
    od, _ = orc.sparse_mla(q, cache, npg, P, np.array([[a, a, b]], np.int32), np.array([3]), None, 0.1)
    qq = bits_to_f64(q[0])
    sa, sb = 0.1 * qq @ K[3], 0.1 * qq @ K[9]
    wa, wb = 2 * np.exp(sa), np.exp(sb)
    ref = (wa[:, None] * K[3, :512] + wb[:, None] * K[9, :512]) / (wa + wb)[:, None]
    assert np.max(np.abs(od[0] - ref)) < 1e-13
    # no valid slot and no sink -> zeros, lse -inf; with a sink -> zeros, lse = z
    oe, le = orc.sparse_mla(q, cache, npg, P, np.array([[-1, -1]], np.int32), np.array([2]), None, 0.1)
    assert np.all(oe == 0) and np.all(np.isneginf(le))
    z = np.full(16, 0.5, np.float32)
    oe, le = orc.sparse_mla(q, cache, npg, P, np.array([[-1]], np.int32), np.array([1]), z, 0.1)
    assert np.all(oe == 0) and np.allclose(le, 0.5)


def test_identical_keys_give_mean_of_values(orc):
    # rows with the same quantised nope/rope keys but different values are impossible
    # (V is part of K), so use identical records: all scores equal -> plain mean.
    rng = np.random.default_rng(8)
    num_pages = 2
    cache = np.zeros(num_pages * P * 648, np.uint8)
    kv = bf16_normal(rng, (1, 576))
    kv = np.repeat(kv, 10, axis=0)
    slots = np.arange(10, dtype=np.int64) * 3
    _, cache = orc.kv_insert(np.zeros((10, 0, 576), np.uint16), kv, np.zeros(10, np.int64), slots,
                             rope_table(4), np.zeros(576, np.uint16), 1e-6, cache, num_pages, P)
    q = bf16_normal(rng, (1, 16, 576))
    o, _ = orc.sparse_mla(q, cache, num_pages, P, slots[None].astype(np.int32), np.array([10]), None, 0.3)
    K = torch_dequant(cache, num_pages, P, slots)
    assert np.max(np.abs(o[0] - K[:, :512].mean(axis=0)[None])) < 1e-15


def test_threads_do_not_change_results(orc):
    rng = np.random.default_rng(9)
    cache, slots = make_cache(orc, rng, 8, 400)
    T, H = 5, 16
    q = bf16_normal(rng, (T, H, 576))
    idx = np.stack([rng.permutation(slots)[:300] for _ in range(T)]).astype(np.int32)
    lens = rng.integers(0, 301, size=T).astype(np.int32)
    a = orc.sparse_mla(q, cache, 8, P, idx, lens, None, 0.04, nthreads=1)
    b = orc.sparse_mla(q, cache, 8, P, idx, lens, None, 0.04, nthreads=3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
