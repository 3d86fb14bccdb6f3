"""GPU parity at the other page sizes the pages list (32 and 256 slots per page, beside
the 64 of every other test): the insert's cache bytes, index combining through a block
table of P-slot pages, the gather/dequantise hook, the decode (whole and split rows) and
the whole step end to end, each against the oracle run with the same page size."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import bf16_normal, rope_table
from tests.gpu_helpers import (assert_attention_close, dev, dev_bf16, host_bits, log,
                               within_rotation_bound)

pytestmark = pytest.mark.gpu
PAGE_SIZES = [32, 256]


def _oracle_cache(rng, P, num_pages, n_slots):
    cache = np.zeros(num_pages * P * 648, np.uint8)
    slots = rng.choice(num_pages * P, size=n_slots, replace=False).astype(np.int64)
    kv = bf16_normal(rng, (n_slots, 576))
    _, cache = oracle.kv_insert(np.zeros((n_slots, 0, 576), np.uint16), kv,
                                rng.integers(0, 1000, n_slots), slots, rope_table(1000),
                                np.zeros(576, np.uint16), 1e-6, cache, num_pages, P)
    return cache, slots


@pytest.mark.parametrize("P", PAGE_SIZES)
def test_insert_page_size(dsv4, P):
    rng = np.random.default_rng(300 + P)
    num_pages = 9
    T, H = 200, 4
    q = bf16_normal(rng, (T, H, 576))
    kv = bf16_normal(rng, (T, 576))
    kv[:20] = bf16_normal(rng, (20, 576), std=1e-3)
    pos = rng.integers(0, 700, T)
    slot_mapping = rng.permutation(num_pages * P)[:T].astype(np.int64)
    slot_mapping[5] = -1
    slot_mapping[6] = num_pages * P
    weight = bf16_normal(rng, (576,), mean=1.0, std=0.1)
    cos_sin = rope_table(700)
    cache0 = rng.integers(0, 256, size=num_pages * P * 648, dtype=np.uint8)
    log(f"insert P={P} T={T} H={H} pages={num_pages}")
    q_ref, c_ref = oracle.kv_insert(q, kv, pos, slot_mapping, cos_sin, weight, 1e-6, cache0,
                                    num_pages, P)
    qd, cache = dev_bf16(q), dev(cache0)
    dsv4.dsv4_kv_insert(qd, dev_bf16(kv), dev(pos, np.int64), dev(slot_mapping, np.int64),
                        dev(cos_sin, np.float32), dev_bf16(weight), 1e-6, cache, page_size=P)
    torch.cuda.synchronize()
    c_gpu = cache.cpu().numpy().reshape(num_pages, -1)
    c_ref = c_ref.reshape(num_pages, -1)
    # codes and scale bytes: bit-exact; rope and q: one bf16 ulp of the oracle value plus
    # 2^-20 of the rotated pair's norm (the same bar as the 64-slot insert test)
    assert np.array_equal(c_gpu[:, :P * 512], c_ref[:, :P * 512])
    assert np.array_equal(c_gpu[:, P * 640:], c_ref[:, P * 640:])
    rg = np.ascontiguousarray(c_gpu[:, P * 512:P * 640]).view(np.uint16).reshape(-1, 64)
    rr = np.ascontiguousarray(c_ref[:, P * 512:P * 640]).view(np.uint16).reshape(-1, 64)
    for what, got, ref in (("rope", rg, rr), ("q", host_bits(qd), q_ref)):
        ok, exact, worst = within_rotation_bound(got, ref, 64)
        log(f"  {what} within bound={ok} exact frac={exact:.6f} worst/bound={worst:.3f}")
        assert ok


@pytest.mark.parametrize("P", PAGE_SIZES)
def test_combine_page_size(dsv4, P):
    rng = np.random.default_rng(400 + P)
    B, top_k, window = 4, 300, 128
    qlens = np.array([1, 3, 2, 1])
    seq_lens = np.array([2000, 777, 1300, 90], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    perm = rng.permutation(sum(pages) + 2)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    topk = rng.integers(-3, 2100, size=(T, top_k)).astype(np.int32)
    tl = rng.integers(0, top_k + 1, size=T).astype(np.int32)
    W = (top_k + window + 127) // 128 * 128
    log(f"combine P={P} T={T}")
    ref, rlen = oracle.combine(topk, tl, qsl, seq_lens, bt, T, top_k, window, P, W)
    comb = torch.full((T, W), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(dev(topk, np.int32), dev(tl, np.int32), dev(qsl, np.int32),
                              dev(seq_lens, np.int32), dev(bt, np.int32), top_k, window, comb,
                              lens, page_size=P)
    torch.cuda.synchronize()
    assert np.array_equal(comb.cpu().numpy(), ref) and np.array_equal(lens.cpu().numpy(), rlen)


@pytest.mark.parametrize("P", PAGE_SIZES)
def test_gather_page_size(dsv4, P):
    rng = np.random.default_rng(500 + P)
    num_pages = 6
    cache, _ = _oracle_cache(rng, P, num_pages, num_pages * P // 2)
    pg = cache.reshape(num_pages, -1)
    raw = rng.integers(0, 256, size=P * 512, dtype=np.uint8)
    raw[(raw & 0x7F) == 0x7F] = 0x05
    pg[2, :P * 512] = raw
    pg[2, P * 640:] = rng.integers(90, 161, size=P * 8, dtype=np.uint8)
    query = np.concatenate([rng.permutation(num_pages * P), [-1, num_pages * P]]).astype(np.int32)
    ref = oracle.gather_dequant(cache, num_pages, P, query)
    out = torch.empty(query.size, 576, dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_gather_dequant(dev(cache), dev(query), out, page_size=P)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), ref)


@pytest.mark.parametrize("P", PAGE_SIZES)
@pytest.mark.parametrize("H", [16, 128])
def test_decode_page_size(dsv4, P, H):
    rng = np.random.default_rng(600 + P + H)
    num_pages = max(2, 2048 // P)
    cache, slots = _oracle_cache(rng, P, num_pages, 1500)
    lens_list = [0, 1, 70, 640, 1100]
    T, stride = len(lens_list), 1152
    idx = np.full((T, stride), 123456789, np.int32)
    for t, L in enumerate(lens_list):
        row = rng.choice(slots, size=L).astype(np.int64)
        row[rng.random(L) < 0.08] = -1
        oor = rng.random(L) < 0.02
        row[oor] = num_pages * P + rng.integers(0, 50, oor.sum())
        idx[t, :L] = row
    lens = np.array(lens_list, np.int32)
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    log(f"decode P={P} H={H} T={T}")
    ref, rlse = oracle.sparse_mla(q, cache, num_pages, P, idx, lens, sinks, 1 / 24, nthreads=8)
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, H, dtype=torch.float32, device="cuda")
    cd, qd, idd, ld, sd = dev(cache), dev_bf16(q), dev(idx), dev(lens), dev(sinks, np.float32)
    dsv4.dsv4_sparse_mla_decode(qd, cd, idd, ld, sd, 1 / 24, out, lse, page_size=P)
    torch.cuda.synchronize()
    assert_attention_close(host_bits(out), ref, f"P={P} H={H}")
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= 2e-3
    # the split-row path reads the cache through the same page geometry
    splits = 4
    ws = torch.empty(dsv4.split_workspace_bytes(T, H, splits), dtype=torch.uint8, device="cuda")
    out2 = torch.empty_like(out)
    dsv4.dsv4_sparse_mla_decode_split(qd, cd, idd, ld, sd, 1 / 24, out2, splits, ws, page_size=P)
    torch.cuda.synchronize()
    assert_attention_close(host_bits(out2), ref, f"split P={P} H={H}")


@pytest.mark.parametrize("P", PAGE_SIZES)
def test_step_end_to_end_page_size(dsv4, P):
    """Insert the context and the new tokens, combine, decode, all on the GPU with P-slot
    pages; the oracle runs the same three steps on the host."""
    rng = np.random.default_rng(700 + P)
    B, H, top_k, window = 3, 64, 256, 64
    seq_lens = np.array([900, 333, 1500], np.int32)
    qsl = np.arange(B + 1, dtype=np.int32)
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    num_pages = sum(pages) + 1
    perm = rng.permutation(num_pages)
    bt = np.full((B, max(pages)), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    ctx_pos = np.concatenate([np.arange(L) for L in seq_lens]).astype(np.int64)
    ctx_b = np.concatenate([np.full(L, b) for b, L in enumerate(seq_lens)])
    ctx_slot = (bt[ctx_b, ctx_pos // P].astype(np.int64) * P + ctx_pos % P)
    kv = bf16_normal(rng, (ctx_pos.size, 576))
    cos_sin = rope_table(2048)
    weight = bf16_normal(rng, (576,), mean=1.0, std=0.1)
    q = bf16_normal(rng, (B, H, 576))
    topk = np.full((B, top_k), -1, np.int32)
    tl = np.zeros(B, np.int32)
    for b, L in enumerate(seq_lens):
        n = min(top_k, int(L))
        topk[b, :n] = rng.choice(L, size=n, replace=False)
        tl[b] = n
    sinks = rng.standard_normal(H).astype(np.float32)
    W = (top_k + window + 127) // 128 * 128
    log(f"end-to-end P={P} pages={num_pages}")
    # oracle: context insert, then the query tokens' q-norm/rope (no cache write), combine, attend
    cache_r = np.zeros(num_pages * P * 648, np.uint8)
    oracle.kv_insert(np.zeros((kv.shape[0], 0, 576), np.uint16), kv, ctx_pos, ctx_slot, cos_sin,
                     weight, 1e-6, cache_r, num_pages, P, inplace=True)
    qpos = seq_lens.astype(np.int64) - 1
    q_r, _ = oracle.kv_insert(q, np.zeros((B, 576), np.uint16), qpos, np.full(B, -1, np.int64),
                              cos_sin, weight, 1e-6, cache_r, num_pages, P)
    comb_r, lens_r = oracle.combine(topk, tl, qsl, seq_lens, bt, B, top_k, window, P, W)
    ref, _ = oracle.sparse_mla(q_r, cache_r, num_pages, P, comb_r, lens_r, sinks, 1 / 24, nthreads=8)
    # library
    cache = dsv4.new_cache(num_pages, page_size=P)
    cs, wd = dev(cos_sin, np.float32), dev_bf16(weight)
    dsv4.dsv4_kv_insert(None, dev_bf16(kv), dev(ctx_pos, np.int64), dev(ctx_slot, np.int64), cs,
                        None, 1e-6, cache, page_size=P)
    qd = dev_bf16(q)
    dsv4.dsv4_kv_insert(qd, dev_bf16(np.zeros((B, 576), np.uint16)), dev(qpos, np.int64),
                        dev(np.full(B, -1, np.int64)), cs, wd, 1e-6, cache, page_size=P)
    comb = torch.empty(B, W, dtype=torch.int32, device="cuda")
    lens = torch.empty(B, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(dev(topk), dev(tl), dev(qsl), dev(seq_lens), dev(bt), top_k,
                              window, comb, lens, page_size=P)
    out = torch.empty(B, H, 512, dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_mla_decode(qd, cache, comb, lens, dev(sinks, np.float32), 1 / 24, out,
                                page_size=P)
    torch.cuda.synchronize()
    assert np.array_equal(comb.cpu().numpy(), comb_r) and np.array_equal(lens.cpu().numpy(), lens_r)
    assert_attention_close(host_bits(out), ref, f"end-to-end P={P}")
