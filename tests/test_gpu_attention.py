"""GPU parity of sparse MLA decode / prefill against the fp64 oracle.

Bar (fp32 accumulation on bf16 operands): |out - oracle| <= 1e-2 on every element and
mean |out - oracle| <= 1e-3, for outputs of unit scale; elements of magnitude m > 1 get
the bar scaled by m and the mean bar by max(1, RMS) (a bf16 result is itself rounded by
2^-9 relative); lse within 2e-3 on the small cases and within 1e-4 on the benchmark
workloads, where the rows are long and the output bar alone would not see one slot too
few or too many (the GPU's lse is an fp32 sum of unrounded probabilities: its error is
~1e-6).  Covered: small
ragged cases spanning several 64-slot chunks for every supported head count, -1 holes,
out-of-range and duplicated slots, empty and all-invalid rows, sinks on/off, peaked
logits (q x 8), every benchmark workload at full size (the oracle on all tokens of the
decode batch, on sampled tokens of the MTP and prefill batches), determinism, and
guard rows around the outputs."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import attention_workload, bf16_normal, rope_table
from tests.gpu_helpers import (assert_attention_close, bits_to_f64, dev, dev_bf16, host_bits,
                               log, oracle_cache)

pytestmark = pytest.mark.gpu
P = 64


def run_gpu(dsv4, q_bits, cache_dev, idx, lens, sinks, scale, prefill=False, guard=3):
    T, H = q_bits.shape[0], q_bits.shape[1]
    out_full = torch.full((T + guard, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_full = torch.full((T + guard, H), 7.0, dtype=torch.float32, device="cuda")
    out, lse = out_full[:T], lse_full[:T]
    fn = dsv4.dsv4_sparse_mla_prefill if prefill else dsv4.dsv4_sparse_mla_decode
    fn(dev_bf16(q_bits), cache_dev, dev(idx, np.int32), dev(lens, np.int32),
       None if sinks is None else dev(sinks, np.float32), scale, out, lse)
    torch.cuda.synchronize()
    assert torch.all(out_full[T:] == 7.0) and torch.all(lse_full[T:] == 7.0), "guard rows written"
    return host_bits(out), lse.cpu().numpy()


def _random_cache(rng, num_pages, n_slots):
    cache = np.zeros(num_pages * P * 648, np.uint8)
    slots = rng.choice(num_pages * P, size=n_slots, replace=False).astype(np.int64)
    kv = bf16_normal(rng, (n_slots, 576))
    from synth_inputs import rope_table
    _, cache = oracle.kv_insert(np.zeros((n_slots, 0, 576), np.uint16), kv,
                                rng.integers(0, 1000, n_slots), slots, rope_table(1000),
                                np.zeros(576, np.uint16), 1e-6, cache, num_pages, P)
    return cache, slots


def _check(dsv4, name, q, cache, num_pages, idx, lens, sinks, scale, prefill=False):
    log(f"case {name}: T={q.shape[0]} H={q.shape[1]} stride={idx.shape[1]} prefill={prefill}")
    ref, rlse = oracle.sparse_mla(q, cache, num_pages, P, idx, lens, sinks, scale, nthreads=8)
    got, glse = run_gpu(dsv4, q, dev(cache), idx, lens, sinks, scale, prefill=prefill)
    assert_attention_close(got, ref, name)
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(glse)), name
    assert np.all(np.isneginf(glse[~fin])) and np.all(np.isneginf(rlse[~fin]))
    if fin.any():
        assert np.max(np.abs(glse[fin] - rlse[fin])) <= 2e-3, name
    return got


@pytest.mark.parametrize("H", [16, 32, 64, 128])
@pytest.mark.parametrize("sinks_on", [False, True])
def test_small_ragged(dsv4, H, sinks_on):
    rng = np.random.default_rng(H + 7 * sinks_on)
    num_pages = 12
    cache, slots = _random_cache(rng, num_pages, 700)
    lens_list = [0, 1, 15, 63, 64, 65, 130, 200, 333]
    T = len(lens_list)
    stride = 384
    idx = np.full((T, stride), 999999, np.int32)  # garbage past each length
    for t, L in enumerate(lens_list):
        row = rng.choice(slots, size=L, replace=True).astype(np.int64)  # duplicates allowed
        holes = rng.random(L) < 0.1
        row[holes] = -1
        oor = rng.random(L) < 0.03
        row[oor] = num_pages * P + rng.integers(0, 100, oor.sum())
        idx[t, :L] = row
    idx[-1, :] = -1  # an all-invalid row
    lens = np.array(lens_list, np.int32)
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32) if sinks_on else None
    for prefill in (False, True):
        _check(dsv4, f"small H={H} sinks={sinks_on}", q, cache, num_pages, idx, lens, sinks,
               1.0 / 24, prefill=prefill)
    qp = bf16_normal(rng, (T, H, 576), std=8.0)
    _check(dsv4, f"peaked H={H} sinks={sinks_on}", qp, cache, num_pages, idx, lens, sinks, 1.0 / 24)


def test_lens_beyond_stride_and_negative(dsv4):
    rng = np.random.default_rng(3)
    cache, slots = _random_cache(rng, 4, 200)
    idx = rng.choice(slots, size=(3, 96)).astype(np.int32)
    lens = np.array([500, -5, 96], np.int32)
    q = bf16_normal(rng, (3, 16, 576))
    _check(dsv4, "lens clamp", q, cache, 4, idx, lens, None, 0.05)


LSE_BAR = 1e-4  # benchmark workloads: one slot of ~1700 moves lse by ~4e-4 (median weight)


def _drop_median_slot(ref_lse, q, cache, num_pages, idx, lens, sinks, scale, n=6):
    """The oracle with, in each of the first n rows, the entry of median softmax weight
    (head 0) replaced by -1: how far one missing slot moves lse.  Run on the CPU only, to
    show that the lse bar of the GPU comparison would catch it."""
    idx2 = idx[:n].copy()
    for t in range(n):
        L = int(lens[t])
        valid = np.nonzero((idx2[t, :L] >= 0) & (idx2[t, :L] < num_pages * P))[0]
        rows = oracle.gather_dequant(cache, num_pages, P, idx2[t, valid].astype(np.int32))
        s = bits_to_f64(rows) @ bits_to_f64(q[t, 0])
        idx2[t, valid[np.argsort(s)[len(s) // 2]]] = -1
    _, lse2 = oracle.sparse_mla(q[:n], cache, num_pages, P, idx2, lens[:n], sinks, scale,
                                nthreads=16)
    return np.abs(lse2[:, 0] - ref_lse[:n, 0])


def _workload_case(dsv4, cfg, sample=None, prefill=False, q_mul=None):
    wl = attention_workload(cfg, ctx_tokens=sample)
    it = wl["instances"][0]
    q = it["q"]
    if q_mul is not None:  # peaked logits: q scaled by a power of two (exact in bf16)
        q = (bits_to_f64(q) * q_mul).astype(np.float32).view(np.uint32) >> 16
        q = q.astype(np.uint16).reshape(it["q"].shape)
    log(f"workload cfg={cfg}: T={wl['T']} H={wl['H']} ctx rows={wl['ctx_kv'].shape[0]} "
        f"pages={wl['num_pages']} q_mul={q_mul}")
    cache = oracle_cache(wl)
    idx, lens = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                               wl["block_table"], wl["T"], wl["top_k"], wl["window"], P, wl["W"])
    cache_dev = dev(cache)
    got, glse = run_gpu(dsv4, q, cache_dev, idx, lens, it["sinks"], wl["softmax_scale"],
                        prefill=prefill)
    toks = np.arange(wl["T"]) if sample is None else np.asarray(sample)
    ref, rlse = oracle.sparse_mla(q[toks], cache, wl["num_pages"], P, idx[toks], lens[toks],
                                  it["sinks"], wl["softmax_scale"], nthreads=16)
    assert_attention_close(got[toks], ref, f"cfg{cfg}", out_rounding=q_mul is not None)
    lerr = float(np.max(np.abs(glse[toks] - rlse)))
    log(f"  cfg{cfg}: max |lse - oracle| = {lerr:.3e} (bar {LSE_BAR:.0e})")
    assert lerr <= LSE_BAR
    # determinism: a second run is bit-identical
    got2, _ = run_gpu(dsv4, q, cache_dev, idx, lens, it["sinks"], wl["softmax_scale"],
                      prefill=prefill)
    assert np.array_equal(got, got2)
    return wl, idx, lens, (q, cache, rlse, toks)


def test_cfg0_tiny_decode(dsv4):
    _workload_case(dsv4, 0)


def test_cfg2_decode_full(dsv4):
    wl, idx, lens, (q, cache, rlse, toks) = _workload_case(dsv4, 2)
    it = wl["instances"][0]
    moved = _drop_median_slot(rlse, q, cache, wl["num_pages"], idx, lens, it["sinks"],
                              wl["softmax_scale"])
    log(f"  one median-weight slot dropped moves lse by {moved.min():.2e} .. {moved.max():.2e}")
    assert np.all(moved > 2 * LSE_BAR)  # a dropped slot would fail the bar with margin


def test_cfg2_decode_full_peaked(dsv4):
    """The benchmark batch with q x 8: logits with sigma ~8, so a few slots carry most of
    each row's weight and every output element depends on them.  The outputs are then
    whole value rows of unit scale (RMS ~0.8), where the bf16 output's own rounding is
    ~1e-3 on average, so the mean bar adds the oracle value's mean bf16 rounding."""
    _workload_case(dsv4, 2, q_mul=8.0)


def test_cfg3_mtp_decode_sampled(dsv4):
    rng = np.random.default_rng(33)
    sample = np.sort(rng.choice(512, size=24, replace=False))
    _workload_case(dsv4, 3, sample=sample)


def test_cfg4_prefill_sampled(dsv4):
    rng = np.random.default_rng(44)
    sample = np.unique(np.concatenate([[0, 1, 2, 63, 64, 127, 128, 2046, 2047, 2048, 8191],
                                       rng.choice(8192, size=37, replace=False)]))
    _workload_case(dsv4, 4, sample=sample, prefill=True)


def _long_rows(rng, stride, T, H, num_pages=200):
    """Rows longer than the 4096-entry LDS index block: lengths at and around the block
    edges and the stride, -1 holes, out-of-range slots, repeats."""
    cache, slots = _random_cache(rng, num_pages, num_pages * P - 100)
    lens_list = [stride, 4095, 4096, 4097, stride - 37, int(rng.integers(4097, stride + 1))][:T]
    lens_list = [min(L, stride) for L in lens_list]
    idx = np.full((T, stride), -1, np.int32)
    for t, L in enumerate(lens_list):
        row = rng.choice(slots, size=L, replace=True).astype(np.int64)
        row[rng.random(L) < 0.05] = -1
        oor = rng.random(L) < 0.01
        row[oor] = num_pages * P + rng.integers(0, 100, oor.sum())
        idx[t, :L] = row
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    return cache, idx, np.array(lens_list, np.int32), q, sinks


@pytest.mark.parametrize("stride", [4097, 4096 * 2 + 37, 4096 * 3])
@pytest.mark.parametrize("H", [16, 64])
def test_rows_past_one_index_block(dsv4, stride, H):
    """decode, prefill and the split decode (pieces crossing the block edges) on rows of
    more than 4096 entries, against the oracle; the split forms also against the unsplit
    decode within the bar, and the decode with an auto-split workspace bit for bit
    against the split decode with the piece count it reports."""
    rng = np.random.default_rng(stride + H)
    T, num_pages = 6, 200
    cache, idx, lens, q, sinks = _long_rows(rng, stride, T, H, num_pages)
    log(f"long rows: stride={stride} H={H} lens={lens.tolist()}")
    ref, rlse = oracle.sparse_mla(q, cache, num_pages, P, idx, lens, sinks, 1 / 24, nthreads=16)
    cache_dev = dev(cache)

    def check(name, got, glse):
        assert_attention_close(got, ref, name)
        err = float(np.max(np.abs(glse - rlse)))
        log(f"  {name}: max |lse - oracle| = {err:.3e}")
        assert err <= LSE_BAR, name

    for prefill in (False, True):
        got, glse = run_gpu(dsv4, q, cache_dev, idx, lens, sinks, 1 / 24, prefill=prefill)
        check(f"{'prefill' if prefill else 'decode'} stride={stride}", got, glse)
    qd, idd, ld, sd = dev_bf16(q), dev(idx, np.int32), dev(lens, np.int32), dev(sinks, np.float32)
    for splits in (2, 3, 5):
        ws = torch.empty(dsv4.split_workspace_bytes(T, H, splits), dtype=torch.uint8,
                         device="cuda")
        out = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(T, H, dtype=torch.float32, device="cuda")
        dsv4.dsv4_sparse_mla_decode_split(qd, cache_dev, idd, ld, sd, 1 / 24, out, splits, ws,
                                          lse=lse)
        torch.cuda.synchronize()
        check(f"split {splits} stride={stride}", host_bits(out), lse.cpu().numpy())
    # the decode given a workspace picks its own piece count for this small batch
    nb = dsv4.workspace_bytes(T, H, stride)
    groups = 1 if H == 16 else H // 32
    auto = min(8, 256 // (T * groups))
    while auto > 1 and stride < 256 * auto:
        auto -= 1
    assert nb == dsv4.split_workspace_bytes(T, H, auto) > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out_a = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    lse_a = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode(qd, cache_dev, idd, ld, sd, 1 / 24, out_a, lse_a, workspace=ws)
    out_s = torch.empty_like(out_a)
    lse_s = torch.empty_like(lse_a)
    ws2 = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dsv4.dsv4_sparse_mla_decode_split(qd, cache_dev, idd, ld, sd, 1 / 24, out_s, auto, ws2,
                                      lse=lse_s)
    torch.cuda.synchronize()
    assert torch.equal(out_a.view(torch.int16), out_s.view(torch.int16))
    assert torch.equal(lse_a.view(torch.int32), lse_s.view(torch.int32))
    check(f"decode+workspace ({auto} pieces) stride={stride}", host_bits(out_a),
          lse_a.cpu().numpy())


@pytest.mark.parametrize("kvd,kvs", [(0, 1.0), (1, 1.0), (2, 0.0371)], ids=["packed", "bf16", "fp8"])
@pytest.mark.parametrize("H", [32, 64, 128])
def test_prefill_persistent_equals_decode(dsv4, H, kvd, kvs):
    """Prefill batches of many rows run on persistent workgroups that loop over (token,
    head group) items, copying each next row into LDS and requesting its Q while the
    current item finishes: out and lse bit for bit equal to the one-workgroup-per-item
    decode, on 600 tokens (several items per workgroup) with ragged, empty and full rows
    of up to 2304 entries, -1 holes and out-of-range slots; sampled tokens against the
    oracle."""
    rng = np.random.default_rng(5000 + H + 7 * kvd)
    P, num_pages, T, stride = 64, 80, 600, 2304
    rb = oracle.kv_record_bytes(kvd)
    slots = rng.choice(num_pages * P, size=4000, replace=False).astype(np.int64)
    cache = np.zeros(num_pages * P * rb, np.uint8)
    _, cache = oracle.kv_insert(np.zeros((slots.size, 0, 576), np.uint16),
                                bf16_normal(rng, (slots.size, 576)), rng.integers(0, 900, slots.size),
                                slots, rope_table(900), np.zeros(576, np.uint16), 1e-6, cache,
                                num_pages, P, kv_dtype=kvd, kv_scale=kvs)
    lens = rng.integers(0, stride + 1, T).astype(np.int32)
    lens[:5] = [0, 1, 64, stride, stride]
    idx = rng.choice(slots, size=(T, stride)).astype(np.int32)
    idx[rng.random((T, stride)) < 0.05] = -1
    idx[rng.random((T, stride)) < 0.01] = num_pages * P + 3
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    cache_dev, qd, idd, ld, sd = dev(cache), dev_bf16(q), dev(idx), dev(lens), dev(sinks)
    res = []
    for fn in (dsv4.dsv4_sparse_mla_prefill, dsv4.dsv4_sparse_mla_decode):
        out = torch.full((T, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
        lse = torch.full((T, H), 7.0, dtype=torch.float32, device="cuda")
        fn(qd, cache_dev, idd, ld, sd, 1.0 / 24, out, lse, kv_dtype=kvd, kv_scale=kvs)
        torch.cuda.synchronize()
        res.append((out, lse))
    log(f"prefill persistent H={H} kv_dtype={kvd} T={T}")
    (op, lp), (od, ldd) = res
    assert torch.equal(op.view(torch.int16), od.view(torch.int16))
    assert torch.equal(lp.view(torch.int32), ldd.view(torch.int32))
    toks = np.array([0, 1, 2, 3, 4, 299, T - 1])
    ref, rlse = oracle.sparse_mla(q[toks], cache, num_pages, P, idx[toks], lens[toks], sinks,
                                  1.0 / 24, nthreads=8, kv_dtype=kvd, kv_scale=kvs)
    assert_attention_close(host_bits(op)[toks], ref, f"prefill persistent H={H}")
    gl = lp.cpu().numpy()[toks]
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(gl)) and np.max(np.abs(gl[fin] - rlse[fin])) <= 2e-3
