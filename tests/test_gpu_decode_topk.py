"""GPU parity of the fused combine + decode (dsv4_sparse_mla_decode_topk): its output and
lse are bit-identical to dsv4_combine_indices followed by dsv4_sparse_mla_decode (the
same index rows, the same attention arithmetic) on random multi-token requests with
windows, topk_lens, holes and tokens of no request, at both head-group shapes and two
page sizes, on the full benchmark workload, and under HIP-graph replay; and equal to the
oracle within the attention bar on a small case."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import attention_workload, bf16_normal, rope_table
from tests.gpu_helpers import assert_attention_close, dev, dev_bf16, host_bits, log, oracle_cache

pytestmark = pytest.mark.gpu


def _two_step(dsv4, q, cache, topk, tl, qsl, sl, bt, top_k, window, sinks, P, W):
    T, H = q.shape[0], q.shape[1]
    comb = torch.empty(T, W, dtype=torch.int32, device="cuda")
    lens = torch.zeros(T, dtype=torch.int32, device="cuda")  # rows of no request: empty
    comb.fill_(-1)
    dsv4.dsv4_combine_indices(topk, tl, qsl, sl, bt, top_k, window, comb, lens, page_size=P)
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode(q, cache, comb, lens, sinks, 1 / 24, out, lse, page_size=P)
    return out, lse, comb, lens


def _fused(dsv4, q, cache, topk, tl, qsl, sl, bt, top_k, window, sinks, P):
    T, H = q.shape[0], q.shape[1]
    out = torch.full((T, H, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((T, H), 3.0, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_topk(q, cache, topk, tl, qsl, sl, bt, top_k, window, sinks, 1 / 24,
                                     out, lse, page_size=P)
    return out, lse


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


@pytest.mark.parametrize("seed", range(6))
def test_decode_topk_equals_combine_then_decode(dsv4, seed):
    rng = np.random.default_rng(2000 + seed)
    P = [64, 32][seed % 2]
    H = [128, 16, 64][seed % 3]
    B = int(rng.integers(1, 6))
    top_k = int(rng.choice([16, 300, 2048]))
    window = int(rng.choice([0, 1, 128]))
    qlens = rng.integers(1, 4, size=B)
    seq_lens = np.array([int(rng.integers(ql, 3000)) for ql in qlens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32) + int(rng.integers(0, 2))
    T = int(qsl[-1] - qsl[0]) + 2  # the last two tokens belong to no request
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    npg = sum(pages) + 2
    perm = rng.permutation(npg)
    bt = np.full((B, max(pages) + 1), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    bt[0, 0] = -1  # a hole in the table
    pos = np.concatenate([np.arange(L) for L in seq_lens]).astype(np.int64)
    bid = np.concatenate([np.full(L, b) for b, L in enumerate(seq_lens)])
    keep = bt[bid, pos // P] >= 0
    cache = np.zeros(npg * P * 648, np.uint8)
    slots = bt[bid[keep], pos[keep] // P].astype(np.int64) * P + pos[keep] % P
    oracle.kv_insert(np.zeros((slots.size, 0, 576), np.uint16), bf16_normal(rng, (slots.size, 576)),
                     pos[keep], slots, rope_table(3000), np.zeros(576, np.uint16), 1e-6, cache, npg,
                     P, inplace=True)
    topk = rng.integers(-3, 3100, size=(T, top_k)).astype(np.int32)
    tl = rng.integers(0, top_k + 2, size=T).astype(np.int32) if seed % 2 else None
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32) if seed % 3 else None
    W = (top_k + window + 127) // 128 * 128
    log(f"decode_topk seed={seed} P={P} H={H} B={B} T={T} top_k={top_k} window={window}")
    args = (dev_bf16(q), dev(cache), dev(topk), None if tl is None else dev(tl), dev(qsl),
            dev(seq_lens), dev(bt), top_k, window, None if sinks is None else dev(sinks))
    out2, lse2, _, _ = _two_step(dsv4, *args, P, W)
    out1, lse1 = _fused(dsv4, *args, P)
    torch.cuda.synchronize()
    assert _same(out1, out2) and _same(lse1, lse2)
    # tokens of no request attend to no slot: output 0; lse -inf, or the sink alone
    assert torch.all(out1[-2:].float() == 0)
    if sinks is None:
        assert torch.all(torch.isneginf(lse1[-2:]))


@pytest.mark.parametrize("P", [32, 64])
def test_decode_topk_long_block_tables(dsv4, P):
    """Requests whose block-table rows are longer than the entries a workgroup stages in
    LDS (16384 pages: positions past 2^19 at 32 slots a page, 2^20 at 64) take the
    per-entry lookups in memory; shorter ones the staged copy.  Both against the separate
    combine + decode, bit for bit.  The logical pages map into a small pool of physical
    pages (with holes), so the cache stays small."""
    rng = np.random.default_rng(2400 + P)
    npg = 48
    seq_lens = np.array([16384 * P + 977, 16384 * P - 5, 16384 * P + 1, 3000], np.int32)
    B = seq_lens.size
    qlens = np.array([1, 2, 1, 1])
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    pages = (seq_lens.astype(np.int64) + P - 1) // P
    bt = rng.integers(0, npg, size=(B, int(pages.max()))).astype(np.int32)
    bt[rng.random(bt.shape) < 0.01] = -1  # holes
    cache = np.zeros(npg * P * 648, np.uint8)
    slots = np.arange(npg * P, dtype=np.int64)
    oracle.kv_insert(np.zeros((slots.size, 0, 576), np.uint16), bf16_normal(rng, (slots.size, 576)),
                     slots % 3000, slots, rope_table(3000), np.zeros(576, np.uint16), 1e-6, cache,
                     npg, P, inplace=True)
    top_k, window, H = 512, 64, 64
    pos = np.concatenate([L - ql + np.arange(ql) for L, ql in zip(seq_lens, qlens)])
    topk = np.stack([rng.integers(0, p + 1, size=top_k) for p in pos]).astype(np.int32)
    topk[:, -7:] = -1
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    W = (top_k + window + 127) // 128 * 128
    log(f"decode_topk long block tables P={P} rows of {pages.tolist()} pages")
    args = (dev_bf16(q), dev(cache), dev(topk), None, dev(qsl), dev(seq_lens), dev(bt), top_k,
            window, dev(sinks))
    out2, lse2, _, lens = _two_step(dsv4, *args, P, W)
    out1, lse1 = _fused(dsv4, *args, P)
    torch.cuda.synchronize()
    assert _same(out1, out2) and _same(lse1, lse2)
    assert int(lens.min().item()) > 0


def test_decode_topk_benchmark_workload(dsv4):
    wl = attention_workload(2, seed=11, instances=1)
    it = wl["instances"][0]
    cache = dsv4.new_cache(wl["num_pages"])
    dsv4.dsv4_kv_insert(None, dev_bf16(wl["ctx_kv"]), dev(wl["ctx_pos"], np.int64),
                        dev(wl["ctx_slot"], np.int64), dev(wl["cos_sin"], np.float32), None,
                        wl["eps"], cache)
    args = (dev_bf16(it["q"]), cache, dev(it["topk"]), dev(it["topk_lens"]), dev(wl["qsl"]),
            dev(wl["seq_lens"]), dev(wl["block_table"]), wl["top_k"], wl["window"],
            dev(it["sinks"]))
    log("decode_topk benchmark workload")
    out2, lse2, _, _ = _two_step(dsv4, *args, 64, wl["W"])
    out1, lse1 = _fused(dsv4, *args, 64)
    torch.cuda.synchronize()
    assert _same(out1, out2) and _same(lse1, lse2)
    # graph replays of the fused launch reproduce it bit for bit
    gout = torch.empty_like(out1)
    glse = torch.empty_like(lse1)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        dsv4.dsv4_sparse_mla_decode_topk(*args, 1 / 24, gout, glse)
    for r in range(3):
        gout.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(gout, out1) and _same(glse, lse1), r


def test_decode_topk_against_oracle(dsv4):
    wl = attention_workload(0)
    it = wl["instances"][0]
    cache = oracle_cache(wl)
    ref_idx, ref_lens = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                                       wl["block_table"], wl["T"], wl["top_k"], wl["window"], 64,
                                       wl["W"])
    ref, rlse = oracle.sparse_mla(it["q"], cache, wl["num_pages"], 64, ref_idx, ref_lens, None,
                                  wl["softmax_scale"])
    out = torch.empty(wl["T"], wl["H"], 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(wl["T"], wl["H"], dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_topk(dev_bf16(it["q"]), dev(cache), dev(it["topk"]),
                                     dev(it["topk_lens"]), dev(wl["qsl"]), dev(wl["seq_lens"]),
                                     dev(wl["block_table"]), wl["top_k"], wl["window"], None,
                                     wl["softmax_scale"], out, lse)
    torch.cuda.synchronize()
    assert_attention_close(host_bits(out), ref, "decode_topk cfg0")
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= 2e-3
