"""GPU parity of the indexer top-k selection (the step before the combine): bit-exact
ids and counts against the oracle on random rows full of ties, NaN and infinities, on
short rows and top_k 0, at the decode size (64 tokens x 32768 candidates, top-k 2048),
and through the chain indexer -> combine -> decode."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import bf16_normal, rope_table
from tests.gpu_helpers import assert_attention_close, dev, dev_bf16, host_bits, log

pytestmark = pytest.mark.gpu


def _gpu_topk(dsv4, logits, qsl, seq_lens, T, ratio, top_k, stride):
    out = torch.full((T, stride), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    dsv4.dsv4_indexer_topk(dev(logits, np.float32), dev(qsl, np.int32), dev(seq_lens, np.int32),
                           top_k, out, lens, compress_ratio=ratio)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lens.cpu().numpy()


@pytest.mark.parametrize("seed", range(8))
def test_indexer_topk_random(dsv4, seed):
    rng = np.random.default_rng(1200 + seed)
    B = int(rng.integers(1, 5))
    ratio = int(rng.choice([1, 1, 4, 128]))
    top_k = int(rng.choice([0, 1, 64, 700, 2048]))
    width = int(rng.integers(1, 9000))
    qlens = rng.integers(1, 7, size=B)
    seq_lens = np.array([int(rng.integers(ql, 12000)) for ql in qlens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32) + int(rng.integers(0, 3))
    T = int(qsl[-1] - qsl[0]) + 2
    scale = float(rng.choice([1.0, 64.0]))  # coarse values -> many ties at the threshold
    logits = (np.round(rng.standard_normal((T, width)) * scale) / scale).astype(np.float32)
    logits[rng.random((T, width)) < 0.02] = np.nan
    logits[rng.random((T, width)) < 0.02] = -np.inf
    logits[rng.random((T, width)) < 0.002] = np.inf
    logits[rng.random((T, width)) < 0.01] = -0.0
    stride = top_k + int(rng.integers(0, 5))
    log(f"indexer seed={seed} B={B} T={T} ratio={ratio} top_k={top_k} width={width}")
    ref, rlen = oracle.indexer_topk(logits, qsl, seq_lens, T, ratio, top_k, stride)
    got, glen = _gpu_topk(dsv4, logits, qsl, seq_lens, T, ratio, top_k, stride)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def test_indexer_topk_decode_size(dsv4):
    rng = np.random.default_rng(1300)
    T, L, top_k = 64, 32768, 2048
    qsl = np.arange(T + 1, dtype=np.int32)
    seq_lens = np.full(T, L, np.int32)
    seq_lens[:8] = rng.integers(1, 4000, 8)  # some short contexts
    logits = rng.standard_normal((T, L)).astype(np.float32)
    logits[5, :] = 1.0  # one row of all-equal logits: the smallest ids win
    log("indexer decode size 64 x 32768")
    ref, rlen = oracle.indexer_topk(logits, qsl, seq_lens, T, 1, top_k, top_k)
    got, glen = _gpu_topk(dsv4, logits, qsl, seq_lens, T, 1, top_k, top_k)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def test_indexer_combine_decode_chain(dsv4):
    """Indexer -> combine -> decode on the GPU against the same oracle chain."""
    rng = np.random.default_rng(1400)
    P, B, H, top_k, window = 64, 6, 32, 256, 64
    seq_lens = rng.integers(100, 3000, B).astype(np.int32)
    qsl = np.arange(B + 1, dtype=np.int32)
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    npg = sum(pages)
    perm = rng.permutation(npg)
    bt = np.full((B, max(pages)), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    cache = np.zeros(npg * P * 648, np.uint8)
    pos = np.concatenate([np.arange(L) for L in seq_lens]).astype(np.int64)
    bid = np.concatenate([np.full(L, b) for b, L in enumerate(seq_lens)])
    slots = bt[bid, pos // P].astype(np.int64) * P + pos % P
    oracle.kv_insert(np.zeros((pos.size, 0, 576), np.uint16), bf16_normal(rng, (pos.size, 576)),
                     pos, slots, rope_table(3000), np.zeros(576, np.uint16), 1e-6, cache, npg, P,
                     inplace=True)
    logits = rng.standard_normal((B, 3000)).astype(np.float32)
    q = bf16_normal(rng, (B, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    W = (top_k + window + 127) // 128 * 128
    tk_r, tl_r = oracle.indexer_topk(logits, qsl, seq_lens, B, 1, top_k, top_k)
    comb_r, lens_r = oracle.combine(tk_r, tl_r, qsl, seq_lens, bt, B, top_k, window, P, W)
    ref, _ = oracle.sparse_mla(q, cache, npg, P, comb_r, lens_r, sinks, 1 / 24, nthreads=8)
    tk = torch.empty(B, top_k, dtype=torch.int32, device="cuda")
    tl = torch.empty(B, dtype=torch.int32, device="cuda")
    qsl_d, sl_d = dev(qsl), dev(seq_lens)
    dsv4.dsv4_indexer_topk(dev(logits), qsl_d, sl_d, top_k, tk, tl)
    comb = torch.empty(B, W, dtype=torch.int32, device="cuda")
    lens = torch.empty(B, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices(tk, tl, qsl_d, sl_d, dev(bt), top_k, window, comb, lens)
    out = torch.empty(B, H, 512, dtype=torch.bfloat16, device="cuda")
    dsv4.dsv4_sparse_mla_decode(dev_bf16(q), dev(cache), comb, lens, dev(sinks), 1 / 24, out)
    torch.cuda.synchronize()
    assert np.array_equal(tk.cpu().numpy(), tk_r) and np.array_equal(comb.cpu().numpy(), comb_r)
    assert_attention_close(host_bits(out), ref, "indexer chain")


def test_indexer_topk_many_tokens(dsv4):
    """T >= 1024 takes the small-workgroup schedule: a 1500-token prefill, causal
    candidates, coarse logits with ties."""
    rng = np.random.default_rng(1500)
    L, top_k = 1500, 300
    qsl = np.array([0, L], np.int32)
    seq = np.array([L], np.int32)
    logits = (np.round(rng.standard_normal((L, L)) * 8) / 8).astype(np.float32)
    logits[rng.random((L, L)) < 0.01] = np.nan
    log("indexer many tokens 1500 x 1500")
    ref, rlen = oracle.indexer_topk(logits, qsl, seq, L, 1, top_k, top_k)
    got, glen = _gpu_topk(dsv4, logits, qsl, seq, L, 1, top_k, top_k)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def test_indexer_topk_many_tokens_staged_and_reread(dsv4):
    """T >= 1024 takes the 4-wave schedule, which stages rows of up to 8192 candidates in
    LDS and rereads longer ones: a 1100-token request whose causal rows hold 7501..8600
    candidates, coarse logits with ties, NaN and -inf, top-k 2048; two staged rows whose
    2048th-largest logit is shared by 512 and by 513 keys (either side of the list limit
    of keys sharing its first two radix digits)."""
    rng = np.random.default_rng(1700)
    T, width, top_k = 1100, 8700, 2048
    qsl = np.array([0, T], np.int32)
    seq = np.array([8600], np.int32)  # token i at position 7500 + i: n = 7501 + i
    logits = (np.round(rng.standard_normal((T, width)) * 16) / 16).astype(np.float32)
    logits[rng.random((T, width)) < 0.01] = np.nan
    logits[rng.random((T, width)) < 0.01] = -np.inf
    for t, ties in ((3, 512), (4, 513)):
        n = 7501 + t
        perm = rng.permutation(n)
        logits[t, :] = -1.0
        logits[t, perm[:top_k - 1]] = 10.0
        logits[t, perm[top_k - 1:top_k - 1 + ties]] = 5.0
    log("indexer many tokens 1100 x 7501..8600 (staged and reread)")
    ref, rlen = oracle.indexer_topk(logits, qsl, seq, T, 1, top_k, top_k)
    got, glen = _gpu_topk(dsv4, logits, qsl, seq, T, 1, top_k, top_k)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def test_indexer_topk_rows_longer_than_the_lds_stage(dsv4):
    """Few tokens with more than 32768 candidates: the large-workgroup schedule rereads
    the row instead of staging it."""
    rng = np.random.default_rng(1600)
    T, L, top_k = 4, 50000, 2048
    qsl = np.arange(T + 1, dtype=np.int32)
    seq = np.array([50000, 32769, 32768, 40000], np.int32)
    logits = rng.standard_normal((T, L)).astype(np.float32)
    log("indexer long rows 4 x 50000")
    ref, rlen = oracle.indexer_topk(logits, qsl, seq, T, 1, top_k, top_k)
    got, glen = _gpu_topk(dsv4, logits, qsl, seq, T, 1, top_k, top_k)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def test_indexer_topk_zero_width_output(dsv4):
    """top_k 0 with a zero-width topk (a NULL pointer): only the counts are written."""
    qsl = np.array([0, 2], np.int32)
    seq = np.array([100], np.int32)
    lens = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    out = torch.empty((2, 0), dtype=torch.int32, device="cuda")
    dsv4.dsv4_indexer_topk(dev(np.zeros((2, 64), np.float32)), dev(qsl), dev(seq), 0, out, lens)
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [0, 0]


@pytest.mark.parametrize("ties", [1, 511, 512, 513, 1023, 1024, 1025, 5000])
def test_indexer_threshold_bin_sizes(dsv4, ties):
    """Rows staged in LDS list the keys that share the k-th largest key's first two radix
    digits when there are at most 512 of them (the emission's counts then come from the
    list), and count them with a sweep over the row otherwise: a row of 99 logits 10.0,
    `ties` logits 5.0 (the k-th largest, all equal) and -1.0 elsewhere, k = 100, on both
    sides of that limit; ids must match the oracle bit for bit (ties to the smaller id)."""
    rng = np.random.default_rng(1400 + ties)
    T, L, top_k = 3, 8192, 100
    logits = np.full((T, L), -1.0, np.float32)
    for t in range(T):
        perm = rng.permutation(L)
        logits[t, perm[:99]] = 10.0
        logits[t, perm[99:99 + ties]] = 5.0
    qsl = np.arange(T + 1, dtype=np.int32)
    seq_lens = np.full(T, L, np.int32)
    log(f"indexer threshold bin of {ties} equal keys")
    ref, rlen = oracle.indexer_topk(logits, qsl, seq_lens, T, 1, top_k, top_k)
    got, glen = _gpu_topk(dsv4, logits, qsl, seq_lens, T, 1, top_k, top_k)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)
