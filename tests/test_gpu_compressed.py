"""GPU parity of the compressed-cache form (PR #43385: top-k over compressed entries,
the window over raw tokens, indices into a per-request workspace of M rows): the index
combine bit-exact against the oracle on random and edge cases and at a prefill size,
the workspace bytes exact, and the chain combine -> workspace -> attention end to end
against the oracle's same chain."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import bf16_normal, rope_table
from tests.gpu_helpers import assert_attention_close, dev, dev_bf16, host_bits, log

pytestmark = pytest.mark.gpu


def _gpu_combine(dsv4, topk, tl, qsl, sl, gl, T, top_k, ratio, window, M, N, W, topk_width=None):
    comb = torch.full((T, W), -7, dtype=torch.int32, device="cuda")
    lens = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    dsv4.dsv4_combine_indices_compressed(dev(topk, np.int32), None if tl is None else dev(tl, np.int32),
                                         dev(qsl, np.int32), dev(sl, np.int32), dev(gl, np.int32),
                                         top_k, ratio, window, M, N, comb, lens,
                                         topk_width=topk_width)
    torch.cuda.synchronize()
    return comb.cpu().numpy(), lens.cpu().numpy()


@pytest.mark.parametrize("seed", range(8))
def test_combine_compressed_random(dsv4, seed):
    rng = np.random.default_rng(900 + seed)
    B = int(rng.integers(1, 6))
    ratio = int(rng.choice([1, 4, 16, 128]))
    top_k = int(rng.choice([0, 8, 64, 300]))
    window = int(rng.choice([0, 1, 128]))
    width = top_k + int(rng.integers(0, 4))
    qlens = rng.integers(1, 6, size=B)
    seq_lens = np.array([int(rng.integers(ql, 3000)) for ql in qlens], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32) + int(rng.integers(0, 3))
    T = int(qsl[-1] - qsl[0]) + 2
    N = int(rng.integers(0, 400))
    gl = np.array([int(rng.integers(-3, L + 5)) for L in seq_lens], np.int32)
    M = N + int(rng.integers(0, 3200))
    topk = rng.integers(-5, N + 20, size=(T, max(width, 1))).astype(np.int32)
    tl = rng.integers(-2, top_k + 3, size=T).astype(np.int32) if seed % 2 else None
    W = (top_k + window + 127) // 128 * 128 + 128 * int(seed % 3 == 0)
    log(f"compressed combine seed={seed} B={B} ratio={ratio} top_k={top_k} window={window} M={M} N={N}")
    ref, rlen = oracle.combine_compressed(topk, tl, qsl, seq_lens, gl, T, top_k, ratio, window, M, N,
                                          W, topk_width=width)
    got, glen = _gpu_combine(dsv4, topk, tl, qsl, seq_lens, gl, T, top_k, ratio, window, M, N, W,
                             topk_width=width)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def test_combine_compressed_prefill_size(dsv4):
    """One 8192-token sequence, ratio 4 (2048 compressed entries), top-k 2048, window 128,
    every raw token gathered: M = N + 8192."""
    rng = np.random.default_rng(77)
    L, ratio, top_k, window = 8192, 4, 2048, 128
    N, M = L // ratio, L // ratio + L
    seq = np.array([L], np.int32)
    qsl = np.array([0, L], np.int32)
    topk = np.full((L, top_k), -1, np.int32)
    for pos in range(0, L, 97):  # a spread of rows filled, the rest all -1
        n = min((pos + 1) // ratio, top_k)
        topk[pos, :n] = rng.choice(max(n, 1), size=n, replace=False)
    W = (top_k + window + 127) // 128 * 128
    ref, rlen = oracle.combine_compressed(topk, None, qsl, seq, seq, L, top_k, ratio, window, M, N, W)
    got, glen = _gpu_combine(dsv4, topk, None, qsl, seq, seq, L, top_k, ratio, window, M, N, W)
    assert np.array_equal(glen, rlen) and np.array_equal(got, ref)


def _caches(rng, P, n_comp_pages, n_swa_pages):
    out = []
    for npg in (n_comp_pages, n_swa_pages):
        c = np.zeros(npg * P * 648, np.uint8)
        n = npg * P
        kv = bf16_normal(rng, (n, 576))
        oracle.kv_insert(np.zeros((n, 0, 576), np.uint16), kv, rng.integers(0, 300, n),
                         np.arange(n, dtype=np.int64), rope_table(300), np.zeros(576, np.uint16),
                         1e-6, c, npg, P, inplace=True)
        out.append(c)
    return out


@pytest.mark.parametrize("P", [32, 64])
def test_gather_workspace_exact(dsv4, P):
    rng = np.random.default_rng(950 + P)
    B, ratio = 3, 4
    seq_lens = np.array([300, 57, 1], np.int32)
    gather_lens = np.array([128, 60, 1], np.int32)  # request 1 asks for more than it has
    N = 80
    M = N + 130
    comp_pages, swa_pages = 6, 16
    comp, swa = _caches(rng, P, comp_pages, swa_pages)
    cbt = rng.permutation(comp_pages)[:B * 2].reshape(B, 2).astype(np.int32)
    sbt = np.full((B, 10), -1, np.int32)
    sp = rng.permutation(swa_pages)
    sbt[0, :10] = sp[:10]
    sbt[1, :2] = sp[10:12]
    sbt[2, :1] = sp[12:13]
    sbt[0, 5] = -1       # a hole
    cbt[1, 1] = 999      # past the compressed cache: zero rows
    ws_pages = (B * M + P - 1) // P + 1
    ws0 = rng.integers(0, 256, size=ws_pages * P * 648, dtype=np.uint8)
    log(f"workspace P={P} B={B} M={M} N={N} pages={ws_pages}")
    ref = oracle.gather_workspace(comp, comp_pages, cbt, swa, swa_pages, sbt, P, seq_lens,
                                  gather_lens, ratio, M, N, ws_pages, ws=ws0)
    ws = dev(ws0)
    dsv4.dsv4_gather_workspace(dev(comp), dev(cbt), dev(swa), dev(sbt), dev(seq_lens),
                               dev(gather_lens), ratio, M, N, ws, page_size=P)
    torch.cuda.synchronize()
    assert np.array_equal(ws.cpu().numpy(), ref)


def test_compressed_prefill_end_to_end(dsv4):
    """Compressed combine -> workspace -> prefill attention on the GPU against the same
    three oracle steps: 2 sequences, ratio 4, H=64, sinks."""
    rng = np.random.default_rng(990)
    P, ratio, top_k, window, H = 64, 4, 128, 64, 64
    seq_lens = np.array([700, 333], np.int32)
    qlens = np.array([40, 25])
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    gather_lens = np.minimum(seq_lens, 160).astype(np.int32)
    N = 256
    M = N + 160
    comp_pages, swa_pages = 8, 24
    comp, swa = _caches(rng, P, comp_pages, swa_pages)
    perm_c, perm_s = rng.permutation(comp_pages), rng.permutation(swa_pages)
    cbt = np.stack([perm_c[0:4], perm_c[4:8]]).astype(np.int32)
    sbt = np.stack([perm_s[0:12], perm_s[12:24]]).astype(np.int32)
    topk = np.full((T, top_k), -1, np.int32)
    for b in range(2):
        for i in range(qlens[b]):
            t = qsl[b] + i
            pos = seq_lens[b] - qlens[b] + i
            n = min((pos + 1) // ratio, top_k)
            topk[t, :n] = rng.choice((pos + 1) // ratio, size=n, replace=False)
    W = (top_k + window + 127) // 128 * 128
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    ws_pages = (2 * M + P - 1) // P
    # oracle chain
    comb_r, lens_r = oracle.combine_compressed(topk, None, qsl, seq_lens, gather_lens, T, top_k,
                                               ratio, window, M, N, W)
    ws_r = oracle.gather_workspace(comp, comp_pages, cbt, swa, swa_pages, sbt, P, seq_lens,
                                   gather_lens, ratio, M, N, ws_pages,
                                   ws=np.zeros(ws_pages * P * 648, np.uint8))
    ref, rlse = oracle.sparse_mla(q, ws_r, ws_pages, P, comb_r, lens_r, sinks, 1 / 24, nthreads=8)
    # library chain
    comb = torch.empty(T, W, dtype=torch.int32, device="cuda")
    lens = torch.empty(T, dtype=torch.int32, device="cuda")
    sl, gl = dev(seq_lens), dev(gather_lens)
    dsv4.dsv4_combine_indices_compressed(dev(topk), None, dev(qsl), sl, gl, top_k, ratio, window,
                                         M, N, comb, lens)
    ws = dsv4.new_cache(ws_pages)
    dsv4.dsv4_gather_workspace(dev(comp), dev(cbt), dev(swa), dev(sbt), sl, gl, ratio, M, N, ws)
    out = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, H, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_prefill(dev_bf16(q), ws, comb, lens, dev(sinks, np.float32), 1 / 24, out,
                                 lse)
    torch.cuda.synchronize()
    assert np.array_equal(comb.cpu().numpy(), comb_r) and np.array_equal(lens.cpu().numpy(), lens_r)
    assert np.array_equal(ws.cpu().numpy(), ws_r)  # both start from zeros
    assert_attention_close(host_bits(out), ref, "compressed prefill")
    assert np.max(np.abs(lse.cpu().numpy() - rlse)) <= 2e-3
