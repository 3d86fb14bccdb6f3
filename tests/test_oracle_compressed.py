"""Pins of the oracle's compressed-cache form of the combine and of the workspace it
addresses (PR #43385, Key source excerpts: the combine kernel with COMPRESS_RATIO, M, N
and gather_lens): a hand-worked example, the link to the plain combine at ratio 1, the
transparency of the workspace (attention through it equals attention over the directly
mapped slots), and the zero rows."""
import os

import numpy as np

import oracle
from synth_inputs import bf16_normal, rope_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "combine_compressed_worked.txt")


def _load_golden():
    d = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split(":", 1)
        d[k.strip()] = np.array([int(x) for x in v.split()], np.int64)
    return d


def test_combine_compressed_worked_example():
    g = _load_golden()
    topk = np.stack([g["topk_t0"], g["topk_t1"], g["topk_t2"]]).astype(np.int32)
    out, lens = oracle.combine_compressed(topk, None, g["qsl"], g["seq_lens"], g["gather_lens"], 3,
                                          int(g["top_k"][0]), int(g["ratio"][0]),
                                          int(g["window"][0]), int(g["M"][0]), int(g["N"][0]),
                                          int(g["stride"][0]))
    assert np.array_equal(out, np.stack([g["expect_t0"], g["expect_t1"], g["expect_t2"]]))
    assert np.array_equal(lens, g["expect_lens"])


def test_combine_compressed_ratio_one_matches_plain_combine():
    """Ratio 1, one request, identity page table, every raw token gathered, top-k entries
    causal and outside the window: the plain combine gives x for a top-k entry x and for a
    window position; the compressed form gives x and N + x (the window rows follow the N
    compressed rows)."""
    rng = np.random.default_rng(3)
    P, L, qlen, top_k, window = 64, 700, 3, 50, 32
    N = 1024
    M = N + L
    seq_lens = np.array([L], np.int32)
    qsl = np.array([0, qlen], np.int32)
    bt = np.arange((L + P - 1) // P, dtype=np.int32)[None, :]
    topk = np.full((qlen, top_k), -1, np.int32)
    for i in range(qlen):
        pos = L - qlen + i
        lo = pos - window + 1
        topk[i] = rng.choice(lo, size=top_k, replace=False)
    W = 128
    plain, plens = oracle.combine(topk, None, qsl, seq_lens, bt, qlen, top_k, window, P, W)
    comp, clens = oracle.combine_compressed(topk, None, qsl, seq_lens, seq_lens, qlen, top_k, 1,
                                            window, M, N, W)
    assert np.array_equal(plens, clens)
    assert np.array_equal(comp[:, :top_k], plain[:, :top_k])
    assert np.array_equal(comp[:, top_k:top_k + window], plain[:, top_k:top_k + window] + N)
    assert np.all(comp[:, top_k + window:] == -1) and np.all(plain[:, top_k + window:] == -1)


def test_combine_compressed_special_cases():
    qsl = np.array([0, 1], np.int32)
    seq = np.array([40], np.int32)
    topk = np.arange(16, dtype=np.int32)[None, :]
    # window 0: only the top-k part, (pos + 1) // ratio = 40 // 8 = 5 entries
    out, lens = oracle.combine_compressed(topk, None, qsl, seq, seq, 1, 16, 8, 0, 100, 50, 32)
    assert lens[0] == 5 and np.array_equal(out[0, :5], np.arange(5)) and np.all(out[0, 5:] == -1)
    # top_k 0: only the window, ascending, right after the N compressed rows
    out, lens = oracle.combine_compressed(topk, None, qsl, seq, seq, 1, 0, 8, 6, 100, 50, 32)
    assert lens[0] == 6 and np.array_equal(out[0, :6], 50 + np.arange(34, 40))
    # window positions before the gathered tokens are -1; topk_lens caps the top-k part
    gl = np.array([3], np.int32)
    out, lens = oracle.combine_compressed(topk, np.array([2], np.int32), qsl, seq, gl, 1, 16, 8,
                                          6, 100, 50, 32)
    assert lens[0] == 8
    assert np.array_equal(out[0, :8], [0, 1, -1, -1, -1, 50, 51, 52])
    # a sequence shorter than the ratio has no compressed entry yet
    out, lens = oracle.combine_compressed(topk, None, qsl, np.array([3], np.int32),
                                          np.array([3], np.int32), 1, 16, 4, 8, 100, 50, 32)
    assert lens[0] == 3 and np.array_equal(out[0, :3], [50, 51, 52])


def _pool(rng, P, num_pages, n):
    cache = np.zeros(num_pages * P * 648, np.uint8)
    slots = rng.choice(num_pages * P, size=n, replace=False).astype(np.int64)
    kv = bf16_normal(rng, (n, 576))
    _, cache = oracle.kv_insert(np.zeros((n, 0, 576), np.uint16), kv, rng.integers(0, 500, n), slots,
                                rope_table(500), np.zeros(576, np.uint16), 1e-6, cache, num_pages, P)
    return cache


def _setup(rng, P=32):
    """Two requests over one page pool: compressed entries and raw tokens each through a
    block table of their own."""
    ratio, N = 4, 48
    seq_lens = np.array([150, 97], np.int32)
    gather_lens = np.array([40, 97], np.int32)
    M = N + 100
    num_pages = 24
    pool = _pool(rng, P, num_pages, num_pages * P)
    perm = rng.permutation(num_pages)
    comp_bt = np.stack([perm[0:2], perm[2:4]]).astype(np.int32)      # 64 compressed entries each
    swa_bt = np.stack([perm[4:9], perm[9:14]]).astype(np.int32)      # 160 raw positions each
    swa_bt[1, 2] = -1                                                # a hole in the table
    return dict(P=P, ratio=ratio, N=N, M=M, seq_lens=seq_lens, gather_lens=gather_lens,
                pool=pool, num_pages=num_pages, comp_bt=comp_bt, swa_bt=swa_bt)


def test_workspace_rows():
    rng = np.random.default_rng(8)
    s = _setup(rng)
    P, M, N = s["P"], s["M"], s["N"]
    ws_pages = (2 * M + P - 1) // P
    ws = oracle.gather_workspace(s["pool"], s["num_pages"], s["comp_bt"], s["pool"],
                                 s["num_pages"], s["swa_bt"], P, s["seq_lens"], s["gather_lens"],
                                 s["ratio"], M, N, ws_pages)
    got = oracle.gather_dequant(ws, ws_pages, P, np.arange(2 * M, dtype=np.int32))
    for b in range(2):
        L, gl = int(s["seq_lens"][b]), int(s["gather_lens"][b])
        src = np.full(M, -1, np.int64)
        for e in range(min(N, L // s["ratio"])):
            src[e] = s["comp_bt"][b, e // P] * P + e % P
        for k in range(gl):
            x = L - gl + k
            pg = s["swa_bt"][b, x // P]
            src[N + k] = pg * P + x % P if pg >= 0 else -1
        want = oracle.gather_dequant(s["pool"], s["num_pages"], P, src.astype(np.int32))
        assert np.array_equal(got[b * M:(b + 1) * M], want), b
        # rows with no source are zero records
        assert np.all(got[b * M:(b + 1) * M][src < 0] == 0)
    # request 0 has 150 // 4 = 37 compressed entries: rows 37..47 are zero
    assert np.all(got[37:48] == 0) and np.any(got[36] != 0)


def test_workspace_is_transparent_to_attention():
    """Attention over the workspace with the compressed-form indices equals, bit for bit,
    attention over the page pool with each index mapped straight to its physical slot."""
    rng = np.random.default_rng(9)
    s = _setup(rng)
    P, M, N, ratio = s["P"], s["M"], s["N"], s["ratio"]
    top_k, window = 24, 16
    qlens = np.array([3, 2])
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    topk = rng.integers(-2, N + 4, size=(T, top_k)).astype(np.int32)
    W = 128
    comb, lens = oracle.combine_compressed(topk, None, qsl, s["seq_lens"], s["gather_lens"], T,
                                           top_k, ratio, window, M, N, W)
    ws_pages = (2 * M + P - 1) // P
    ws = oracle.gather_workspace(s["pool"], s["num_pages"], s["comp_bt"], s["pool"],
                                 s["num_pages"], s["swa_bt"], P, s["seq_lens"], s["gather_lens"],
                                 ratio, M, N, ws_pages)
    # the same rows mapped straight into the pool (-1 where the workspace row is zero)
    direct = np.full_like(comb, -1)
    for t in range(T):
        for j in range(int(lens[t])):
            x = int(comb[t, j])
            if x < 0:
                continue
            b, e = divmod(x, M)
            L, gl = int(s["seq_lens"][b]), int(s["gather_lens"][b])
            if e < N:
                if e < L // ratio:
                    direct[t, j] = s["comp_bt"][b, e // P] * P + e % P
            else:
                pos = L - gl + (e - N)
                pg = s["swa_bt"][b, pos // P]
                direct[t, j] = pg * P + pos % P if pg >= 0 else -1
    H = 16
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    a, la = oracle.sparse_mla(q, ws, ws_pages, P, comb, lens, sinks, 1 / 24)
    # a zero row of the workspace is still a key (score 0, value 0): map it to a zero
    # record in an extra page of the pool rather than to -1, which would drop it
    zero_slot = np.int64(s["num_pages"] * P)
    pool = np.concatenate([s["pool"], np.zeros(P * 648, np.uint8)])
    direct[(direct < 0) & (comb >= 0)] = zero_slot
    b_, lb = oracle.sparse_mla(q, pool, s["num_pages"] + 1, P, direct, lens, sinks, 1 / 24)
    assert np.array_equal(a, b_) and np.array_equal(la, lb)
