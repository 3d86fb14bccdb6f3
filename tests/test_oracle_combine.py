"""Pins of the oracle's index-combining step by brute force on tiny inputs.

The reference formulation here is a set model, written independently of the oracle's
positional rules: the slots a query attends are (valid top-k  UNION  window), each once,
where valid means 0 <= x <= pos; the row has length tk + sw, the window part lists the
last sw positions in ascending order, and everything past the length is -1.
Special case: with window 0 the step reduces to the plain per-request logical ->
physical conversion through the block table (PR #43477 digest, forward_mqa excerpt).
"""
import numpy as np
import pytest

P = 64


def _case(rng, B, top_k, window, width, with_lens, dup=False, P=P):
    qlens = rng.integers(1, 5, size=B)
    seq_lens = np.array([int(rng.integers(ql, 300)) for ql in qlens], np.int32)
    qsl = np.zeros(B + 1, np.int32)
    qsl[1:] = np.cumsum(qlens)
    base = int(rng.integers(0, 3))
    qsl = qsl + base  # a non-zero query_start_loc[0] is subtracted by the step
    T = int(qsl[-1] - qsl[0])
    pages = [int(np.ceil(L / P)) for L in seq_lens]
    perm = rng.permutation(sum(pages) + 5)
    bt = np.full((B, max(pages) + int(rng.integers(0, 2))), -1, np.int32)
    o = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[o:o + n]
        o += n
    topk = np.full((T, width), -1, np.int32)
    for t in range(T):
        n = int(rng.integers(0, width + 1))
        vals = rng.integers(-3, 320, size=n)
        if not dup:
            vals = np.unique(vals)
            rng.shuffle(vals)
        topk[t, :len(vals)] = vals
    lens = rng.integers(0, top_k + 2, size=T).astype(np.int32) if with_lens else None
    return qsl, seq_lens, bt, topk, lens, T


def _phys(bt, b, x, P=P):
    if x < 0 or x // P >= bt.shape[1] or bt[b, x // P] < 0:
        return -1
    return int(bt[b, x // P]) * P + x % P


@pytest.mark.parametrize("seed", range(12))
def test_combine_set_model(orc, seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 5))
    top_k = int(rng.choice([4, 16, 64]))
    window = int(rng.choice([0, 1, 4, 16]))
    width = top_k + int(rng.integers(0, 3))
    qsl, seq_lens, bt, topk, tl, T = _case(rng, B, top_k, window, width, with_lens=bool(seed % 2))
    W = (top_k + window + 127) // 128 * 128
    out, lens = orc.combine(topk, tl, qsl, seq_lens, bt, T, top_k, window, P, W)
    for b in range(B):
        qlen = qsl[b + 1] - qsl[b]
        for i in range(qlen):
            t = qsl[b] - qsl[0] + i
            pos = int(seq_lens[b] - qlen + i)
            tk = min(pos + 1, top_k) if tl is None else min(pos + 1, top_k, int(tl[t]))
            tk = max(tk, 0)
            sw = max(min(pos + 1, window), 0)
            row = out[t]
            assert lens[t] == tk + sw
            assert np.all(row[tk + sw:] == -1)
            win = list(range(pos - sw + 1, pos + 1))
            assert list(row[tk:tk + sw]) == [_phys(bt, b, x) for x in win]
            valid_topk = {int(x) for x in topk[t, :tk] if 0 <= x <= pos}
            expect = {_phys(bt, b, x) for x in valid_topk | set(win)}
            got = [int(v) for v in row[:tk + sw] if v >= 0]
            assert set(got) == expect - {-1}
            assert len(got) == len(set(got))  # each attended slot once (distinct top-k)


@pytest.mark.parametrize("seed", range(4))
def test_combine_window0_is_block_table_conversion(orc, seed):
    rng = np.random.default_rng(100 + seed)
    B, top_k = 3, 32
    qsl, seq_lens, bt, topk, tl, T = _case(rng, B, top_k, 0, top_k, with_lens=True)
    out, lens = orc.combine(topk, tl, qsl, seq_lens, bt, T, top_k, 0, P, 128)
    for b in range(B):
        qlen = qsl[b + 1] - qsl[b]
        for i in range(qlen):
            t = qsl[b] - qsl[0] + i
            pos = int(seq_lens[b] - qlen + i)
            n = max(0, min(pos + 1, top_k, int(tl[t])))
            x = topk[t, :n].astype(np.int64)
            ok = (x >= 0) & (x <= pos)
            page = np.where(ok, bt[b][np.clip(x // P, 0, bt.shape[1] - 1)], -1)
            conv = np.where(ok & (page >= 0), page.astype(np.int64) * P + x % P, -1)
            assert np.array_equal(out[t, :n], conv)
            assert lens[t] == n


def test_combine_width_and_duplicates(orc):
    rng = np.random.default_rng(7)
    # entries beyond topk_width read as -1; duplicated top-k entries are kept as given
    qsl = np.array([0, 1], np.int32)
    seq_lens = np.array([100], np.int32)
    bt = np.arange(2, dtype=np.int32)[None, :]
    topk = np.array([[5, 5, 7, 99, 60, 61]], np.int32)
    out, lens = orc.combine(topk, None, qsl, seq_lens, bt, 1, 6, 4, P, 128, topk_width=4)
    assert lens[0] == 10
    assert list(out[0, :10]) == [5, 5, 7, -1, -1, -1, 96, 97, 98, 99]
    assert np.all(out[0, 10:] == -1)


def test_combine_rows_of_unowned_tokens_untouched(orc):
    qsl = np.array([0, 1], np.int32)
    seq_lens = np.array([10], np.int32)
    bt = np.zeros((1, 1), np.int32)
    topk = np.full((3, 4), -1, np.int32)
    out, lens = orc.combine(topk, None, qsl, seq_lens, bt, 3, 4, 0, P, 128, fill=-7)
    assert lens[0] == 4 and np.all(out[1:] == -7) and np.all(lens[1:] == -7)
