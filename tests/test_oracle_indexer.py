"""Pins of the oracle's indexer top-k selection: the result equals the first top_k ids of
numpy's stable argsort by descending logit (ties to the smaller id), listed ascending;
every picked logit is >= every unpicked one; the candidate range is causal
((pos+1) // ratio ids, capped by the row width); short rows give every candidate."""
import numpy as np
import pytest

import oracle


def _numpy_topk(row, n, k):
    v = np.where(np.isnan(row[:n]), -np.inf, row[:n]).astype(np.float64)
    order = np.argsort(-v, kind="stable")  # stable: equal logits keep ascending ids
    return np.sort(order[:k])


@pytest.mark.parametrize("ratio", [1, 4, 128])
def test_indexer_topk_matches_stable_argsort(ratio):
    rng = np.random.default_rng(40 + ratio)
    B = 4
    qlens = np.array([1, 5, 2, 3])
    seq_lens = np.array([3000, 900, 40, 2500], np.int32)
    qsl = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(qsl[-1])
    width = 2600
    top_k = 300
    # coarse logits so that ties are common, plus NaN and infinities
    logits = rng.integers(-20, 20, size=(T, width)).astype(np.float32) / 4
    logits[rng.random((T, width)) < 0.01] = np.nan
    logits[rng.random((T, width)) < 0.01] = -np.inf
    logits[rng.random((T, width)) < 0.002] = np.inf
    out, lens = oracle.indexer_topk(logits, qsl, seq_lens, T, ratio, top_k, top_k + 7)
    for b in range(B):
        for i in range(qlens[b]):
            t = qsl[b] + i
            pos = seq_lens[b] - qlens[b] + i
            n = min((pos + 1) // ratio, width)
            k = min(n, top_k)
            want = _numpy_topk(logits[t], n, k)
            assert lens[t] == k
            assert np.array_equal(out[t, :k], want)
            assert np.all(out[t, k:] == -1)
            # picked logits dominate the unpicked ones
            v = np.where(np.isnan(logits[t, :n]), -np.inf, logits[t, :n])
            picked = np.zeros(n, bool)
            picked[out[t, :k]] = True
            if k and k < n:
                assert v[picked].min() >= v[~picked].max()


def test_indexer_topk_short_rows_and_ratio():
    qsl = np.array([0, 1, 2], np.int32)
    seq_lens = np.array([10, 8000], np.int32)
    logits = np.random.default_rng(1).standard_normal((2, 4000)).astype(np.float32)
    out, lens = oracle.indexer_topk(logits, qsl, seq_lens, 2, 4, 2048, 2048)
    # token 0: (9+1)//4 = 2 candidates -> both; token 1: 8000//4 = 2000 < 2048 -> all
    assert lens[0] == 2 and np.array_equal(out[0, :2], [0, 1]) and np.all(out[0, 2:] == -1)
    assert lens[1] == 2000 and np.array_equal(out[1, :2000], np.arange(2000))
    # the row width caps the candidates: 8000 positions but only 4000 logits
    out, lens = oracle.indexer_topk(logits, qsl, seq_lens, 2, 1, 3000, 3000)
    assert lens[1] == 3000 and out[1, :3000].max() < 4000
