"""GPU parity of the split-slot decode (each token's row cut into pieces whose partial
results are merged by their lse) against the fp64 oracle, with the same bar as the
unsplit decode: ragged rows whose pieces are partly or wholly empty, -1 holes,
out-of-range and duplicated slots, empty and all-invalid rows, sinks on/off, several
split counts, a small batch of the benchmark workload at full row length, and one
workspace reused by consecutive calls of different shapes."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import attention_workload, bf16_normal
from tests.gpu_helpers import assert_attention_close, dev, dev_bf16, host_bits, log, oracle_cache
from tests.test_gpu_attention import P, _random_cache

pytestmark = pytest.mark.gpu


def run_split(dsv4, q_bits, cache_dev, idx, lens, sinks, scale, splits, workspace=None, guard=2):
    T, H = q_bits.shape[0], q_bits.shape[1]
    out_full = torch.full((T + guard, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_full = torch.full((T + guard, H), 7.0, dtype=torch.float32, device="cuda")
    out, lse = out_full[:T], lse_full[:T]
    if workspace is None:
        workspace = torch.empty(max(dsv4.split_workspace_bytes(T, H, splits), 16),
                                dtype=torch.uint8, device="cuda")
    dsv4.dsv4_sparse_mla_decode_split(dev_bf16(q_bits), cache_dev, dev(idx, np.int32),
                                      dev(lens, np.int32),
                                      None if sinks is None else dev(sinks, np.float32), scale, out,
                                      splits, workspace, lse)
    torch.cuda.synchronize()
    assert torch.all(out_full[T:] == 7.0) and torch.all(lse_full[T:] == 7.0), "guard rows written"
    return host_bits(out), lse.cpu().numpy()


def check_split(dsv4, name, q, cache, num_pages, idx, lens, sinks, scale, splits, workspace=None):
    log(f"split case {name}: T={q.shape[0]} H={q.shape[1]} stride={idx.shape[1]} splits={splits}")
    ref, rlse = oracle.sparse_mla(q, cache, num_pages, P, idx, lens, sinks, scale, nthreads=8)
    got, glse = run_split(dsv4, q, dev(cache), idx, lens, sinks, scale, splits, workspace)
    assert_attention_close(got, ref, name)
    fin = np.isfinite(rlse)
    assert np.array_equal(fin, np.isfinite(glse)), name
    assert np.all(np.isneginf(glse[~fin]))
    if fin.any():
        assert np.max(np.abs(glse[fin] - rlse[fin])) <= 2e-3, name


@pytest.mark.parametrize("H", [16, 128])
@pytest.mark.parametrize("splits", [2, 5, 8])
@pytest.mark.parametrize("sinks_on", [False, True])
def test_split_small_ragged(dsv4, H, splits, sinks_on):
    rng = np.random.default_rng(1000 + 10 * H + splits + 3 * sinks_on)
    num_pages = 12
    cache, slots = _random_cache(rng, num_pages, 700)
    lens_list = [0, 1, 63, 65, 200, 333, 600]
    T = len(lens_list)
    stride = 640
    idx = np.full((T, stride), 999999, np.int32)  # garbage past each length
    for t, L in enumerate(lens_list):
        row = rng.choice(slots, size=L, replace=True).astype(np.int64)
        row[rng.random(L) < 0.1] = -1
        oor = rng.random(L) < 0.03
        row[oor] = num_pages * P + rng.integers(0, 100, oor.sum())
        idx[t, :L] = row
    idx[1, :] = -1  # an all-invalid row
    lens = np.array(lens_list, np.int32)
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32) if sinks_on else None
    check_split(dsv4, f"H={H} sinks={sinks_on}", q, cache, num_pages, idx, lens, sinks, 1.0 / 24, splits)


def test_split_small_batch_of_benchmark_workload(dsv4):
    wl = attention_workload(2)
    it = wl["instances"][0]
    B = 8
    cache = oracle_cache(wl)
    idx, lens = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                               wl["block_table"], wl["T"], wl["top_k"], wl["window"], P, wl["W"])
    check_split(dsv4, "cfg2 rows 0..7", it["q"][:B], cache, wl["num_pages"], idx[:B], lens[:B],
                it["sinks"], wl["softmax_scale"], 8)


def test_split_workspace_reuse_and_unsplit_agreement(dsv4):
    rng = np.random.default_rng(77)
    cache, slots = _random_cache(rng, 8, 500)
    big = dsv4.split_workspace_bytes(6, 128, 8)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    for T, H, splits in ((6, 128, 8), (3, 16, 3), (2, 64, 4)):
        stride = 448
        idx = rng.choice(slots, size=(T, stride)).astype(np.int32)
        lens = rng.integers(1, stride + 1, T).astype(np.int32)
        q = bf16_normal(rng, (T, H, 576))
        check_split(dsv4, f"reuse T={T} H={H}", q, cache, 8, idx, lens, None, 0.05, splits,
                    workspace=ws)
        # agreement with the unsplit decode (different rounding order only)
        got_s, _ = run_split(dsv4, q, dev(cache), idx, lens, None, 0.05, splits, workspace=ws)
        out = torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda")
        dsv4.dsv4_sparse_mla_decode(dev_bf16(q), dev(cache), dev(idx, np.int32), dev(lens, np.int32),
                                    None, 0.05, out)
        torch.cuda.synchronize()
        a = (host_bits(out).astype(np.uint32) << 16).view(np.float32)
        b = (got_s.astype(np.uint32) << 16).view(np.float32)
        assert np.max(np.abs(a - b)) <= 2e-2 * max(1.0, float(np.abs(a).max()))
