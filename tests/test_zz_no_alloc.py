"""The split decode's entry point that allocates nothing
(dsv4_sparse_mla_decode_split_noalloc: workspace in the library's static per-GPU array),
called through the C ABI: bit-identical to dsv4_sparse_mla_decode_split with a caller
workspace, on two calls in a row, the second with a smaller input (the array keeps the
first call's contents), and within the attention bar of the oracle; a size past the
array's limit is refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
from synth_inputs import bf16_normal
from tests.gpu_helpers import assert_attention_close, dev, dev_bf16, host_bits, log
from tests.test_gpu_attention import P, _random_cache

pytestmark = pytest.mark.gpu


def _case(rng, T, H, stride, num_pages=40):
    cache, slots = _random_cache(rng, num_pages, num_pages * P - 50)
    lens = rng.integers(stride // 2, stride + 1, size=T).astype(np.int32)
    lens[0] = stride
    idx = np.full((T, stride), -1, np.int32)
    for t in range(T):
        row = rng.choice(slots, size=int(lens[t]), replace=True).astype(np.int64)
        row[rng.random(row.size) < 0.05] = -1
        idx[t, :lens[t]] = row
    q = bf16_normal(rng, (T, H, 576))
    sinks = rng.standard_normal(H).astype(np.float32)
    return cache, idx, lens, q, sinks, num_pages


def _both(dsv4, cache_d, idx, lens, q, sinks, splits):
    T, H = q.shape[0], q.shape[1]
    qd, idd, ld, sd = dev_bf16(q), dev(idx, np.int32), dev(lens, np.int32), dev(sinks, np.float32)
    out_n = torch.full((T, H, 512), 5.0, dtype=torch.bfloat16, device="cuda")
    lse_n = torch.full((T, H), 5.0, dtype=torch.float32, device="cuda")
    dsv4.dsv4_sparse_mla_decode_split_noalloc(qd, cache_d, idd, ld, sd, 1 / 24, out_n, splits,
                                              lse=lse_n)
    ws = torch.empty(dsv4.split_workspace_bytes(T, H, splits), dtype=torch.uint8, device="cuda")
    out_w = torch.full_like(out_n, 6.0)
    lse_w = torch.full_like(lse_n, 6.0)
    dsv4.dsv4_sparse_mla_decode_split(qd, cache_d, idd, ld, sd, 1 / 24, out_w, splits, ws,
                                      lse=lse_w)
    torch.cuda.synchronize()
    return out_n, lse_n, out_w, lse_w


def test_noalloc_split_decode_two_calls(dsv4):
    rng = np.random.default_rng(7070)
    lib = dsv4.library()
    # first call: 8 tokens x 4 head groups x 8 pieces (16.8 MB of the 32 MiB array)
    cache, idx, lens, q, sinks, npg = _case(rng, 8, 128, 2176)
    log(f"noalloc call 1: T=8 H=128 splits=8 bytes={dsv4.split_workspace_bytes(8, 128, 8)}")
    cache_d = dev(cache)
    out_n, lse_n, out_w, lse_w = _both(dsv4, cache_d, idx, lens, q, sinks, 8)
    assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
    assert torch.equal(lse_n.view(torch.int32), lse_w.view(torch.int32))
    ref, rlse = oracle.sparse_mla(q, cache, npg, P, idx, lens, sinks, 1 / 24, nthreads=16)
    assert_attention_close(host_bits(out_n), ref, "noalloc call 1")
    assert np.max(np.abs(lse_n.cpu().numpy() - rlse)) <= 1e-4
    # second call, smaller: 3 tokens, 32 heads, 5 pieces of shorter rows
    cache2, idx2, lens2, q2, sinks2, npg2 = _case(rng, 3, 32, 700, num_pages=16)
    log("noalloc call 2: T=3 H=32 splits=5")
    out_n, lse_n, out_w, lse_w = _both(dsv4, dev(cache2), idx2, lens2, q2, sinks2, 5)
    assert torch.equal(out_n.view(torch.int16), out_w.view(torch.int16))
    assert torch.equal(lse_n.view(torch.int32), lse_w.view(torch.int32))
    ref2, rlse2 = oracle.sparse_mla(q2, cache2, npg2, P, idx2, lens2, sinks2, 1 / 24, nthreads=16)
    assert_attention_close(host_bits(out_n), ref2, "noalloc call 2")
    # past the array: refused before any launch, outputs untouched
    T3, H3 = 64, 128
    assert dsv4.split_workspace_bytes(T3, H3, 8) > dsv4.NOALLOC_SCRATCH_BYTES
    q3 = torch.zeros(T3, H3, 576, dtype=torch.bfloat16, device="cuda")
    o3 = torch.full((T3, H3, 512), 2.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsv4.Dsv4Error) as ei:
        dsv4.dsv4_sparse_mla_decode_split_noalloc(
            q3, cache_d, torch.zeros(T3, 64, dtype=torch.int32, device="cuda"),
            torch.zeros(T3, dtype=torch.int32, device="cuda"), None, 1 / 24, o3, 8)
    assert ei.value.status == 5 and "static scratch" in ei.value.reason
    torch.cuda.synchronize()
    assert torch.all(o3 == 2.0)
