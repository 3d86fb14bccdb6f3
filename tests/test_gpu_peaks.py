"""The measurement probes behind the roofline's measured peaks do the work they count:
every MFMA's result reaches the sink (exact closed form, independent of the lane
layout), the read probe's per-thread xor equals the xor of the units that thread owns,
and the copy probe copies."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,start,per_iter,per_call", [(0, 448.0, 144.0, 2 * 32 * 32 * 16),
                                                          (1, 112.0, 72.0, 2 * 16 * 16 * 32)])
def test_peak_mfma_closed_form(dsv4, shape, start, per_iter, per_call):
    wg, iters = 5, 37
    sink = torch.full((wg * 256,), -1.0, dtype=torch.float32, device="cuda")
    flops = dsv4.dsv4_peak_mfma(shape, iters, sink)
    torch.cuda.synchronize()
    assert flops == per_call * 8 * iters * 4 * wg
    # accumulator k starts at k: sum over 8 chains of (elements x k) + iters x per-step growth
    assert torch.all(sink == start + per_iter * iters).item()


@pytest.mark.parametrize("n16,wg", [(0, 3), (1, 1), (4096 * 3 + 5, 7), (1 << 16, 64)])
def test_peak_stream_read_and_copy(dsv4, n16, wg):
    rng = np.random.default_rng(n16 + wg)
    host = rng.integers(0, 2 ** 32, size=max(n16, 1) * 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    src_view = src[: n16 * 4]
    sink = torch.full((wg * 256,), 7, dtype=torch.int32, device="cuda")
    dsv4.dsv4_peak_stream(src_view, sink)
    torch.cuda.synchronize()
    # thread j owns units j, j + stride, ...; its value is the xor of their 4 words
    stride = wg * 256
    unit = np.bitwise_xor.reduce(host[: n16 * 4].reshape(n16, 4), axis=1) if n16 else np.zeros(0, np.uint32)
    pad = np.zeros((-n16) % stride, np.uint32)
    want = np.bitwise_xor.reduce(np.concatenate([unit, pad]).reshape(-1, stride), axis=0) \
        if n16 else np.zeros(stride, np.uint32)
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), want)
    dst = torch.full_like(src, -3)
    dsv4.dsv4_peak_stream(src_view, sink, dst=dst)
    torch.cuda.synchronize()
    assert torch.equal(dst[: n16 * 4], src_view)
    if n16 == 0:
        assert torch.all(dst == -3).item()
