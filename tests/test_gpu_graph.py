"""One decode step (insert + combine + decode) captured into a HIP graph, as the
benchmark replays it: every replay must reproduce the eager step bit for bit (the
kernels are deterministic and allocate nothing), with eager work and synchronisations
between the replays."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, dev_bf16, log
from synth_inputs import attention_workload, bf16_normal

pytestmark = pytest.mark.gpu


def test_step_graph_replays_match_eager(dsv4):
    wl = attention_workload(2, seed=5, instances=1)
    it = wl["instances"][0]
    T, H, W, npg = wl["T"], wl["H"], wl["W"], wl["num_pages"]
    log(f"graph: T={T} H={H} W={W} pages={npg}")
    cache = dsv4.new_cache(npg)
    cos_sin = dev(wl["cos_sin"], np.float32)
    weight = dev_bf16(wl["q_norm_weight"])
    dsv4.dsv4_kv_insert(None, dev_bf16(wl["ctx_kv"]), dev(wl["ctx_pos"], np.int64),
                        dev(wl["ctx_slot"], np.int64), cos_sin, None, wl["eps"], cache)
    pos = wl["seq_lens"].astype(np.int64) - 1
    slots = wl["block_table"][np.arange(T), pos // 64].astype(np.int64) * 64 + pos % 64
    positions, slot_mapping = dev(pos, np.int64), dev(slots, np.int64)
    q0 = dev_bf16(it["q"])
    kv_new = dev_bf16(bf16_normal(np.random.default_rng(7), (T, 576)))
    topk, topk_lens = dev(it["topk"], np.int32), dev(it["topk_lens"], np.int32)
    qsl, seq_lens, bt = dev(wl["qsl"], np.int32), dev(wl["seq_lens"], np.int32), dev(wl["block_table"], np.int32)
    sinks = dev(it["sinks"], np.float32)

    def step(q, comb, clen, out):
        dsv4.dsv4_kv_insert(q, kv_new, positions, slot_mapping, cos_sin, weight, wl["eps"], cache)
        dsv4.dsv4_combine_indices(topk, topk_lens, qsl, seq_lens, bt, wl["top_k"], wl["window"], comb, clen)
        dsv4.dsv4_sparse_mla_decode(q, cache, comb, clen, sinks, wl["softmax_scale"], out)

    def buffers():
        return (q0.clone(), torch.empty(T, W, dtype=torch.int32, device="cuda"),
                torch.empty(T, dtype=torch.int32, device="cuda"),
                torch.empty(T, H, 512, dtype=torch.bfloat16, device="cuda"))

    ref = buffers()
    step(*ref)
    torch.cuda.synchronize()

    gbuf = buffers()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        step(*gbuf)
    torch.cuda.synchronize()
    x = torch.randn(512, 512, device="cuda")
    for r in range(3):
        gbuf[0].copy_(q0)
        torch.cuda.synchronize()
        y = x @ x  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(y).all()
        for name, a, b in zip(("q", "combined", "lens", "out"), gbuf, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), (r, name)
        log(f"graph replay {r}: q, combined, lens, out bit-identical to the eager step")
