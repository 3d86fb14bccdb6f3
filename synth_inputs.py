"""Seeded synthetic inputs for the sparse MLA hot path (shared by tests, smoke and bench).

This module only draws random numbers and lays them out.  It computes none of the
method's steps: no index combining, no quantisation, no normalisation, no attention.
The cache contents are produced later by an insert step (the CPU oracle in tests, the
HIP library in the benchmark) from the raw latent rows drawn here.

Workloads (sizes from the benchmark configurations of this project):
  0 tiny decode    B=2, contexts 256 and 200, 1 query each, H=16, top-k 64 (lens 64/50),
                   no window (window 0), no sinks, pages in a seeded random order.
  1 insert         4096 new tokens across 32 requests, H=128, 2048-page cache, distinct
                   random slots, random positions < 131072, weight ~ N(1, 0.1).
  2 decode         B=64, context 32768, H=128, top-k 2048 with lens ~ U{1024..2048},
                   window 128 (row width 2176), sinks ~ N(0,1).
  3 MTP decode     256 requests x 2 query tokens, contexts ~ U{8192..131072}, H=128,
                   top-k 2048 causal per token, window 128, no sinks.
  4 prefill        one sequence of 8192 query tokens, H=64, top-k min(pos+1, 2048) causal,
                   window 128, sinks ~ N(0,1).
Random streams: numpy PCG64 seeded from SeedSequence(seed).spawn(9) in the fixed order
q, kv, topk, topk_lens, sinks, page permutation, positions, slots, weight.
bf16 values are fp32 standard normals rounded to bf16 by torch (round to nearest even).
"""
from __future__ import annotations

import math

import numpy as np

LATENT, NOPE, ROPE = 576, 512, 64
PAGE = 64
ALIGN = 128


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp32 values rounded to bf16 (torch's RNE conversion)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_normal(rng: np.random.Generator, shape, mean=0.0, std=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return bf16_bits(x)


def rope_table(max_pos: int, theta: float = 10000.0) -> np.ndarray:
    """Caller-supplied GPT-J RoPE table, fp32 [max_pos, 64] = cos[32] | sin[32] with
    angle p * theta^(-2i/64), evaluated in fp64 (an input of the insert entry point)."""
    p = np.arange(max_pos, dtype=np.float64)[:, None]
    inv = theta ** (-np.arange(0, ROPE, 2, dtype=np.float64) / ROPE)[None, :]
    ang = p * inv
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def round_up(x: int, a: int) -> int:
    return (x + a - 1) // a * a


def _streams(seed: int):
    ss = np.random.SeedSequence(seed).spawn(9)
    names = ["q", "kv", "topk", "topk_lens", "sinks", "perm", "pos", "slots", "weight"]
    return {n: np.random.Generator(np.random.PCG64(s)) for n, s in zip(names, ss)}


def _distinct(rng, hi: int, k: int) -> np.ndarray:
    """k distinct uniform integers in [0, hi), unsorted."""
    if k <= 0:
        return np.zeros(0, np.int64)
    if 4 * k >= hi:
        return rng.permutation(hi)[:k]
    out = np.unique(rng.integers(0, hi, size=2 * k))
    while out.size < k:
        out = np.unique(np.concatenate([out, rng.integers(0, hi, size=k)]))
    return rng.permutation(out)[:k]


def _block_table(rng, seq_lens, P=PAGE):
    """Per-request logical pages mapped onto one global seeded random permutation."""
    pages_per = [int(math.ceil(L / P)) for L in seq_lens]
    total = int(sum(pages_per))
    perm = rng.permutation(total).astype(np.int32)
    width = max(pages_per) if pages_per else 1
    bt = np.full((len(seq_lens), width), -1, np.int32)
    o = 0
    for b, n in enumerate(pages_per):
        bt[b, :n] = perm[o:o + n]
        o += n
    return bt, total


def attention_workload(cfg: int, seed: int | None = None, instances: int = 1,
                       context_kv: str = "referenced", ctx_tokens=None, page_size: int = PAGE):
    """Inputs of the combine + attention steps for configs 0, 2, 3, 4.

    Returns a dict.  ``instances`` > 1 draws independent (q, topk, topk_lens, sinks)
    sets over the same cache geometry (used to rotate the benchmark's working set).
    ``ctx_*`` describe the context tokens whose latent rows must be inserted into the
    cache before attention: every position a top-k row or a window may touch
    ("referenced"), or every context position ("all").  ``ctx_tokens`` restricts the
    referenced set to the rows of those query tokens (sampled parity checks).
    ``page_size`` sets the slots per cache page (and so the block table)."""
    seed = cfg if seed is None else seed
    r = _streams(seed)
    if cfg == 0:
        B, H, top_k, window = 2, 16, 64, 0
        seq_lens = np.array([256, 200], np.int32)
        qlens = np.array([1, 1], np.int32)
        sinks_on = False
    elif cfg == 2:
        B, H, top_k, window = 64, 128, 2048, 128
        seq_lens = np.full(B, 32768, np.int32)
        qlens = np.ones(B, np.int32)
        sinks_on = True
    elif cfg == 3:
        B, H, top_k, window = 256, 128, 2048, 128
        seq_lens = r["pos"].integers(8192, 131072 + 1, size=B).astype(np.int32)
        qlens = np.full(B, 2, np.int32)
        sinks_on = False
    elif cfg == 4:
        B, H, top_k, window = 1, 64, 2048, 128
        seq_lens = np.array([8192], np.int32)
        qlens = np.array([8192], np.int32)
        sinks_on = True
    else:
        raise ValueError(f"no attention workload {cfg}")
    qsl = np.zeros(B + 1, np.int32)
    qsl[1:] = np.cumsum(qlens)
    T = int(qsl[-1])
    block_table, num_pages = _block_table(r["perm"], seq_lens, page_size)
    W = round_up(top_k + window, ALIGN)

    inst = []
    for _ in range(instances):
        topk = np.full((T, top_k), -1, np.int32)
        topk_lens = None
        if cfg == 0:
            topk_lens = np.array([64, 50], np.int32)
            for b in range(B):
                n = int(topk_lens[b])
                topk[b, :n] = _distinct(r["topk"], int(seq_lens[b]), n)
        elif cfg == 2:
            topk_lens = r["topk_lens"].integers(1024, 2048 + 1, size=T).astype(np.int32)
            for t in range(T):
                n = int(topk_lens[t])
                topk[t, :n] = _distinct(r["topk"], int(seq_lens[0]), n)
        else:
            for b in range(B):
                for i in range(int(qlens[b])):
                    t = int(qsl[b]) + i
                    pos = int(seq_lens[b]) - int(qlens[b]) + i
                    n = min(pos + 1, top_k)
                    topk[t, :n] = _distinct(r["topk"], pos + 1, n)
        q = bf16_normal(r["q"], (T, H, LATENT))
        sinks = r["sinks"].standard_normal(H).astype(np.float32) if sinks_on else None
        inst.append(dict(q=q, topk=topk, topk_lens=topk_lens, sinks=sinks))

    # context tokens whose latent rows the cache must hold
    ctx_b, ctx_x = [], []
    for b in range(B):
        L = int(seq_lens[b])
        if context_kv == "all" or cfg in (0, 4):
            xs = np.arange(L, dtype=np.int64)
        else:
            parts = [np.zeros(0, np.int64)]
            t0, t1 = int(qsl[b]), int(qsl[b + 1])
            toks = np.arange(t0, t1)
            if ctx_tokens is not None:
                toks = np.intersect1d(toks, np.asarray(ctx_tokens))
            for t in toks:
                pos = L - int(qlens[b]) + (int(t) - t0)
                for it in inst:
                    row = it["topk"][t]
                    parts.append(row[(row >= 0) & (row <= pos)].astype(np.int64))
                parts.append(np.arange(max(0, pos - window + 1), pos + 1, dtype=np.int64))
            xs = np.unique(np.concatenate(parts))
        ctx_b.append(np.full(xs.size, b, np.int64))
        ctx_x.append(xs)
    ctx_b = np.concatenate(ctx_b)
    ctx_x = np.concatenate(ctx_x)
    ctx_slot = (block_table[ctx_b, ctx_x // page_size].astype(np.int64) * page_size +
                ctx_x % page_size)
    ctx_kv = bf16_normal(r["kv"], (ctx_x.size, LATENT))
    max_pos = int(seq_lens.max())
    return dict(cfg=cfg, B=B, H=H, T=T, top_k=top_k, window=window, W=W, page_size=page_size,
                softmax_scale=1.0 / math.sqrt(LATENT), seq_lens=seq_lens, qsl=qsl,
                block_table=block_table, num_pages=num_pages, instances=inst,
                ctx_kv=ctx_kv, ctx_pos=ctx_x, ctx_slot=ctx_slot,
                cos_sin=rope_table(max(max_pos, 1)), eps=1e-6,
                q_norm_weight=bf16_normal(r["weight"], (LATENT,), mean=1.0, std=0.1))


def insert_workload(seed: int = 1, T: int = 4096, H: int = 128, requests: int = 32,
                    num_pages: int = 2048, max_pos: int = 131072):
    """Inputs of the fused insert step (config 1 at the default sizes)."""
    r = _streams(seed)
    q = bf16_normal(r["q"], (T, H, LATENT))
    kv = bf16_normal(r["kv"], (T, LATENT))
    positions = r["pos"].integers(0, max_pos, size=T).astype(np.int64)
    slots = _distinct(r["slots"], num_pages * PAGE, T).astype(np.int64)
    weight = bf16_normal(r["weight"], (LATENT,), mean=1.0, std=0.1)
    return dict(T=T, H=H, requests=requests, num_pages=num_pages, page_size=PAGE, q=q, kv=kv,
                positions=positions, slot_mapping=slots, q_norm_weight=weight, eps=1e-6,
                cos_sin=rope_table(max_pos))


def compressed_prefill_workload(seed: int = 5, L: int = 8192, H: int = 64, ratio: int = 4,
                                top_k: int = 2048, window: int = 128, P: int = PAGE):
    """One sequence of L query tokens over a compressed KV cache (every `ratio` tokens
    summarised into one entry) plus the raw window cache: top-k min((pos+1)//ratio, top_k)
    distinct uniform compressed entries in [0, (pos+1)//ratio) per token (causal), window
    `window`, every raw token gathered (gather_len = L), sinks ~ N(0,1).  The compressed
    rows are N(0,1) stand-ins for a compressor's output (which needs trained weights);
    each is inserted at position e*ratio + ratio - 1, the last token it covers.  Two
    caches, each with its own seeded random page order."""
    r = _streams(seed)
    N = L // ratio
    q = bf16_normal(r["q"], (L, H, LATENT))
    kv = bf16_normal(r["kv"], (L, LATENT))
    comp_kv = bf16_normal(r["kv"], (N, LATENT))
    topk = np.full((L, top_k), -1, np.int32)
    for pos in range(L):
        hi = (pos + 1) // ratio
        n = min(hi, top_k)
        topk[pos, :n] = _distinct(r["topk"], hi, n)
    sinks = r["sinks"].standard_normal(H).astype(np.float32)
    comp_bt, comp_pages = _block_table(r["perm"], [N], P)
    swa_bt, swa_pages = _block_table(r["perm"], [L], P)
    pos = np.arange(L, dtype=np.int64)
    swa_slots = swa_bt[0, pos // P].astype(np.int64) * P + pos % P
    e = np.arange(N, dtype=np.int64)
    comp_slots = comp_bt[0, e // P].astype(np.int64) * P + e % P
    weight = bf16_normal(r["weight"], (LATENT,), mean=1.0, std=0.1)
    return dict(L=L, H=H, ratio=ratio, top_k=top_k, window=window, P=P, N=N, M=N + L,
                W=round_up(top_k + window, ALIGN), q=q, kv=kv, comp_kv=comp_kv, topk=topk,
                sinks=sinks, comp_bt=comp_bt, comp_pages=comp_pages, swa_bt=swa_bt,
                swa_pages=swa_pages, positions=pos, swa_slots=swa_slots,
                comp_positions=e * ratio + ratio - 1, comp_slots=comp_slots, q_norm_weight=weight,
                eps=1e-6, cos_sin=rope_table(L), qsl=np.array([0, L], np.int32),
                seq_lens=np.array([L], np.int32), gather_lens=np.array([L], np.int32),
                softmax_scale=1.0 / math.sqrt(LATENT))
