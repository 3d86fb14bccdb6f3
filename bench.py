#!/usr/bin/env python3
"""Benchmark of the sparse MLA decode hot path on one MI355X.

A step is one pass of the whole path over one decode batch (B = 64 requests, one query
token each, H = 128 heads, context 32768, top-k 2048 with lengths ~ U{1024..2048}, a
128-token sliding window, per-head sinks): q RMSNorm + RoPE in place and the new latent
rows into the FP8 cache, top-k + window -> one physical index row per token, sparse MLA
over it.  By default one launch does it all (dsv4_sparse_mla_decode_step); --launches 2
times dsv4_kv_insert + dsv4_sparse_mla_decode_topk (the row built in LDS), --launches 3
(or --unfused) dsv4_kv_insert + dsv4_combine_indices + dsv4_sparse_mla_decode.
Steps rotate over independent (q, top-k, lengths, sinks) instances so the gathered
cache records (~69 MB per step, ~550 MB over 8 instances) cannot stay in the 256 MB
Infinity Cache.  Inputs are resident in HBM before timing starts.  The launches of a
step are captured into HIP graphs (no allocation, no memset node), one per instance and
one per rotation over all instances (8 complete steps in order), and the timed region
replays whole rotations; a second pass, outside the timed region,
runs the same steps eagerly with HIP events around every launch for the per-kernel
times and the roofline of the decode kernel.

Output: one JSON line (metric, value = query tokens/s, roofline of the dominant kernel
from HIP events around each of its launches in the timed region, and the CPU oracle
timed on the host as a reported baseline).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--instances I] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

METRIC = "sparse MLA decode query-tokens/s + % of HBM/MFMA roofline (B=64,H=128,k=2048)"
KV_DTYPES = {"fp8_ds_mla": 0, "bf16": 1, "fp8_e4m3": 2}
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (spec)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (spec)
LATENT, NOPE, RECORD = 576, 512, 648


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_code_hash(sources):
    """sha256 over the kernel's source files with // comments and blank lines removed
    (comment edits leave the counters valid; any code change invalidates them)."""
    import hashlib
    h = hashlib.sha256()
    for src in sources:
        with open(os.path.join(HERE, src)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def measured_traffic(which="fused"):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    readings (each scaled by the reading of a 256 MiB copy), or None when the kernel's
    sources have changed since the counters were taken.  `which`: the one-launch step,
    the fused combine + decode launch or the plain decode launch."""
    name = {"step": "sparse_mla_decode_step_b64_h128_traffic.json",
            "fused": "sparse_mla_decode_topk_b64_h128_traffic.json",
            "decode": "sparse_mla_decode_b64_h128_traffic.json",
            "step_bf16": "sparse_mla_decode_step_b64_h128_bf16_traffic.json",
            "step_fp8_e4m3": "sparse_mla_decode_step_b64_h128_fp8_e4m3_traffic.json",
            "insert": "insert_t4096_h128_traffic.json",
            "prefill": "sparse_mla_prefill_l8192_h64_traffic.json",
            "mtp": "sparse_mla_decode_step_mtp_b256x2_h128_traffic.json"}.get(which)
    if name is None:
        return None
    path = os.path.join(HERE, "profiles", name)
    try:
        with open(path) as f:
            d = json.load(f)
        if kernel_code_hash(d["kernel_sources"]) != d["kernel_code_sha256"]:
            return None
        return (d["fetch_size_kib_per_dispatch"] * 1024 * d["fetch_factor"] +
                d["write_size_kib_per_dispatch"] * 1024 * d["write_factor"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--instances", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--batch", type=int, default=64,
                    help="decode batch: the first B requests of the workload (default 64, the "
                         "headline configuration; smaller batches exercise --splits)")
    ap.add_argument("--splits", type=int, default=1,
                    help="pieces per index row for dsv4_sparse_mla_decode_split (1 = the "
                         "one-workgroup-per-(token, head group) decode)")
    ap.add_argument("--launches", type=int, default=1, choices=[1, 2, 3],
                    help="1: the whole step in one launch (dsv4_sparse_mla_decode_step); 2: "
                         "insert + fused combine/decode; 3: insert, combine, decode")
    ap.add_argument("--unfused", action="store_true", help="same as --launches 3")
    ap.add_argument("--page-size", type=int, default=64, choices=[32, 64, 256],
                    help="cache page size of the decode workload (default 64)")
    ap.add_argument("--kv-dtype", default="fp8_ds_mla", choices=["fp8_ds_mla", "bf16", "fp8_e4m3"],
                    help="cache dtype of the decode workload: the packed FP8/UE8M0 record "
                         "(default), bf16 records, or E4M3 records with a per-tensor scale")
    ap.add_argument("--kv-scale", type=float, default=0.0625,
                    help="per-tensor scale of the fp8_e4m3 cache")
    ap.add_argument("--workload",
                    choices=["decode", "insert", "mtp", "prefill", "compressed-prefill", "indexer"],
                    default="decode",
                    help="decode (default: the headline decode step); insert (the fused q-norm/"
                         "RoPE/FP8 insert of 4096 tokens x 128 heads); mtp (MTP-style decode: 256 "
                         "requests x 2 query tokens, contexts U{8192..131072}); prefill (one "
                         "8192-token sequence, 64 heads: insert + combine + sparse prefill); "
                         "compressed-prefill (the same over a 4x compressed cache: insert + "
                         "compressed combine + workspace fill + prefill attention); indexer (the "
                         "top-k selection over 64 x 32768 indexer logits, top-k 2048)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed replays of the step before the warm-up steps, so that the GPU "
                         "runs at its sustained clock when timing starts (default 200 ms; 0 = off)")
    ap.add_argument("--reps", type=int, default=5,
                    help="repetitions of the K timed steps for the median (the first is the "
                         "reported value; default 5)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the cache-flushed pass (512 MB written between steps)")
    ap.add_argument("--no-measured-peaks", action="store_true",
                    help="skip the measured peaks (a bf16 GEMM and 1 GiB copy / reduction after "
                         "the timed region) that the roofline is also reported against")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device-to-device copy 3 times (the known-size "
                         "kernel that scales FETCH_SIZE / WRITE_SIZE counter readings)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); multi-GPU runs are not part of it.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        src = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] copied 256 MiB x 3")
        return
    import sparse_mla_attention_combine_amd as dsv4
    from synth_inputs import attention_workload, bf16_normal
    if args.workload == "compressed-prefill":
        return bench_compressed_prefill(args, torch, dsv4)
    if args.workload == "indexer":
        return bench_indexer(args, torch, dsv4)
    if args.workload == "insert":
        return bench_insert(args, torch, dsv4)
    if args.workload == "mtp":
        return bench_mtp(args, torch, dsv4)
    if args.workload == "prefill":
        return bench_prefill(args, torch, dsv4)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    PS = args.page_size
    wl = attention_workload(2, seed=args.seed, instances=args.instances, page_size=PS)
    if not 1 <= args.batch <= wl["T"]:
        print(f"bench.py: --batch must be in 1..{wl['T']}", file=sys.stderr)
        sys.exit(2)
    if args.batch < wl["T"]:  # the first B requests (one query token each)
        B = args.batch
        wl["qsl"], wl["seq_lens"] = wl["qsl"][:B + 1], wl["seq_lens"][:B]
        wl["block_table"], wl["B"], wl["T"] = wl["block_table"][:B], B, B
        for it in wl["instances"]:
            it["q"], it["topk"], it["topk_lens"] = it["q"][:B], it["topk"][:B], it["topk_lens"][:B]
    T, H, W = wl["T"], wl["H"], wl["W"]
    npg = wl["num_pages"]
    log(f"[bench] workload generated in {time.time() - t0:.1f}s: T={T} H={H} W={W} "
        f"pages={npg} context rows={wl['ctx_kv'].shape[0]}")

    def to_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def to_dev(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).to(dev)

    # cache filled by the library's own insert (cache-only: no q heads)
    KVD = KV_DTYPES[args.kv_dtype]
    kvs = args.kv_scale if KVD == 2 else 1.0
    rec_bytes = dsv4.cache_page_bytes(1, KVD)
    cache = dsv4.new_cache(npg, page_size=PS, kv_dtype=KVD)
    cos_sin = to_dev(wl["cos_sin"], np.float32)
    weight = to_bf16(wl["q_norm_weight"])
    dsv4.dsv4_kv_insert(None, to_bf16(wl["ctx_kv"]), to_dev(wl["ctx_pos"], np.int64),
                        to_dev(wl["ctx_slot"], np.int64), cos_sin, None, wl["eps"], cache,
                        page_size=PS, kv_dtype=KVD, kv_scale=kvs)
    qsl = to_dev(wl["qsl"], np.int32)
    seq_lens = to_dev(wl["seq_lens"], np.int32)
    bt = to_dev(wl["block_table"], np.int32)
    pos_np = (wl["seq_lens"].astype(np.int64) - 1)
    slot_np = wl["block_table"][np.arange(T), pos_np // PS].astype(np.int64) * PS + pos_np % PS
    positions = to_dev(pos_np, np.int64)
    slot_mapping = to_dev(slot_np, np.int64)
    rng = np.random.default_rng(1000 + args.seed)

    inst = []
    for it in wl["instances"]:
        d = dict(q=to_bf16(it["q"]), kv=to_bf16(bf16_normal(rng, (T, LATENT))),
                 topk=to_dev(it["topk"], np.int32), topk_lens=to_dev(it["topk_lens"], np.int32),
                 sinks=to_dev(it["sinks"], np.float32),
                 comb=torch.empty(T, W, dtype=torch.int32, device=dev),
                 lens=torch.empty(T, dtype=torch.int32, device=dev),
                 out=torch.empty(T, H, NOPE, dtype=torch.bfloat16, device=dev))
        inst.append(d)
    torch.cuda.synchronize()

    lib = dsv4.library()
    splits = args.splits
    ws_bytes = lib.dsv4_sparse_mla_split_workspace_bytes(T, H, splits) if splits > 1 else 0
    workspace = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = ctypes.c_void_p

    # pre-marshalled C-ABI argument tuples (pointers never change between steps)
    calls = []
    for d in inst:
        ins = (P(d["q"].data_ptr()), P(d["kv"].data_ptr()), P(positions.data_ptr()),
               P(slot_mapping.data_ptr()), P(cos_sin.data_ptr()), cos_sin.shape[0],
               P(weight.data_ptr()), ctypes.c_float(wl["eps"]), P(cache.data_ptr()), npg, PS, KVD,
               ctypes.c_float(kvs), T, H, sp)
        comb = (P(d["topk"].data_ptr()), d["topk"].shape[1], d["topk"].shape[1],
                P(d["topk_lens"].data_ptr()), P(qsl.data_ptr()), P(seq_lens.data_ptr()),
                P(bt.data_ptr()), bt.shape[1], wl["B"], T, wl["top_k"], wl["window"], PS,
                P(d["comb"].data_ptr()), W, P(d["lens"].data_ptr()), sp)
        dec = (P(d["q"].data_ptr()), P(cache.data_ptr()), npg, PS, KVD, ctypes.c_float(kvs),
               P(d["comb"].data_ptr()), W,
               P(d["lens"].data_ptr()), P(d["sinks"].data_ptr()),
               ctypes.c_float(wl["softmax_scale"]), P(d["out"].data_ptr()), None, T, H)
        dec = dec + ((splits, P(workspace.data_ptr()), ctypes.c_size_t(ws_bytes), sp) if splits > 1
                     else (None, ctypes.c_size_t(0), sp))
        fused = (P(d["q"].data_ptr()), P(cache.data_ptr()), npg, PS, KVD, ctypes.c_float(kvs),
                 P(d["topk"].data_ptr()),
                 d["topk"].shape[1], d["topk"].shape[1], P(d["topk_lens"].data_ptr()),
                 P(qsl.data_ptr()), P(seq_lens.data_ptr()), P(bt.data_ptr()), bt.shape[1], wl["B"],
                 wl["top_k"], wl["window"], P(d["sinks"].data_ptr()),
                 ctypes.c_float(wl["softmax_scale"]), P(d["out"].data_ptr()), None, T, H, sp)
        one = ins[:11] + fused[4:]
        if splits > 1:  # the split step: pieces merged by their lse, same workspace
            one = one[:-1] + (splits, P(workspace.data_ptr()), ctypes.c_size_t(ws_bytes), sp)
        calls.append((ins, comb, dec, fused, one))

    def check(st):
        if st != 0:
            raise RuntimeError(lib.dsv4_last_error().decode())

    decode_fn = lib.dsv4_sparse_mla_decode_split if splits > 1 else lib.dsv4_sparse_mla_decode
    launches = 3 if args.unfused else args.launches
    if splits > 1 and launches == 2:
        print("bench.py: --splits needs --launches 1 (the split step) or 3", file=sys.stderr)
        sys.exit(2)
    fused_step = launches == 2
    one_launch = launches == 1
    step_fn = (lib.dsv4_sparse_mla_decode_step_split if splits > 1
               else lib.dsv4_sparse_mla_decode_step)

    def with_stream(args_tuple, stream_ptr):
        return args_tuple[:-1] + (stream_ptr,)

    # valid slots per instance (algorithmic work), from one combine per instance
    n_valid = []
    num_slots = npg * PS
    for (ins, comb, dec, fu, one), d in zip(calls, inst):
        check(lib.dsv4_combine_indices(*comb))
    torch.cuda.synchronize()
    for d in inst:
        c = d["comb"].cpu().numpy()
        L = d["lens"].cpu().numpy()
        mask = (np.arange(W)[None, :] < L[:, None]) & (c >= 0) & (c < num_slots)
        n_valid.append(int(mask.sum()))
    lens_sum = [int(d["lens"].cpu().numpy().sum()) for d in inst]

    n_inst = len(inst)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6 * (args.steps))]

    def run_step(ins, comb, dec, fu, one, stream_ptr=None):
        def s_(a):
            return a if stream_ptr is None else with_stream(a, stream_ptr)
        if one_launch:
            check(step_fn(*s_(one)))
            return
        check(lib.dsv4_kv_insert(*s_(ins)))
        if fused_step:
            check(lib.dsv4_sparse_mla_decode_topk(*s_(fu)))
        else:
            check(lib.dsv4_combine_indices(*s_(comb)))
            check(decode_fn(*s_(dec)))

    def step(i, timed_idx=None):
        ins, comb, dec, fu, one = calls[i % n_inst]
        if timed_idx is None:
            run_step(ins, comb, dec, fu, one)
            return
        e = ev[6 * timed_idx:6 * timed_idx + 6]
        e[0].record(stream)
        if not one_launch:
            check(lib.dsv4_kv_insert(*ins))
        e[1].record(stream)
        e[2].record(stream)
        if launches == 3:
            check(lib.dsv4_combine_indices(*comb))
        e[3].record(stream)
        e[4].record(stream)
        if one_launch:
            check(step_fn(*one))
        else:
            check(lib.dsv4_sparse_mla_decode_topk(*fu) if fused_step else decode_fn(*dec))
        e[5].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # HIP graphs: one per instance holding its step's launches, and one holding a whole
    # rotation (every instance's step in order, n_inst complete steps back to back on one
    # stream), which spares the per-replay gap between steps
    graphs = []
    cap = torch.cuda.Stream()
    for ins, comb, dec, fu, one in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            run_step(ins, comb, dec, fu, one,
                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        graphs.append(g)
    rotation = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rotation, stream=cap):
        for ins, comb, dec, fu, one in calls:
            run_step(ins, comb, dec, fu, one,
                     ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    settle(args, torch, rotation.replay)
    for i in range(args.warmup):
        graphs[i % n_inst].replay()
    rotation.replay()
    torch.cuda.synchronize()

    # timed region: K steps as graph replays (whole rotations, then single steps)
    def timed_steps():
        t0_ = time.perf_counter()
        for _ in range(args.steps // n_inst):
            rotation.replay()
        for k in range(args.steps - args.steps % n_inst, args.steps):
            graphs[k % n_inst].replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0_

    elapsed = timed_steps()
    reps = [elapsed] + [timed_steps() for _ in range(max(args.reps, 1) - 1)]

    # per-kernel times (not part of the timed region): eager steps with events
    for k in range(args.steps):
        step(k, timed_idx=k)
    torch.cuda.synchronize()

    # cache-flushed variant: 512 MB written between steps (not timed), each step timed alone
    flushed_us = None
    if not args.no_flush:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        for k in range(args.steps):
            scratch.fill_(k & 0xFF)
            fe[k][0].record(stream)
            run_step(*calls[k % n_inst])
            fe[k][1].record(stream)
        torch.cuda.synchronize()
        flushed_us = float(np.mean([a.elapsed_time(b) for a, b in fe])) * 1e3
        del scratch

    ins_ms = np.array([ev[6 * k].elapsed_time(ev[6 * k + 1]) for k in range(args.steps)])
    comb_ms = np.array([ev[6 * k + 2].elapsed_time(ev[6 * k + 3]) for k in range(args.steps)])
    dec_ms = np.array([ev[6 * k + 4].elapsed_time(ev[6 * k + 5]) for k in range(args.steps)])
    dec_s = float(dec_ms.mean()) * 1e-3

    # algorithmic work per decode launch, averaged over the rotation actually timed
    used = [k % n_inst for k in range(args.steps)]
    nv = float(np.mean([n_valid[i] for i in used]))
    ls = float(np.mean([lens_sum[i] for i in used]))
    flops = 2.0 * H * (LATENT + NOPE) * nv
    bytes_alg = rec_bytes * nv + T * H * (LATENT + NOPE) * 2 + 4.0 * ls + 4.0 * T + 4.0 * H
    if one_launch:  # + the insert's q write-back, kv rows, cache rows, cos/sin, positions
        bytes_alg += T * H * LATENT * 2 + T * (LATENT * 2 + rec_bytes + 64 * 4 + 16) + LATENT * 2
    achieved_tflops = flops / dec_s / 1e12
    achieved_gbs = bytes_alg / dec_s / 1e9
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = bytes_alg / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"

    value = T * args.steps / elapsed
    dec_name = ("insert+combine+decode (one launch)" if one_launch
                else "combine+decode (fused)" if fused_step else "decode")
    log(f"[bench] {args.steps} steps (graph replays) in {elapsed * 1e3:.2f} ms -> {elapsed / args.steps * 1e6:.1f} us/step; "
        "kernel means: " + ("" if one_launch else f"insert {ins_ms.mean() * 1e3:.1f} us, ")
        + (f"combine {comb_ms.mean() * 1e3:.1f} us, " if launches == 3 else "")
        + f"{dec_name} {dec_ms.mean() * 1e3:.1f} us (median {np.median(dec_ms) * 1e3:.1f}, "
        f"min {dec_ms.min() * 1e3:.1f})")
    log(f"[bench] decode: valid slots/launch {nv:.0f}, {flops / 1e9:.2f} GFLOP, {bytes_alg / 1e6:.1f} MB "
        f"-> {achieved_tflops:.0f} TFLOP/s ({achieved_tflops / PEAK_BF16_TFLOPS * 100:.1f}% of bf16 MFMA), "
        f"{achieved_gbs:.0f} GB/s ({achieved_gbs / PEAK_HBM_GBS * 100:.1f}% of HBM)")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "sparse MLA decode step: fused q-norm/RoPE/FP8 insert + top-k/window "
                        "index combine + sparse MLA over an FP8/UE8M0 paged latent cache",
            "launches": ("insert+combine+decode pieces, lse merge (two launches)"
                         if one_launch and splits > 1 else
                         "insert+combine+decode (one launch)" if one_launch
                         else "insert, combine+decode (fused)" if fused_step
                         else "insert, combine, decode"),
            "batch": T, "heads": H, "top_k": wl["top_k"], "topk_lens": "U{1024..2048}",
            "window": wl["window"], "combined_width": W, "context": int(wl["seq_lens"][0]),
            "page_size": PS, "latent_dim": LATENT, "value_dim": NOPE, "sinks": True,
            "instances_rotated": n_inst,
            "cache": {0: "FP8 e4m3 nope + UE8M0 scales + bf16 rope",
                      1: "bf16 records (576 values)",
                      2: f"FP8 e4m3 records (576 codes), per-tensor scale {kvs}"}[KVD],
            **({"decode_splits": splits} if splits > 1 else {}),
        },
        "roofline": {
            "bound": bound,
            "achieved": round(achieved_tflops if bound == "mfma" else achieved_gbs, 2),
            "peak": PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round((achieved_tflops / PEAK_BF16_TFLOPS) if bound == "mfma"
                          else (achieved_gbs / PEAK_HBM_GBS), 4),
            "traffic": (measured_traffic(("step" if one_launch else "fused" if fused_step
                                          else "decode") + ("" if KVD == 0 else "_" + args.kv_dtype))
                        if (splits == 1 and T == 64 and PS == 64) else None),
            "kernel": ("sparse_mla_kernel<2, fused combine, insert> pieces + split_merge_kernel "
                       "(dsv4_sparse_mla_decode_step_split)" if splits > 1 and one_launch else
                       "sparse_mla_kernel<2> + split_merge_kernel (dsv4_sparse_mla_decode_split)"
                       if splits > 1 else
                       "sparse_mla_kernel<2, fused combine, insert> (dsv4_sparse_mla_decode_step)"
                       if one_launch else
                       "sparse_mla_kernel<2, fused combine> (dsv4_sparse_mla_decode_topk)"
                       if fused_step else "sparse_mla_kernel<2> (dsv4_sparse_mla_decode)"),
            "launch_us": round(dec_s * 1e6, 2),
            "alg_flops": flops, "alg_bytes": bytes_alg,
            "hbm_frac": round(achieved_gbs / PEAK_HBM_GBS, 4),
        },
        "reps_ms_per_step": [round(r / args.steps * 1e3, 5) for r in reps],
        "median_ms_per_step": round(float(np.median(reps)) / args.steps * 1e3, 5),
        "flushed_us_per_step": None if flushed_us is None else round(flushed_us, 2),
        "settle_ms": args.settle_ms,
        "kernels_us": ({"sparse_mla_decode_step": round(float(dec_ms.mean()) * 1e3, 2)}
                       if one_launch else
                       {"kv_insert": round(float(ins_ms.mean()) * 1e3, 2),
                        "sparse_mla_decode_topk": round(float(dec_ms.mean()) * 1e3, 2)}
                       if fused_step else
                       {"kv_insert": round(float(ins_ms.mean()) * 1e3, 2),
                        "combine_indices": round(float(comb_ms.mean()) * 1e3, 2),
                        "sparse_mla_decode": round(float(dec_ms.mean()) * 1e3, 2)}),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, inst[0], calls, H, T, W, PS, KVD, kvs)
    emit(args, torch, result)


def bench_indexer(args, torch, dsv4):
    """The indexer top-k selection at the decode shape: 64 query tokens, each with 32768
    candidate positions (context 32768) of N(0,1) fp32 indexer logits, top-k 2048; 8
    logit instances rotated.  Eager launches with HIP events around each; also logs the
    prefill shape (one 8192-token sequence, causal candidates)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, L, K = 64, 32768, 2048
    rng = np.random.default_rng(args.seed)
    logits = [torch.from_numpy(rng.standard_normal((T, L)).astype(np.float32)).to(dev)
              for _ in range(8)]
    qsl = torch.arange(T + 1, dtype=torch.int32, device=dev)
    seq = torch.full((T,), L, dtype=torch.int32, device=dev)
    out = torch.empty(T, K, dtype=torch.int32, device=dev)
    lens = torch.empty(T, dtype=torch.int32, device=dev)
    for i in range(args.warmup):
        dsv4.dsv4_indexer_topk(logits[i % 8], qsl, seq, K, out, lens)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps)]
    t_start = time.perf_counter()
    for k in range(args.steps):
        ev[2 * k].record()
        dsv4.dsv4_indexer_topk(logits[k % 8], qsl, seq, K, out, lens)
        ev[2 * k + 1].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    us = np.array([ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)]) * 1e3
    bytes_alg = T * L * 4.0 + T * K * 4.0 + T * 4.0
    gbs = bytes_alg / (us.mean() * 1e-6) / 1e9
    # prefill shape: one 8192-token sequence, token i has i+1 candidates
    Lp = 8192
    lp = torch.from_numpy(rng.standard_normal((Lp, Lp)).astype(np.float32)).to(dev)
    qp = torch.tensor([0, Lp], dtype=torch.int32, device=dev)
    sp_ = torch.tensor([Lp], dtype=torch.int32, device=dev)
    op = torch.empty(Lp, K, dtype=torch.int32, device=dev)
    lnp = torch.empty(Lp, dtype=torch.int32, device=dev)
    dsv4.dsv4_indexer_topk(lp, qp, sp_, K, op, lnp)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        dsv4.dsv4_indexer_topk(lp, qp, sp_, K, op, lnp)
    e1.record()
    torch.cuda.synchronize()
    pre_us = e0.elapsed_time(e1) / 5 * 1e3
    pre_bytes = 4.0 * Lp * (Lp + 1) / 2 + 4.0 * Lp * K
    log(f"[bench] indexer top-k {T} x {L} -> {K}: {us.mean():.1f} us mean (median {np.median(us):.1f}, "
        f"min {us.min():.1f}) = {gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS * 100:.1f}% of HBM); "
        f"prefill shape {Lp} causal rows: {pre_us:.0f} us ({pre_bytes / (pre_us * 1e-6) / 1e9:.0f} GB/s)")
    result = {
        "metric": "indexer top-k query-tokens/s + % of HBM roofline (T=64, 32768 candidates, k=2048)",
        "value": round(T / (us.mean() * 1e-6), 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(float(us.mean()) * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "indexer top-k selection over N(0,1) fp32 logits", "tokens": T,
                   "candidates": L, "top_k": K, "instances_rotated": 8},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "indexer_topk_kernel (dsv4_indexer_topk)",
                     "launch_us": round(float(us.mean()), 2), "alg_bytes": bytes_alg},
        "prefill_shape_us": round(pre_us, 1),
    }
    emit(args, torch, result)


def bench_compressed_prefill(args, torch, dsv4):
    """One 8192-token prefill over a compressed cache (ratio 4: 2048 compressed entries)
    plus the raw window cache, H = 64, top-k 2048, window 128.  A step: dsv4_kv_insert
    (q norm/RoPE in place + the 8192 raw rows into the window cache),
    dsv4_combine_indices_compressed, dsv4_gather_workspace (M = 10240 rows),
    dsv4_sparse_mla_prefill over the workspace; captured once into a HIP graph and
    replayed; per-kernel times from a separate eager pass with HIP events."""
    from synth_inputs import compressed_prefill_workload
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = compressed_prefill_workload(seed=args.seed)
    L, H, P, M, N, W = wl["L"], wl["H"], wl["P"], wl["M"], wl["N"], wl["W"]
    log(f"[bench] compressed prefill workload in {time.time() - t0:.1f}s: L={L} H={H} ratio={wl['ratio']} "
        f"N={N} M={M} W={W}")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def dv(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).to(dev)

    comp = dsv4.new_cache(wl["comp_pages"], page_size=P)
    swa = dsv4.new_cache(wl["swa_pages"], page_size=P)
    ws_pages = (M + P - 1) // P
    ws = dsv4.new_cache(ws_pages, page_size=P)
    cos_sin = dv(wl["cos_sin"], np.float32)
    dsv4.dsv4_kv_insert(None, bf(wl["comp_kv"]), dv(wl["comp_positions"], np.int64),
                        dv(wl["comp_slots"], np.int64), cos_sin, None, wl["eps"], comp, page_size=P)
    q, kv = bf(wl["q"]), bf(wl["kv"])
    positions, swa_slots = dv(wl["positions"], np.int64), dv(wl["swa_slots"], np.int64)
    weight = bf(wl["q_norm_weight"])
    topk = dv(wl["topk"], np.int32)
    qsl, seq_lens, gl = dv(wl["qsl"], np.int32), dv(wl["seq_lens"], np.int32), dv(wl["gather_lens"], np.int32)
    comp_bt, swa_bt = dv(wl["comp_bt"], np.int32), dv(wl["swa_bt"], np.int32)
    sinks = dv(wl["sinks"], np.float32)
    comb = torch.empty(L, W, dtype=torch.int32, device=dev)
    lens = torch.empty(L, dtype=torch.int32, device=dev)
    out = torch.empty(L, H, NOPE, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def run(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(torch.cuda.current_stream())
        mark(0)
        dsv4.dsv4_kv_insert(q, kv, positions, swa_slots, cos_sin, weight, wl["eps"], swa, page_size=P)
        mark(1)
        dsv4.dsv4_combine_indices_compressed(topk, None, qsl, seq_lens, gl, wl["top_k"], wl["ratio"],
                                             wl["window"], M, N, comb, lens)
        mark(2)
        dsv4.dsv4_gather_workspace(comp, comp_bt, swa, swa_bt, seq_lens, gl, wl["ratio"], M, N, ws,
                                   page_size=P)
        mark(3)
        dsv4.dsv4_sparse_mla_prefill(q, ws, comb, lens, sinks, wl["softmax_scale"], out, page_size=P)
        mark(4)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        run()
    torch.cuda.synchronize()
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for k in range(args.steps):
        run(evs[k])
    torch.cuda.synchronize()
    kt = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs]) * 1e3  # us

    c = comb.cpu().numpy()
    ln = lens.cpu().numpy()
    valid = (np.arange(W)[None, :] < ln[:, None]) & (c >= 0) & (c < ws_pages * P)
    nv = int(valid.sum())
    rows = int(np.unique(c[valid]).size)
    attn_s = float(kt[:, 3].mean()) * 1e-6
    flops = 2.0 * H * (LATENT + NOPE) * nv
    bytes_alg = RECORD * rows + L * H * (LATENT + NOPE) * 2 + 4.0 * float(ln.sum()) + 4.0 * L + 4.0 * H
    tflops, gbs = flops / attn_s / 1e12, bytes_alg / attn_s / 1e9
    bound = "mfma" if flops / (PEAK_BF16_TFLOPS * 1e12) >= bytes_alg / (PEAK_HBM_GBS * 1e9) else "hbm"
    ws_bytes = 2.0 * RECORD * M
    log(f"[bench] {args.steps} steps (graph replays) in {elapsed * 1e3:.1f} ms -> {elapsed / args.steps * 1e3:.3f} ms/step; "
        f"kernel means: insert {kt[:, 0].mean():.1f} us, combine {kt[:, 1].mean():.1f} us, "
        f"workspace {kt[:, 2].mean():.1f} us ({ws_bytes / (kt[:, 2].mean() * 1e-6) / 1e9:.0f} GB/s), "
        f"attention {kt[:, 3].mean():.1f} us")
    log(f"[bench] attention: {nv} slot visits, {rows} distinct rows, {flops / 1e12:.3f} TFLOP -> "
        f"{tflops:.0f} TFLOP/s ({tflops / PEAK_BF16_TFLOPS * 100:.1f}% of bf16 MFMA)")
    result = {
        "metric": "sparse MLA compressed-cache prefill query-tokens/s + % of MFMA roofline "
                  "(L=8192, H=64, ratio 4, k=2048)",
        "value": round(L * args.steps / elapsed, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "compressed-cache sparse MLA prefill: fused q-norm/RoPE/FP8 insert + "
                               "compressed top-k/window index combine + workspace fill + sparse "
                               "MLA over the workspace",
                   "tokens": L, "heads": H, "compress_ratio": wl["ratio"], "top_k": wl["top_k"],
                   "window": wl["window"], "N": N, "M": M, "page_size": P, "sinks": True},
        "roofline": {"bound": bound,
                     "achieved": round(tflops if bound == "mfma" else gbs, 2),
                     "peak": PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS,
                     "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS, 4),
                     "traffic": None,
                     "kernel": "sparse_mla_prefill_kernel (dsv4_sparse_mla_prefill over the workspace)",
                     "launch_us": round(attn_s * 1e6, 2), "alg_flops": flops, "alg_bytes": bytes_alg},
        "kernels_us": {"kv_insert": round(float(kt[:, 0].mean()), 2),
                       "combine_indices_compressed": round(float(kt[:, 1].mean()), 2),
                       "gather_workspace": round(float(kt[:, 2].mean()), 2),
                       "sparse_mla_prefill": round(float(kt[:, 3].mean()), 2)},
    }
    emit(args, torch, result)


def _graph_of(torch, fn):
    """A HIP graph holding fn's launches (captured on a side stream)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        fn()
    torch.cuda.synchronize()
    return g


def _timed_graph(args, torch, g):
    """settle, W warm-up replays, then K replays timed (repeated args.reps times); returns
    the list of elapsed seconds, the first being the reported one."""
    settle(args, torch, g.replay)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    reps = []
    for _ in range(max(args.reps, 1)):
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        reps.append(time.perf_counter() - t0)
    return reps


def _event_times(torch, launches, steps):
    """Per-launch durations (us) of an eager pass: `launches` is a list of callables, each
    one library call; HIP events around each on the current stream."""
    st = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
          for _ in range(steps)]
    for k in range(steps):
        ev[k][0].record(st)
        for i, f in enumerate(launches):
            f()
            ev[k][i + 1].record(st)
    torch.cuda.synchronize()
    return np.array([[ev[k][i].elapsed_time(ev[k][i + 1]) * 1e3 for i in range(len(launches))]
                     for k in range(steps)])


def _roofline(flops, nbytes, seconds, kernel, traffic=None):
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if t_mfma >= t_hbm else "hbm"
    tflops, gbs = flops / seconds / 1e12, nbytes / seconds / 1e9
    return {"bound": bound,
            "achieved": round(tflops if bound == "mfma" else gbs, 2),
            "peak": PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS if bound == "mfma" else gbs / PEAK_HBM_GBS, 4),
            "traffic": traffic, "kernel": kernel, "launch_us": round(seconds * 1e6, 2),
            "alg_flops": flops, "alg_bytes": nbytes,
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4)}


def _result(args, metric, value, unit, reps, steps, config, roofline, kernels_us, dtype="bf16"):
    return {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1,
            "steps": steps, "warmup": args.warmup,
            "ms_per_step": round(reps[0] / steps * 1e3, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic",
            "config": config, "roofline": roofline,
            "reps_ms_per_step": [round(r / steps * 1e3, 5) for r in reps],
            "median_ms_per_step": round(float(np.median(reps)) / steps * 1e3, 5),
            "settle_ms": args.settle_ms, "kernels_us": kernels_us}


def bench_insert(args, torch, dsv4):
    """The fused insert at its own configuration: 4096 new tokens of 32 requests, 128 heads
    (q RMSNorm + GPT-J RoPE in place, the new latent rows quantised into a 2048-page FP8
    cache at distinct random slots, positions < 131072).  HBM-bound: q read and written
    once (604 MB each way) dominates."""
    from synth_inputs import insert_workload
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = insert_workload(seed=args.seed)
    T, H = wl["T"], wl["H"]

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, kv = bf(wl["q"]), bf(wl["kv"])
    pos = torch.from_numpy(wl["positions"]).to(dev)
    slots = torch.from_numpy(wl["slot_mapping"]).to(dev)
    cs = torch.from_numpy(wl["cos_sin"]).to(dev)
    w = bf(wl["q_norm_weight"])
    cache = dsv4.new_cache(wl["num_pages"])

    def step():
        dsv4.dsv4_kv_insert(q, kv, pos, slots, cs, w, wl["eps"], cache)

    step()
    g = _graph_of(torch, step)
    reps = _timed_graph(args, torch, g)
    us = _event_times(torch, [step], args.steps)[:, 0]
    nbytes = 2.0 * T * H * LATENT * 2 + T * (LATENT * 2 + RECORD + 16 + 64 * 4) + LATENT * 2
    roof = _roofline(0.0, nbytes, float(us.mean()) * 1e-6, "insert_kernel (dsv4_kv_insert)",
                     measured_traffic("insert"))
    log(f"[bench] insert {T} tokens x {H} heads: {reps[0] / args.steps * 1e6:.1f} us/step (graph), "
        f"kernel {us.mean():.1f} us = {nbytes / (us.mean() * 1e-6) / 1e9:.0f} GB/s "
        f"({roof['frac'] * 100:.1f}% of HBM)")
    res = _result(args, "fused insert tokens/s + % of HBM roofline (T=4096, H=128)",
                  T * args.steps / reps[0], "tokens/s", reps, args.steps,
                  {"workload": "fused q RMSNorm + GPT-J RoPE + FP8/UE8M0 KV insert", "tokens": T,
                   "requests": wl["requests"], "heads": H, "cache_pages": wl["num_pages"],
                   "page_size": 64, "max_pos": 131072}, roof,
                  {"kv_insert": round(float(us.mean()), 2)})
    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        n, el, k = 0, 0.0, 0
        cache_h = np.zeros(wl["num_pages"] * 64 * RECORD, np.uint8)
        while el < 10.0 and k + 32 <= T:
            qs = np.array(wl["q"][k:k + 32], copy=True)
            t0 = time.perf_counter()
            oracle.kv_insert(qs, wl["kv"][k:k + 32], wl["positions"][k:k + 32],
                             wl["slot_mapping"][k:k + 32], wl["cos_sin"], wl["q_norm_weight"],
                             wl["eps"], cache_h, wl["num_pages"], 64, inplace=True)
            el += time.perf_counter() - t0
            n += 32
            k += 32
        res["cpu_baseline"] = {"value": round(n / el, 3), "unit": "tokens/s", "cores": 1,
                               "kind": "oracle", "cpu": cpu_model(),
                               "sample": f"the first {n} tokens (all {H} heads), fp64, {el:.1f} s"}
    emit(args, torch, res)


def _compact_cache(wl, idx, lens, tokens):
    """Host cache holding only the rows that `tokens` reference, renumbered to slots 0..m-1,
    and their index rows remapped (the attention result does not depend on slot numbers)."""
    import oracle
    rows = []
    for t in tokens:
        r = idx[t, :lens[t]]
        rows.append(r[r >= 0])
    need = np.unique(np.concatenate(rows))
    new_slot = {int(sl): i for i, sl in enumerate(need)}
    where = {int(sl): i for i, sl in enumerate(wl["ctx_slot"])}
    src = np.array([where[int(sl)] for sl in need], np.int64)
    npg = (len(need) + 63) // 64
    cache = np.zeros(npg * 64 * RECORD, np.uint8)
    oracle.kv_insert(np.zeros((len(need), 0, LATENT), np.uint16), wl["ctx_kv"][src],
                     wl["ctx_pos"][src], np.arange(len(need), dtype=np.int64), wl["cos_sin"],
                     np.zeros(LATENT, np.uint16), wl["eps"], cache, npg, 64, inplace=True)
    idx2 = np.full((len(tokens), idx.shape[1]), -1, np.int32)
    for i, t in enumerate(tokens):
        for j in range(int(lens[t])):
            v = int(idx[t, j])
            idx2[i, j] = new_slot[v] if v >= 0 else -1
    return cache, npg, idx2


def _attention_cpu_baseline(wl, it, idx, lens, H, unit_tokens, budget_s=10.0):
    """The oracle's attention on groups of query tokens spread evenly over the batch (so
    that short causal rows and long ones are sampled alike) until ~budget_s of host work,
    all cores; the rate is scaled by the sample's share of the batch's slot visits."""
    import oracle
    oracle.build()
    cores = len(os.sched_getaffinity(0))
    T = idx.shape[0]
    step = max(cores, 8)
    order = np.random.default_rng(0).permutation(T)
    n, el, visits = 0, 0.0, 0
    while el < budget_s and n + step <= T:
        toks = np.sort(order[n:n + step])
        cache, npg, idx2 = _compact_cache(wl, idx, lens, toks)
        t0 = time.perf_counter()
        oracle.sparse_mla(it["q"][toks], cache, npg, 64, idx2, lens[toks], it["sinks"],
                          wl["softmax_scale"], nthreads=cores, with_lse=False)
        el += time.perf_counter() - t0
        visits += int(lens[toks].sum())
        n += step
    # query tokens per second at the batch's mean row length
    rate = (visits / el) / (float(lens.sum()) / T)
    return {"value": round(rate, 3), "unit": unit_tokens, "cores": cores, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": f"the attention of {n} query tokens drawn uniformly from the batch (H={H}, "
                      f"fp64, all cores; the cache rows they reference renumbered into a compact "
                      f"cache), {el:.1f} s; tokens/s at the batch's mean row length"}


def bench_mtp(args, torch, dsv4):
    """MTP-style decode: 256 requests x 2 query tokens (speculative), 128 heads, contexts
    U{8192..131072} (an ~11.6 GB cache in random page order), top-k 2048 causal per token
    position + a 128-token window, no sinks.  A step is the whole decode step in one launch
    (q norm/RoPE + the 512 new rows + the combine + attention)."""
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = attention_workload_mtp(args)
    it = wl["instances"][0]
    T, H, W, B = wl["T"], wl["H"], wl["W"], wl["B"]
    log(f"[bench] MTP workload in {time.time() - t0:.1f}s: T={T} H={H} pages={wl['num_pages']} "
        f"context rows={wl['ctx_kv'].shape[0]}")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def dv(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).to(dev)

    cache = dsv4.new_cache(wl["num_pages"])
    cs = dv(wl["cos_sin"], np.float32)
    dsv4.dsv4_kv_insert(None, bf(wl["ctx_kv"]), dv(wl["ctx_pos"], np.int64),
                        dv(wl["ctx_slot"], np.int64), cs, None, wl["eps"], cache)
    qsl, sl, bt = dv(wl["qsl"], np.int32), dv(wl["seq_lens"], np.int32), dv(wl["block_table"], np.int32)
    qlens = np.diff(wl["qsl"])
    pos = np.concatenate([np.arange(L - ql, L) for L, ql in zip(wl["seq_lens"], qlens)]).astype(np.int64)
    req = np.repeat(np.arange(B), qlens)
    slots = wl["block_table"][req, pos // 64].astype(np.int64) * 64 + pos % 64
    from synth_inputs import bf16_normal
    rng = np.random.default_rng(2000 + args.seed)
    kv_new = bf(bf16_normal(rng, (T, LATENT)))
    q = bf(it["q"])
    positions, slot_mapping = dv(pos), dv(slots)
    w = bf(wl["q_norm_weight"])
    topk = dv(it["topk"], np.int32)
    out = torch.empty(T, H, NOPE, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step():
        dsv4.dsv4_sparse_mla_decode_step(q, kv_new, positions, slot_mapping, cs, w, wl["eps"], cache,
                                         topk, None, qsl, sl, bt, wl["top_k"], wl["window"], None,
                                         wl["softmax_scale"], out)

    step()
    g = _graph_of(torch, step)
    reps = _timed_graph(args, torch, g)
    us = _event_times(torch, [step], args.steps)[:, 0]
    # algorithmic work from the combined rows (what the decode attends)
    comb = torch.full((T, W), -1, dtype=torch.int32, device=dev)
    lens = torch.zeros(T, dtype=torch.int32, device=dev)
    dsv4.dsv4_combine_indices(topk, None, qsl, sl, bt, wl["top_k"], wl["window"], comb, lens)
    c_np, l_np = comb.cpu().numpy(), lens.cpu().numpy()
    nv = int(((np.arange(W)[None, :] < l_np[:, None]) & (c_np >= 0)).sum())
    flops = 2.0 * H * (LATENT + NOPE) * nv
    nbytes = (RECORD * nv + T * H * (LATENT + NOPE) * 2 + 4.0 * l_np.sum() + 4.0 * T +
              T * H * LATENT * 2 + T * (LATENT * 2 + RECORD + 64 * 4 + 16) + LATENT * 2)
    roof = _roofline(flops, nbytes, float(us.mean()) * 1e-6,
                     "sparse_mla_kernel<2, fused combine, insert> (dsv4_sparse_mla_decode_step)",
                     measured_traffic("mtp"))
    log(f"[bench] MTP step: {reps[0] / args.steps * 1e6:.1f} us/step (graph), kernel {us.mean():.1f} us, "
        f"{nv} valid slots, {flops / 1e9:.1f} GFLOP, {nbytes / 1e6:.0f} MB -> "
        f"{flops / (us.mean() * 1e-6) / 1e12:.0f} TFLOP/s, {nbytes / (us.mean() * 1e-6) / 1e9:.0f} GB/s")
    res = _result(args, "sparse MLA MTP decode query-tokens/s + % of HBM/MFMA roofline "
                        "(B=256 x 2 tokens, H=128, k=2048)",
                  T * args.steps / reps[0], "query-tokens/s", reps, args.steps,
                  {"workload": "MTP decode step: fused q-norm/RoPE/FP8 insert + top-k/window index "
                               "combine + sparse MLA, one launch",
                   "requests": B, "query_tokens": T, "heads": H, "top_k": wl["top_k"],
                   "window": wl["window"], "context": "U{8192..131072}", "page_size": 64,
                   "sinks": False, "cache_GB": round(wl["num_pages"] * 64 * RECORD / 1e9, 2)},
                  roof, {"sparse_mla_decode_step": round(float(us.mean()), 2)})
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _attention_cpu_baseline(wl, it, c_np, l_np, H, "query-tokens/s")
    emit(args, torch, res)


def attention_workload_mtp(args):
    from synth_inputs import attention_workload
    return attention_workload(3, seed=args.seed, instances=1)


def bench_prefill(args, torch, dsv4):
    """Sparse prefill of one 8192-token sequence, 64 heads: every query token attends its
    own causal top-k (min(pos+1, 2048) distinct picks) merged with a 128-token causal
    window, sinks on, over the FP8 cache the step's own insert fills.  A step: dsv4_kv_insert
    (q norm/RoPE in place + the 8192 new latent rows) + dsv4_combine_indices +
    dsv4_sparse_mla_prefill."""
    from synth_inputs import attention_workload
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    wl = attention_workload(4, seed=args.seed, instances=1)
    it = wl["instances"][0]
    T, H, W = wl["T"], wl["H"], wl["W"]
    log(f"[bench] prefill workload in {time.time() - t0:.1f}s: T={T} H={H} pages={wl['num_pages']}")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def dv(a, dt=None):
        return torch.from_numpy(np.ascontiguousarray(a if dt is None else a.astype(dt))).to(dev)

    cache = dsv4.new_cache(wl["num_pages"])
    cs = dv(wl["cos_sin"], np.float32)
    q, kv = bf(it["q"]), bf(wl["ctx_kv"])
    positions, slots = dv(wl["ctx_pos"], np.int64), dv(wl["ctx_slot"], np.int64)
    w = bf(wl["q_norm_weight"])
    qsl, sl, bt = dv(wl["qsl"], np.int32), dv(wl["seq_lens"], np.int32), dv(wl["block_table"], np.int32)
    topk = dv(it["topk"], np.int32)
    sinks = dv(it["sinks"], np.float32)
    comb = torch.full((T, W), -1, dtype=torch.int32, device=dev)
    lens = torch.zeros(T, dtype=torch.int32, device=dev)
    out = torch.empty(T, H, NOPE, dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    launches = [
        lambda: dsv4.dsv4_kv_insert(q, kv, positions, slots, cs, w, wl["eps"], cache),
        lambda: dsv4.dsv4_combine_indices(topk, None, qsl, sl, bt, wl["top_k"], wl["window"],
                                          comb, lens),
        lambda: dsv4.dsv4_sparse_mla_prefill(q, cache, comb, lens, sinks, wl["softmax_scale"], out),
    ]

    def step():
        for f in launches:
            f()

    step()
    g = _graph_of(torch, step)
    reps = _timed_graph(args, torch, g)
    kt = _event_times(torch, launches, args.steps)
    c_np, l_np = comb.cpu().numpy(), lens.cpu().numpy()
    nv = int(((np.arange(W)[None, :] < l_np[:, None]) & (c_np >= 0)).sum())
    attn_s = float(kt[:, 2].mean()) * 1e-6
    flops = 2.0 * H * (LATENT + NOPE) * nv
    nbytes = RECORD * T + T * H * (LATENT + NOPE) * 2 + 4.0 * l_np.sum() + 4.0 * T + 4.0 * H
    roof = _roofline(flops, nbytes, attn_s, "sparse_mla_prefill_kernel (dsv4_sparse_mla_prefill)",
                     measured_traffic("prefill"))
    log(f"[bench] prefill step: {reps[0] / args.steps * 1e3:.3f} ms/step (graph); insert "
        f"{kt[:, 0].mean():.1f} us, combine {kt[:, 1].mean():.1f} us, attention {kt[:, 2].mean():.1f} us "
        f"({nv} slot visits, {flops / 1e12:.3f} TFLOP -> {flops / attn_s / 1e12:.0f} TFLOP/s)")
    res = _result(args, "sparse MLA prefill query-tokens/s + % of MFMA roofline (L=8192, H=64, k=2048)",
                  T * args.steps / reps[0], "query-tokens/s", reps, args.steps,
                  {"workload": "sparse prefill step: fused q-norm/RoPE/FP8 insert + top-k/window "
                               "index combine + sparse MLA prefill",
                   "tokens": T, "heads": H, "top_k": wl["top_k"], "window": wl["window"],
                   "page_size": 64, "sinks": True}, roof,
                  {"kv_insert": round(float(kt[:, 0].mean()), 2),
                   "combine_indices": round(float(kt[:, 1].mean()), 2),
                   "sparse_mla_prefill": round(float(kt[:, 2].mean()), 2)})
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = _attention_cpu_baseline(wl, it, c_np, l_np, H, "query-tokens/s")
    emit(args, torch, res)


def cpu_baseline(wl, d0, calls, H, T, W, PS=64, kv_dtype=0, kv_scale=1.0):
    """The CPU oracle (fp64, as it stands) timed on this host on one full step of
    instance 0: insert + combine + attention for all 64 query tokens."""
    import oracle
    from synth_inputs import bf16_normal  # noqa: F401
    oracle.build()
    cores = len(os.sched_getaffinity(0))
    it = wl["instances"][0]
    npg = wl["num_pages"]
    # host cache holding the rows instance 0 references (built untimed)
    idx0, lens0 = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                                 wl["block_table"], T, wl["top_k"], wl["window"], PS, W)
    need = np.unique(idx0[idx0 >= 0])
    sel = np.isin(wl["ctx_slot"], need)
    cache = np.zeros(npg * PS * oracle.kv_record_bytes(kv_dtype), np.uint8)
    kvk = dict(kv_dtype=kv_dtype, kv_scale=kv_scale)
    oracle.kv_insert(np.zeros((int(sel.sum()), 0, LATENT), np.uint16), wl["ctx_kv"][sel],
                     wl["ctx_pos"][sel], wl["ctx_slot"][sel], wl["cos_sin"],
                     np.zeros(LATENT, np.uint16), wl["eps"], cache, npg, PS, inplace=True, **kvk)
    kv_new = d0["kv"].cpu().view(__import__("torch").int16).numpy().view(np.uint16)
    pos = wl["seq_lens"].astype(np.int64) - 1
    slots = wl["block_table"][np.arange(T), pos // PS].astype(np.int64) * PS + pos % PS

    def one_step():
        # q is normalised in place, so each step starts from a fresh copy; re-inserting the
        # same rows rewrites the same cache bytes
        q = np.array(it["q"], copy=True)
        oracle.kv_insert(q, kv_new, pos, slots, wl["cos_sin"], wl["q_norm_weight"], wl["eps"],
                         cache, npg, PS, inplace=True, **kvk)
        idx, lens = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                                   wl["block_table"], T, wl["top_k"], wl["window"], PS, W)
        oracle.sparse_mla(q, cache, npg, PS, idx, lens, it["sinks"], wl["softmax_scale"],
                          nthreads=cores, with_lse=False, **kvk)

    # repeated full steps until about 10 s of host work (at most 30 steps)
    reps, el = 0, 0.0
    while reps < 30 and (reps == 0 or el < 10.0):
        t0 = time.perf_counter()
        one_step()
        el += time.perf_counter() - t0
        reps += 1
    log(f"[bench] cpu oracle: {reps} steps ({T} query tokens each) in {el:.2f} s on {cores} threads")
    # one core: the attention step of the first 4 query tokens (the step's dominant part)
    n1 = 4
    idx, lens = oracle.combine(it["topk"], it["topk_lens"], wl["qsl"], wl["seq_lens"],
                               wl["block_table"], T, wl["top_k"], wl["window"], PS, W)
    q1 = np.array(it["q"][:n1], copy=True)
    t0 = time.perf_counter()
    oracle.sparse_mla(q1, cache, npg, PS, idx[:n1], lens[:n1], it["sinks"], wl["softmax_scale"],
                      nthreads=1, with_lse=False, **kvk)
    el1 = time.perf_counter() - t0
    return {"value": round(T * reps / el, 3), "unit": "query-tokens/s", "cores": cores,
            "kind": "oracle", "cpu": cpu_model(),
            "value_1core": round(n1 / el1, 3),
            "sample": f"{reps} full decode steps of the same workload (instance 0: {T} query "
                      f"tokens, H={H}; fp64 insert + combine + attention), {el:.1f} s wall; "
                      f"1 core: the attention of {n1} query tokens, {el1:.2f} s"}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_PEAKS = None


def measured_peaks(torch):
    """Peaks this GPU reaches in the library's own probes (dsv4_peak_mfma,
    dsv4_peak_stream), measured once per run after the timed region: dense bf16 MFMAs of
    both shapes the attention kernels use (1024 workgroups, 8 independent accumulators a
    wave), and a 1 GiB streaming read (8192 workgroups) and a 1 GiB copy (16384
    workgroups; bytes read + written) for HBM.
    The roofline's measured fraction uses the larger MFMA rate and the larger HBM rate."""
    global _PEAKS
    if _PEAKS is not None:
        return _PEAKS
    import sparse_mla_attention_combine_amd as dsv4
    dev = torch.device("cuda:0")

    def per_call(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n

    wg = 1024
    fsink = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    mfma = {}
    for shape, name in ((0, "32x32x16"), (1, "16x16x32")):
        flops = dsv4.dsv4_peak_mfma(shape, 2000, fsink)
        mfma[name] = flops / per_call(lambda: dsv4.dsv4_peak_mfma(shape, 2000, fsink), 10) / 1e12
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
    dst = torch.empty_like(src)
    rsink = torch.empty(8192 * 256, dtype=torch.int32, device=dev)
    csink = torch.empty(16384 * 256, dtype=torch.int32, device=dev)
    read_gbs = nbytes / per_call(lambda: dsv4.dsv4_peak_stream(src, rsink), 20) / 1e9
    copy_gbs = 2.0 * nbytes / per_call(lambda: dsv4.dsv4_peak_stream(src, csink, dst=dst), 20) / 1e9
    del src, dst, rsink, csink, fsink
    torch.cuda.synchronize()
    _PEAKS = {"mfma_tflops": round(max(mfma.values()), 1),
              "mfma_32x32x16_tflops": round(mfma["32x32x16"], 1),
              "mfma_16x16x32_tflops": round(mfma["16x16x32"], 1),
              "hbm_gbs": round(max(read_gbs, copy_gbs), 1),
              "hbm_read_gbs": round(read_gbs, 1), "hbm_copy_gbs": round(copy_gbs, 1),
              "how": "dsv4_peak_mfma (dense bf16 MFMA loops, both shapes) and dsv4_peak_stream "
                     "(1 GiB read-only and 1 GiB copy); the larger rate of each kind"}
    log(f"[bench] measured peaks: bf16 MFMA 32x32x16 {mfma['32x32x16']:.0f} / 16x16x32 "
        f"{mfma['16x16x32']:.0f} TFLOP/s; HBM read {read_gbs:.0f} GB/s, copy {copy_gbs:.0f} GB/s")
    return _PEAKS


def emit(args, torch, result):
    """Print the one JSON line; unless disabled, the roofline object also carries the
    measured peaks and the fraction of the binding one that the kernel reached."""
    roof = result.get("roofline")
    if roof is not None and not args.no_measured_peaks and torch.cuda.is_available():
        pk = measured_peaks(torch)
        peak = pk["mfma_tflops"] if roof["bound"] == "mfma" else pk["hbm_gbs"]
        roof["measured_peaks"] = pk
        roof["frac_measured"] = round(roof["achieved"] / peak, 4) if peak > 0 else None
    print(json.dumps(result), flush=True)


def settle(args, torch, replay):
    """Untimed replays for about args.settle_ms, so that timing starts at the sustained clock
    (the decode kernel's duration falls over its first ~40 launches on a fresh process)."""
    if args.settle_ms <= 0:
        return
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        replay()
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
