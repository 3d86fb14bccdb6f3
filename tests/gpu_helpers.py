"""Helpers shared by the GPU parity tests (host <-> device marshalling, caches built by
the oracle, error metrics)."""
import sys

import numpy as np
import torch

import oracle
from synth_inputs import attention_workload


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    a = np.ascontiguousarray(a if dtype is None else a.astype(dtype))
    return torch.from_numpy(a).cuda()


def bits_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def oracle_cache(wl, num_pages=None, kv_dtype=0, kv_scale=1.0):
    """Host cache (pages of 64 slots, dtype kv_dtype) holding the workload's context rows,
    inserted by the oracle."""
    npg = wl["num_pages"] if num_pages is None else num_pages
    cache = np.zeros(npg * 64 * oracle.kv_record_bytes(kv_dtype), np.uint8)
    T = wl["ctx_kv"].shape[0]
    q0 = np.zeros((T, 0, 576), np.uint16)
    oracle.kv_insert(q0, wl["ctx_kv"], wl["ctx_pos"], wl["ctx_slot"], wl["cos_sin"],
                     np.zeros(576, np.uint16), 1e-6, cache, npg, 64, inplace=True,
                     kv_dtype=kv_dtype, kv_scale=kv_scale)
    return cache


def errors(got_bits, ref):
    g = bits_to_f64(got_bits)
    d = np.abs(g - ref)
    rms = float(np.sqrt(np.mean(ref ** 2))) if ref.size else 0.0
    return d, rms


def assert_attention_close(got_bits, ref, what, max_abs=1e-2, mean_abs=1e-3, out_rounding=False):
    """The 1e-2 max / 1e-3 mean absolute bar holds for outputs of unit scale.  An element
    of magnitude m > 1 gets the bar scaled by m (the bf16 result alone carries a relative
    rounding of 2^-9, i.e. 0.0156 absolute at |out| = 4-8); the mean bar is scaled by
    max(1, RMS of the oracle output).  out_rounding: the mean bar also allows the bf16
    output format's own rounding of the oracle value (ulp / 4 on average for round to
    nearest), which alone is ~1e-3 for outputs near 0.8: the case of peaked logits over
    long rows, whose outputs are whole value rows of unit scale."""
    d, rms = errors(got_bits, ref)
    g = bits_to_f64(got_bits)
    assert np.all(np.isfinite(g)), what
    if d.size == 0:
        return
    bound = max_abs * np.maximum(1.0, np.abs(ref))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7)
    log(f"  {what}: max|d|={d.max():.3e} mean|d|={d.mean():.3e} rms(ref)={rms:.3e} "
        f"max|d|/rms={d.max() / max(rms, 1e-30):.3e} max|d|/ulp_bf16(ref)={np.max(d / ulp):.2f} "
        f"worst/bound={np.max(d / bound):.3f}")
    assert np.all(d <= bound), what
    extra = float(np.mean(ulp) / 4) if out_rounding else 0.0
    assert d.mean() <= mean_abs * max(1.0, rms) + extra, (what, d.mean(), extra)


def within_rotation_bound(got_bits, ref_bits, rope_dims_last):
    """|gpu - oracle| <= 1 bf16 ulp of the oracle value + 2^-20 * the norm of the rotated
    pair it belongs to.  The GPU rotates in fp32 (rounding error ~2^-23 of the pair norm,
    visible as many ulps when a*c - b*s cancels to a tiny value); the oracle rounds the
    exact fp64 value once."""
    g = bits_to_f64(got_bits)
    r = bits_to_f64(ref_bits)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(r), 2.0 ** -126))) - 7)
    tol = ulp.copy()
    rr = r[..., -rope_dims_last:]
    pair = np.sqrt(rr[..., 0::2] ** 2 + rr[..., 1::2] ** 2)
    tol[..., -rope_dims_last:] += np.repeat(pair, 2, axis=-1) * 2.0 ** -20
    same = got_bits == ref_bits  # includes untouched bytes that happen to encode NaN
    with np.errstate(invalid="ignore"):
        d = np.where(same, 0.0, np.abs(g - r))
    ok = bool(np.all(same | (d <= tol)))
    return ok, float(np.mean(same)), float(np.nanmax(np.where(same, 0.0, d / tol)))
