"""Independent fp64 references used to pin the oracle (tests only).

These use library routines (torch's float8_e4m3fn and bfloat16 conversions, softmax,
matmul, rms_norm, numpy complex arithmetic) rather than the oracle's own code.
"""
import numpy as np
import torch

NOPE, ROPE, LATENT, RECORD = 512, 64, 576, 648


def bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cache_fields(cache: np.ndarray, num_pages: int, P: int):
    pages = cache.reshape(num_pages, P * RECORD)
    nope = pages[:, :P * NOPE].reshape(num_pages, P, NOPE)
    rope = pages[:, P * NOPE:P * (NOPE + 2 * ROPE)].reshape(num_pages, P, 2 * ROPE)
    scale = pages[:, P * (NOPE + 2 * ROPE):].reshape(num_pages, P, 8)
    return nope, rope, scale


def torch_dequant(cache, num_pages, P, slots) -> np.ndarray:
    """fp64 [n, 576] dequantised rows via torch's E4M3 decode; zeros for invalid slots."""
    slots = np.asarray(slots, np.int64)
    nope, rope, scale = cache_fields(cache, num_pages, P)
    out = np.zeros((slots.size, LATENT))
    ok = (slots >= 0) & (slots < num_pages * P)
    s = slots[ok]
    pg, off = s // P, s % P
    codes = torch.from_numpy(np.ascontiguousarray(nope[pg, off])).view(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy()
    sc = np.ldexp(1.0, scale[pg, off].astype(np.int64) - 127)
    v = vals * np.repeat(sc, 64, axis=1)
    v = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    r = bits_to_f64(np.ascontiguousarray(rope[pg, off]).view(np.uint16))
    out[ok] = np.concatenate([v, r], axis=1)
    return out


def dense_attention(q_bits, K, scale, sinks=None):
    """q [H, 576] bf16 bits, K [n, 576] fp64 -> (out [H, 512], lse [H]) in fp64 with
    torch.softmax; a sink is an extra logit column with a zero value row."""
    q = torch.from_numpy(bits_to_f64(q_bits))
    Kt = torch.from_numpy(K)
    s = (q @ Kt.T) * scale
    if sinks is not None:
        s = torch.cat([s, torch.from_numpy(np.asarray(sinks, np.float64))[:, None]], dim=1)
        V = torch.cat([Kt[:, :NOPE], torch.zeros(1, NOPE, dtype=torch.float64)], dim=0)
    else:
        V = Kt[:, :NOPE]
    p = torch.softmax(s, dim=1)
    lse = torch.logsumexp(s, dim=1)
    return (p @ V).numpy(), lse.numpy()
