"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws the workloads' random tensors and rounds them to bf16.  It
holds none of the attention arithmetic: both the oracle and the HIP path are
fed the identical bf16 bit patterns produced here.

Recipe (the workloads are iid Gaussian tensors of shape [B, H, N, d]):
  1. draw float32 ``standard_normal`` values from ``numpy.random.default_rng(seed)``
     and multiply by the stated standard deviation;
  2. round each float32 to bfloat16 with round-to-nearest-even on the bit
     pattern (u + 0x7FFF + ((u >> 16) & 1)) >> 16;
  3. the oracle widens those bits exactly to float64; the GPU receives the same
     uint16 words reinterpreted as torch.bfloat16.

Seeds are 1000*k + {0: Q, 1: K, 2: V, 3: dO} for workload k.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
SCALE = 1.0 / np.sqrt(128.0)  # 1/sqrt(d), d = 128

# name -> (B, H, N, causal, qk_std, has_backward, seed base)
WORKLOADS = {
    "fwd_b1_h1_n512": dict(B=1, H=1, N=512, causal=False, qk_std=1.0, bwd=False, seed=1000),
    "fwd_b4_h32_n2048": dict(B=4, H=32, N=2048, causal=False, qk_std=1.0, bwd=False, seed=2000),
    "causal_b1_h64_n8192": dict(B=1, H=64, N=8192, causal=True, qk_std=1.0, bwd=True, seed=3000),
    "causal_b2_h16_n4096": dict(B=2, H=16, N=4096, causal=True, qk_std=1.0, bwd=True, seed=4000),
    "causal_b1_h8_n32768_std4": dict(B=1, H=8, N=32768, causal=True, qk_std=4.0, bwd=False, seed=5000),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def gaussian_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """iid N(0, std^2) values drawn as float32 then rounded to bf16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bf16_bits(x)


def make(B: int, H: int, N: int, seed: int, qk_std: float = 1.0, with_do: bool = False,
         d: int = HEAD_DIM) -> dict:
    """Q, K, V (and dO) as bf16 bit arrays of shape [B, H, N, d]."""
    shape = (B, H, N, d)
    out = {
        "q": gaussian_bf16(seed + 0, shape, qk_std),
        "k": gaussian_bf16(seed + 1, shape, qk_std),
        "v": gaussian_bf16(seed + 2, shape, 1.0),
    }
    if with_do:
        out["do"] = gaussian_bf16(seed + 3, shape, 1.0)
    return out


def make_workload(name: str, with_do: bool | None = None) -> dict:
    w = WORKLOADS[name]
    if with_do is None:
        with_do = w["bwd"]
    return make(w["B"], w["H"], w["N"], w["seed"], w["qk_std"], with_do)


def rotation_signs(seed: int, d: int = HEAD_DIM) -> np.ndarray:
    """The FP8 path's random sign vector (float32 entries +-1), drawn here so
    that the oracle and the GPU receive the same one."""
    rng = np.random.default_rng(seed)
    return np.where(rng.random(d) < 0.5, -1.0, 1.0).astype(np.float32)


FP8_SIGN_SEED = 9000


def make_outlier(B: int, H: int, N: int, seed: int, amp: float, channels=(3, 40, 77, 120)) -> dict:
    """Q, K, V (bf16 bits) where a few head dimensions of K and V are `amp`
    times larger than the rest (the outlier features that incoherent
    processing is meant for), and Q is divided by sqrt(amp) to keep the scores
    in a moderate range."""
    x = make(B, H, N, seed)
    out = {}
    for name, factor in (("q", None), ("k", amp), ("v", amp)):
        f = bf16_bits_to_f64(x[name])
        if factor is None:
            f = f / np.sqrt(amp)
        else:
            f[..., list(channels)] *= factor
        out[name] = f32_to_bf16_bits(f.astype(np.float32))
    return out
