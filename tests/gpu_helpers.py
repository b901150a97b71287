"""Shared helpers for the GPU parity tests (torch only for device memory)."""
import numpy as np

import fa_inputs

TOL_OUT = 2e-2   # max abs error on O, dQ, dK, dV against the fp64 oracle
TOL_LSE = 1e-3   # max abs error on LSE


def to_dev(bits, torch, device="cuda"):
    """uint16 bf16 bit array -> torch.bfloat16 device tensor (same bits)."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_dev(t):
    """bf16 / fp32 device tensor -> float64 numpy (exact widening)."""
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def f64(bits):
    return fa_inputs.bf16_bits_to_f64(bits)


def max_err(a, b):
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))
