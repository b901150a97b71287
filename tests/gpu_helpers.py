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


def map_heads(fn, heads, label, workers=None):
    """fn(head) for every head, on a pool of threads (numpy releases the GIL
    inside its array operations), with the BLAS threads split between them
    so that they do not oversubscribe the cores.  Prints one progress line
    per eighth of the heads.  Returns the results in the order of `heads`."""
    import concurrent.futures as cf
    import os
    import time

    from threadpoolctl import threadpool_limits

    heads = list(heads)
    cores = len(os.sched_getaffinity(0))
    if workers is None:
        workers = max(1, min(8, cores))
    t0 = time.time()
    out = [None] * len(heads)
    step = max(1, len(heads) // 8)
    with threadpool_limits(limits=max(1, cores // workers), user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = {ex.submit(fn, h): i for i, h in enumerate(heads)}
            done = 0
            for f in cf.as_completed(futs):
                out[futs[f]] = f.result()
                done += 1
                if done % step == 0 or done == len(heads):
                    print(f"{label}: oracle {done}/{len(heads)} heads ({time.time() - t0:.0f}s)", flush=True)
    return out
