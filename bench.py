#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step = the whole path over one batch of synthetic input:
  fa_fwd (O, LSE)  ->  fa_bwd_dq (D, L log2 e, dQ)  ->  fa_bwd_dkdv (dK, dV)
on B=1, H=64, N=8192, d=128, causal, bf16 (the N = 8192 workload the
throughput target is stated at; forward-only workloads can be selected with
--workload).  Inputs are seeded iid N(0,1) bf16 tensors already resident in
device memory when the timed region starts.

Prints ONE JSON line on stdout.  `value` is the step's credited TFLOP/s
(forward 4 N^2 d B H, backward 2.5x that, both halved when causal); the
per-kernel durations come from HIP events recorded on the launch stream
around every kernel of every timed step.  The board's power and graphics
clock, sampled while the timed steps run, are reported under `power`.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import threading
import time


def _oracle_threads() -> int:
    """BLAS threads for the oracle timing: the cores this process may run on
    (its affinity mask), capped by OMP_NUM_THREADS where the host sets one
    (the CPU share a shared host grants this process)."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return n


# Set before numpy is first imported (the BLAS library reads these once, at load).
ORACLE_THREADS = _oracle_threads()
for _var in ("OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
    os.environ[_var] = str(ORACLE_THREADS)

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import fa_inputs  # noqa: E402
from exact_io_aware_10_amd import accounting as acc  # noqa: E402

METRIC = "attention fwd/bwd TFLOP/s at d=128 bf16, % of MI355X dense bf16 MFMA peak"
KERNEL_FILES = ("fa_device.hpp", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_atomic.hip", "fa_fp8.hip", "fa_api.cpp", "fa_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def strip_comments(src: str) -> str:
    """C/C++ source without its comments (// to end of line, /* ... */), string
    literals kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c == '"':
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return "".join(out)


def source_hash() -> str:
    """Hash of the kernel and boundary sources with comments removed and
    whitespace collapsed: the counters in profiles/traffic.json stay valid
    across edits of comments and layout."""
    h = hashlib.sha256()
    for f in KERNEL_FILES:
        with open(os.path.join(ROOT, "exact_io_aware_10_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(" ".join(strip_comments(fh.read()).split()).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the current kernel sources (profiles/traffic.json), else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    ent = data.get(f"{kernel}@{workload}")
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


# Oracle sample per workload: (batch 0) heads 0 .. n-1, sized for about
# 10-30 s of CPU work on 16 cores.
CPU_SAMPLE_HEADS = {"fwd_b1_h1_n512": 1, "fwd_b4_h32_n2048": 32, "causal_b1_h64_n8192": 16,
                    "causal_b2_h16_n4096": 8, "causal_b1_h8_n32768_std4": 1}


def cpu_model() -> str:
    """The host CPU's model name (the field lscpu reports as "Model name")."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


CPU_MIN_SECONDS = 10.0  # the sample is repeated until the oracle has run this long


def cpu_baseline(x, w, heads: int):
    """The fp64 oracle (forward, and backward where the workload has one) on
    heads 0 .. heads-1 of batch 0, after an untimed warm-up on a small head;
    the sample is run again until CPU_MIN_SECONDS have passed (small
    workloads), and the rate is the credited FLOPs over the total time."""
    from oracle import attention as ora
    from threadpoolctl import threadpool_info
    blas = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
    has_bwd = "do" in x
    # Warm-up: the same calls on the first 256 rows of head 0 (loads the BLAS
    # library, starts its threads, faults in the code paths).
    wq = fa_inputs.make(1, 1, 256, seed=w["seed"], qk_std=w["qk_std"], with_do=True)
    WQ, WK, WV, WD = (fa_inputs.bf16_bits_to_f64(wq[n]) for n in ("q", "k", "v", "do"))
    wo, _ = ora.forward(WQ, WK, WV, fa_inputs.SCALE, w["causal"])
    if has_bwd:
        ora.backward(WQ, WK, WV, wo, WD, fa_inputs.SCALE, w["causal"])
    sl = (slice(0, 1), slice(0, heads))
    Q, K, V = (fa_inputs.bf16_bits_to_f64(x[n][sl]) for n in "qkv")
    DO = fa_inputs.bf16_bits_to_f64(x["do"][sl]) if has_bwd else None
    flops = acc.fwd_flops(1, heads, w["N"], 128, w["causal"])
    if has_bwd:
        flops += acc.bwd_flops(1, heads, w["N"], 128, w["causal"])
    reps, dt = 0, 0.0
    while reps == 0 or dt < CPU_MIN_SECONDS:
        t0 = time.perf_counter()
        o, _ = ora.forward(Q, K, V, fa_inputs.SCALE, w["causal"])
        if has_bwd:
            ora.backward(Q, K, V, o, DO, fa_inputs.SCALE, w["causal"])
        dt += time.perf_counter() - t0
        reps += 1
    return {
        "value": flops * reps / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": ORACLE_THREADS,
        "kind": "oracle",
        "sample": (f"fp64 oracle {'forward+backward' if has_bwd else 'forward'} on heads 0-{heads - 1} "
                   f"of batch 0 of the same workload, run {reps} time(s), {dt:.1f} s wall in all "
                   f"after a warm-up on 256 rows; credited FLOPs of that sample"),
        "seconds": dt,
        "repetitions": reps,
        "blas_threads": max(blas, default=None),
        "affinity_cores": len(os.sched_getaffinity(0)),
        "host_cpu": cpu_model(),
    }


def gpu_clocks():
    """Current graphics (sclk) and memory (mclk) clock levels in MHz, read
    from the driver's DPM tables (the level marked '*'), or None."""
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            if open(os.path.join(card, "vendor")).read().strip() != "0x1002":
                continue
            for name in ("sclk", "mclk"):
                for line in open(os.path.join(card, f"pp_dpm_{name}")):
                    if line.rstrip().endswith("*"):
                        out[name + "_mhz"] = float(line.split(":")[1].strip().rstrip("*").strip()
                                                   .lower().replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            continue
        if out:
            out["source"] = card + "/pp_dpm_{sclk,mclk}"
            return out
    return None


class PowerSampler:
    """Board power (hwmon power1_input, W) and graphics clock (the '*' level of
    pp_dpm_sclk, MHz) of the first AMD GPU, sampled every 5 ms on a thread
    while the timed steps run; summary() gives their mean, min and max and the
    board's power cap (power1_cap).  Nothing is sampled where sysfs does not
    expose them."""

    def __init__(self, drm_root: str = "/sys/class/drm"):
        self.card = self.power = self.cap = None
        for card in sorted(glob.glob(os.path.join(drm_root, "card*", "device"))):
            try:
                if open(os.path.join(card, "vendor")).read().strip() != "0x1002":
                    continue
            except OSError:
                continue
            hw = sorted(glob.glob(os.path.join(card, "hwmon", "hwmon*", "power1_input")))
            if hw:
                self.card, self.power = card, hw[0]
                cap = os.path.join(os.path.dirname(hw[0]), "power1_cap")
                self.cap = cap if os.path.exists(cap) else None
                break
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    def _read(self):
        w = int(open(self.power).read()) / 1e6
        mhz = None
        for line in open(os.path.join(self.card, "pp_dpm_sclk")):
            if line.rstrip().endswith("*"):
                mhz = float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
        return w, mhz

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except (OSError, ValueError, IndexError):
                return
            self._stop.wait(0.005)

    def start(self):
        if self.power:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        if self._thread:
            self._stop.set()
            self._thread.join()

    def summary(self, skip: float = 0.0):
        """Statistics of the samples after the first `skip` fraction."""
        kept = self.samples[int(len(self.samples) * skip):]
        if not kept:
            return None
        watts = [w for w, _ in kept]
        mhz = [m for _, m in kept if m is not None]
        out = {"samples": len(watts), "interval_ms": 5, "power_w_mean": statistics.mean(watts),
               "power_w_min": min(watts), "power_w_max": max(watts), "source": self.power}
        if self.cap:
            try:
                out["power_cap_w"] = int(open(self.cap).read()) / 1e6
            except (OSError, ValueError):
                pass
        if mhz:
            out.update({"sclk_mhz_mean": statistics.mean(mhz), "sclk_mhz_min": min(mhz),
                        "sclk_mhz_max": max(mhz)})
        return out


def hold_kernels(torch, fa, stream, seconds, kernels):
    """Each kernel alone, back to back for `seconds`, with the board power and
    clock sampled meanwhile; statistics over the second half of the samples
    (the power reading has caught up with the load by then)."""
    out = {}
    for name, fn in kernels.items():
        torch.cuda.synchronize()
        time.sleep(0.5)  # let the board cool back towards idle between kernels
        ps = PowerSampler()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ps.start()
        n, t0 = 0, time.perf_counter()
        ev[0].record(stream)
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                fn()
            n += 10
            torch.cuda.synchronize()
        ev[1].record(stream)
        torch.cuda.synchronize()
        ps.stop()
        out[name] = {"ms": ev[0].elapsed_time(ev[1]) / n, "launches": n, **(ps.summary(skip=0.5) or {})}
        log(f"hold {name}: {out[name]['ms']:.4f} ms, "
            f"{out[name].get('power_w_mean', float('nan')):.0f} W, "
            f"{out[name].get('sclk_mhz_mean', float('nan')):.0f} MHz")
    return out


def kernel_stats(samples):
    """mean, median and min of per-launch durations (ms)."""
    return {"mean": sum(samples) / len(samples), "median": statistics.median(samples),
            "min": min(samples)}


def atomic_dq_backward(fa, torch, q, k, v, o, do, lse, scale, causal, B, H, N, d, stream,
                       warmup: int, steps: int):
    """fa_bwd_atomic_dq (dQ fused into the dK/dV pass through fp32 atomics; "LLM
    flash attention", section "End-to-end flow") on the step's inputs: its four
    launches timed together with HIP events on the launch stream, credited the
    backward's FLOPs; not part of `value`."""
    flops = acc.bwd_flops(B, H, N, d, causal)
    ws = torch.empty(fa.fa_bwd_atomic_workspace_size(B, H, N, d, causal), dtype=torch.uint8, device=q.device)
    g = [torch.empty_like(q) for _ in range(3)]
    for _ in range(max(warmup, 5)):
        fa.fa_bwd_atomic_dq(q, k, v, o, do, lse, *g, scale, causal, ws, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        fa.fa_bwd_atomic_dq(q, k, v, o, do, lse, *g, scale, causal, ws, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    tf = flops / (ms * 1e-3) / 1e12
    del ws, g
    return {"kernels": "bwd_pre_kernel, dq_clear_kernel, bwd_atomic_kernel, dq_convert_kernel", "ms": ms,
            "tflops": tf, "frac_of_peak": tf / acc.MI355X_BF16_DENSE_TFLOPS}


def pingpong_forward(fa, torch, q, k, v, o, lse, scale, causal, B, H, N, d, stream, warmup: int,
                     steps: int):
    """fa_fwd_pingpong (the forward scheduled as FlashAttention-3's ping-pong:
    "Interrogating the GPU, part 5", FlashAttention-3 section) on the step's
    inputs and outputs, timed like the step's kernels; not part of `value`."""
    flops = acc.fwd_flops(B, H, N, d, causal)
    for _ in range(max(warmup, 5)):
        fa.fa_fwd_pingpong(q, k, v, o, lse, scale, causal, stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(steps):
        fa.fa_fwd_pingpong(q, k, v, o, lse, scale, causal, stream)
    ev[1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    tf = flops / (ms * 1e-3) / 1e12
    return {"kernel": "fwd_pp_kernel", "ms": ms, "tflops": tf,
            "frac_of_peak": tf / acc.MI355X_BF16_DENSE_TFLOPS}


def soft_exp2_forward(fa, torch, q, k, v, o, lse, scale, causal, B, H, N, d, stream, warmup: int,
                      steps: int):
    """The row-block forward with 0, 8, 16 or 32 of each lane's 32 exponentials
    per tile evaluated in software (fa_fwd_soft_exp2; "Interrogating the GPU,
    part 5", FlashAttention-4 section), on the same inputs and outputs as the
    step, each share timed over `steps` launches with HIP events on the
    launch stream after `warmup` untimed ones.  Not part of the step or of
    `value`: it measures whether moving exponentials to the FMA path pays
    on this GPU."""
    flops = acc.fwd_flops(B, H, N, d, causal)
    out = {}
    for share in (0, 8, 16, 32):
        for _ in range(max(warmup, 5)):
            fa.fa_fwd_soft_exp2(q, k, v, o, lse, scale, causal, share, stream)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(steps):
            fa.fa_fwd_soft_exp2(q, k, v, o, lse, scale, causal, share, stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / steps
        out[str(share)] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                           "frac_of_peak": flops / (ms * 1e-3) / 1e12 / acc.MI355X_BF16_DENSE_TFLOPS}
    return {"kernel": "row-block forward, share of 32 exponentials per tile in software",
            "by_share": out}


def fp8_forward(fa, torch, q, k, v, w, workload, stream, warmup: int, steps: int):
    """The FP8 forward (incoherent processing) on the same Q, K, V: rotate and
    quantise Q, K, V (three launches), then FP8 attention.  Timed apart from
    the bf16 step with HIP events on the launch stream; FLOPs are credited
    as for the bf16 forward (4 N^2 d per head, halved when causal)."""
    B, H, N, causal = w["B"], w["H"], w["N"], w["causal"]
    d = fa_inputs.HEAD_DIM
    signs = torch.from_numpy(fa_inputs.rotation_signs(fa_inputs.FP8_SIGN_SEED)).to(q.device)
    bufs = {}
    for name, x, layout in (("q", q, fa.FA_FP8_ROWS), ("k", k, fa.FA_FP8_ROWS), ("v", v, fa.FA_FP8_VT)):
        codes = torch.empty(fa.fa_fp8_codes_size(B, H, N, d, layout), dtype=torch.uint8, device=q.device)
        exps = torch.empty(fa.fa_fp8_exps_size(B, H, N, d) // 4, dtype=torch.int32, device=q.device)
        bufs[name] = (x, codes, exps, layout)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        for x, codes, exps, layout in bufs.values():
            fa.fa_fp8_quantize(x, signs, codes, exps, layout, stream)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_fwd_fp8(bufs["q"][1], bufs["q"][2], bufs["k"][1], bufs["k"][2], bufs["v"][1],
                      bufs["v"][2], signs, o, lse, fa_inputs.SCALE, causal, stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for s in range(steps):
        run(evs[s])
    torch.cuda.synchronize()
    quant_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    flops = acc.fwd_flops(B, H, N, d, causal)
    attn_tf = flops / (attn_ms * 1e-3) / 1e12
    return {
        "dtype": "fp8 e4m3 (Q, K, V, P), fp32 accumulate, bf16 O",
        "quantize_ms": quant_ms,
        "quantize_hbm_gbps": 3 * acc.fp8_quant_bytes(B, H, N, d) / (quant_ms * 1e-3) / 1e9,
        "attn_ms": attn_ms,
        "attn_tflops": attn_tf,
        "attn_frac_of_fp8_peak": attn_tf / acc.MI355X_FP8_DENSE_TFLOPS,
        "attn_frac_of_bf16_peak": attn_tf / acc.MI355X_BF16_DENSE_TFLOPS,
        "attn_traffic": traffic_for("fwd_fp8", workload),
        "attn_algorithmic_bytes": acc.fp8_fwd_bytes(B, H, N, d),
        "with_quantize_tflops": flops / ((attn_ms + quant_ms) * 1e-3) / 1e12,
        "fp8_peak_tflops": acc.MI355X_FP8_DENSE_TFLOPS,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40,
                    help="untimed steps first; about 0.2 s lets the clocks settle")
    ap.add_argument("--workload", default="causal_b1_h64_n8192", choices=sorted(fa_inputs.WORKLOADS))
    ap.add_argument("--cpu-heads", type=int, default=None,
                    help="heads in the oracle timing sample (default: per workload, 10-30 s)")
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="forward-only workloads: write this many MiB of scratch before every "
                         "timed step, outside the timed region, so that no input is still in the "
                         "256 MB last-level cache (0: no flush; the K steps then run as one graph)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward timing")
    ap.add_argument("--no-pingpong", action="store_true", help="skip the ping-pong forward timing")
    ap.add_argument("--no-atomic-dq", action="store_true",
                    help="skip the timing of the backward with dQ fused through atomics")
    ap.add_argument("--no-soft-exp2", action="store_true",
                    help="skip the timing of the forward with software exponentials")
    ap.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                    help="time the K steps as one HIP graph replay (auto: for forward-only "
                         "workloads, whose microsecond kernels would otherwise wait on the host)")
    ap.add_argument("--operands", choices=("gaussian", "constant"), default="gaussian",
                    help="constant: every input element 0.5 instead of the workload's Gaussian "
                         "draws -- a diagnostic of how much the operands' switching activity "
                         "costs at the power cap (same instructions, same shapes); not the "
                         "metric's inputs, and the oracle baseline is skipped")
    ap.add_argument("--hold", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, run each kernel of the step alone, back to back, "
                         "for SECONDS and report the board power and graphics clock while it "
                         "runs (the power reading trails the load by a fraction of a second, so "
                         "the timed steps alone are too short to show its steady state)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch
        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n, "calibrate_copy_bytes_written": n}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(heads are independent, so several GPUs would each run this same kernel "
              "on their own share of heads; see the sharding note in the design document).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_io_aware_10_amd as fa

    w = fa_inputs.WORKLOADS[args.workload]
    B, H, N, causal = w["B"], w["H"], w["N"], w["causal"]
    d = fa_inputs.HEAD_DIM
    with_bwd = w["bwd"]
    scale = fa_inputs.SCALE
    log(f"workload {args.workload}: B={B} H={H} N={N} d={d} causal={causal} bwd={with_bwd}")

    x = fa_inputs.make_workload(args.workload, with_do=with_bwd)
    if args.operands == "constant":
        import numpy as np
        x = {n: np.full_like(a, 0x3F00) for n, a in x.items()}  # bf16 bits of 0.5
        args.no_cpu_baseline = True
    dev = torch.device("cuda:0")

    def put(bits):
        import numpy as np
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = put(x["q"]), put(x["k"]), put(x["v"])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    if with_bwd:
        do = put(x["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = fa.workspace_for(B, H, N, causal, dev)
    stream = torch.cuda.current_stream()
    names = ["fwd"] + (["bwd_dq", "bwd_dkdv"] if with_bwd else [])

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, scale, causal, stream)
        if ev is not None:
            ev[1].record(stream)
        if with_bwd:
            fa.fa_bwd_dq(q, k, v, o, do, lse, ws, dq, scale, causal, stream)
            if ev is not None:
                ev[2].record(stream)
            fa.fa_bwd_dkdv(q, k, v, do, ws, dk, dv, scale, causal, stream)
            if ev is not None:
                ev[3].record(stream)

    flush_bytes = (args.flush_mib << 20) if not with_bwd else 0
    scratch = torch.empty(max(flush_bytes // 4, 1), dtype=torch.float32, device=dev)

    def flush():
        # Write more than the 256 MB last-level cache holds, so that the next
        # step finds none of its inputs there (outside the timed region).
        scratch.fill_(1.0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} done")
    clocks_before = gpu_clocks()
    sampler = PowerSampler()
    sampler.start()

    use_graph = args.graph == "on" or (args.graph == "auto" and not with_bwd and not flush_bytes)
    samples = {n: [] for n in names}
    if use_graph:
        # The K steps captured once and replayed: the GPU runs them back to
        # back with no host launch work in between.  Kernel time = replay
        # time / K (events on the stream the replay is launched on).
        graph = torch.cuda.CUDAGraph()
        gstream = torch.cuda.Stream()
        with torch.cuda.stream(gstream):
            with torch.cuda.graph(graph, stream=gstream):
                for _ in range(args.steps):
                    fa.fa_fwd(q, k, v, o, lse, scale, causal)
        graph.replay()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        graph.replay()
        ev[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        samples["fwd"] = [ev[0].elapsed_time(ev[1]) / args.steps]
        ms_per_step = wall / args.steps * 1e3
        timing = "one HIP graph of the K steps (inputs may stay in the last-level cache)"
    elif flush_bytes:
        # Forward-only workloads: every timed step follows a scratch write of
        # flush_bytes; the step's time is its own event pair, so the flush is
        # outside it (and the flush, enqueued first, also hides the host's
        # launch latency from these microsecond kernels).
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            flush()
            step(evs[s_])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        samples["fwd"] = [e[0].elapsed_time(e[1]) for e in evs]
        ms_per_step = sum(samples["fwd"]) / args.steps
        timing = (f"HIP events around every step, each after a {args.flush_mib} MiB scratch write "
                  f"(outside the events); {wall / args.steps * 1e3:.3f} ms per step and flush on the "
                  f"host clock")
    else:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(args.steps):
            step(evs[s_])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for i, n in enumerate(names):
            samples[n] = [e[i].elapsed_time(e[i + 1]) for e in evs]
        ms_per_step = wall / args.steps * 1e3
        timing = "HIP events around every kernel; value from the host clock around the K steps"
    sampler.stop()
    clocks_after = gpu_clocks()
    power = sampler.summary()
    stats = {n: kernel_stats(v_) for n, v_ in samples.items()}
    kern_ms = {n: st["mean"] for n, st in stats.items()}
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step; per kernel mean/median/min (ms): "
        + ", ".join(f"{n} {t['mean']:.4f}/{t['median']:.4f}/{t['min']:.4f}" for n, t in stats.items()))
    log(f"clocks before {clocks_before}, after {clocks_after}")
    if power:
        log(f"board power over the timed steps: mean {power['power_w_mean']:.0f} W, max "
            f"{power['power_w_max']:.0f} W (cap {power.get('power_cap_w', float('nan')):.0f} W), "
            f"sclk mean {power.get('sclk_mhz_mean', float('nan')):.0f} MHz, {power['samples']} samples")

    peak = acc.MI355X_BF16_DENSE_TFLOPS
    fwd_f = acc.fwd_flops(B, H, N, d, causal)
    bwd_f = acc.bwd_flops(B, H, N, d, causal) if with_bwd else 0.0
    step_f = fwd_f + bwd_f
    value = step_f / (ms_per_step * 1e-3) / 1e12
    fwd_tf = fwd_f / (kern_ms["fwd"] * 1e-3) / 1e12
    out_extra = {
        "timing": timing,
        "fwd_ms": kern_ms["fwd"],
        "fwd_tflops": fwd_tf,
        "fwd_frac_of_peak": fwd_tf / peak,
        "fwd_hbm_gbps": acc.fwd_bytes(B, H, N, d) / (kern_ms["fwd"] * 1e-3) / 1e9,
    }
    if with_bwd:
        bwd_ms = kern_ms["bwd_dq"] + kern_ms["bwd_dkdv"]
        bwd_tf = bwd_f / (bwd_ms * 1e-3) / 1e12
        out_extra.update({"bwd_ms": bwd_ms, "bwd_tflops": bwd_tf, "bwd_frac_of_peak": bwd_tf / peak})
    out_extra["kernel_ms"] = kern_ms
    out_extra["kernel_ms_median"] = {n: st["median"] for n, st in stats.items()}
    out_extra["kernel_ms_min"] = {n: st["min"] for n, st in stats.items()}
    out_extra["clocks"] = {"before": clocks_before, "after": clocks_after}
    out_extra["power"] = power
    if with_bwd:
        # The standalone pre-pass (fa_bwd_preprocess: the same workspace the dQ
        # stage writes), timed apart: it is not part of the step, whose dQ
        # kernel computes D itself, but it is the HBM-bound form of that step.
        ws2 = fa.workspace_for(B, H, N, causal, dev)
        for _ in range(5):
            fa.fa_bwd_preprocess(o, do, lse, ws2, stream)
        pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        pev[0].record(stream)
        for _ in range(args.steps):
            fa.fa_bwd_preprocess(o, do, lse, ws2, stream)
        pev[1].record(stream)
        torch.cuda.synchronize()
        pre_ms = pev[0].elapsed_time(pev[1]) / args.steps
        out_extra["bwd_preprocess_standalone"] = {
            "ms": pre_ms, "hbm_gbps": acc.bwd_pre_bytes(B, H, N, d) / (pre_ms * 1e-3) / 1e9,
            "peak_gbps": acc.MI355X_HBM_GBPS}
        del ws2

    if args.hold > 0:
        out_extra["power_per_kernel"] = hold_kernels(torch, fa, stream, args.hold, {
            "fwd": lambda: fa.fa_fwd(q, k, v, o, lse, scale, causal, stream),
            **({"bwd_dq": lambda: fa.fa_bwd_dq(q, k, v, o, do, lse, ws, dq, scale, causal, stream),
                "bwd_dkdv": lambda: fa.fa_bwd_dkdv(q, k, v, do, ws, dk, dv, scale, causal, stream)}
               if with_bwd else {})})

    # Roofline of the kernel that takes the most time per step.
    half = 0.5 if causal else 1.0
    per_head_mm = 2.0 * N * N * d * half  # one N x N x d matmul, causal-halved
    work = {
        "fwd": ("mfma", 2 * per_head_mm * B * H, "fa_fwd: S = Q K^T and O = P V"),
        "bwd_dkdv": ("mfma", 4 * per_head_mm * B * H, "fa_bwd_dkdv: S, dP, dV, dK matmuls"),
        "bwd_dq": ("mfma", 3 * per_head_mm * B * H, "fa_bwd_dq: S, dP, dQ matmuls (and D, L log2e)"),
    }
    dom = max(names, key=lambda n: kern_ms[n])
    bound, units, what = work[dom]
    if bound == "mfma":
        achieved = units / (kern_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                "frac": achieved / peak}
    else:
        achieved = units / (kern_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": acc.MI355X_HBM_GBPS, "unit": "GB/s",
                "frac": achieved / acc.MI355X_HBM_GBPS}
    roof["traffic"] = traffic_for(dom, args.workload)
    roof["kernel"] = dom
    roof["work_per_launch"] = units
    roof["work"] = what
    roof["avg_launch_ms"] = kern_ms[dom]

    # The extra legs run after the timed step and do not enter `value`; an
    # exception in one (an allocation, a status code) is recorded in its field
    # instead of ending the run.
    def leg(name, fn, summary):
        try:
            r = fn()
        except Exception as e:  # noqa: BLE001  (any failure of an auxiliary leg)
            log(f"{name}: failed ({type(e).__name__}: {e})")
            return {"error": f"{type(e).__name__}: {e}"}
        log(summary(r))
        return r

    fp8 = None
    if not args.no_fp8:
        fp8 = leg("fp8 forward",
                  lambda: fp8_forward(fa, torch, q, k, v, w, args.workload, stream, args.warmup, args.steps),
                  lambda r: f"fp8 forward: quantise {r['quantize_ms']:.3f} ms, attention {r['attn_ms']:.3f} ms "
                            f"({r['attn_tflops']:.0f} TFLOP/s credited)")

    pingpong = None
    if not args.no_pingpong:
        pingpong = leg("ping-pong forward",
                       lambda: pingpong_forward(fa, torch, q, k, v, o, lse, scale, causal, B, H, N, d,
                                                stream, args.warmup, args.steps),
                       lambda r: f"ping-pong forward: {r['ms']:.4f} ms ({r['tflops']:.0f} TFLOP/s)")

    atomic = None
    if with_bwd and not args.no_atomic_dq:
        atomic = leg("backward with fused atomic dQ",
                     lambda: atomic_dq_backward(fa, torch, q, k, v, o, do, lse, scale, causal, B, H, N, d,
                                                stream, args.warmup, args.steps),
                     lambda r: f"backward with fused atomic dQ: {r['ms']:.4f} ms ({r['tflops']:.0f} TFLOP/s)")

    soft = None
    if not args.no_soft_exp2:
        soft = leg("forward with software exponentials",
                   lambda: soft_exp2_forward(fa, torch, q, k, v, o, lse, scale, causal, B, H, N, d, stream,
                                             args.warmup, args.steps),
                   lambda r: "forward with software exponentials (share of 32 per tile: ms): "
                             + ", ".join(f"{s_}: {x_['ms']:.4f}" for s_, x_ in r["by_share"].items()))

    cpu = None
    if not args.no_cpu_baseline:
        heads = args.cpu_heads or CPU_SAMPLE_HEADS[args.workload]
        log(f"timing the fp64 oracle on {heads} heads ({ORACLE_THREADS} BLAS threads) ...")
        cpu = cpu_baseline(x, w, heads)
        log(f"oracle: {cpu['seconds']:.1f} s, {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": ("synthetic: seeded iid Gaussian bf16 Q, K, V" + (", dO" if with_bwd else "")
                 + (f" (Q, K std {w['qk_std']:g})" if w["qk_std"] != 1.0 else "")
                 if args.operands == "gaussian" else
                 "diagnostic: every input element 0.5 (not the metric's inputs)"),
        "config": {"workload": args.workload + ("_fwd_bwd" if with_bwd else "_fwd"), "B": B, "H": H,
                   "N": N, "d": d, "causal": causal, "scale": scale},
        "frac_of_peak": value / peak,
        "peak_tflops": peak,
        **out_extra,
        "roofline": roof,
        "fp8_forward": fp8,
        "fwd_pingpong": pingpong,
        "bwd_atomic_dq": atomic,
        "fwd_soft_exp2": soft,
        "cpu_baseline": cpu,
        "source_hash": source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
