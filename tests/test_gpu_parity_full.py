"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times, against the fp64 oracle, over the whole output tensors.

Every head of every output (O, LSE and, where the workload has a backward,
dQ, dK, dV) is compared element by element with the oracle, one head per
oracle call, heads spread over a pool of threads.  The one exception is the
N = 32768 workload, whose oracle costs about 20 s per head: two whole heads
through each forward kernel, and sampled rows of every head (each row is
computed exactly as the full oracle computes it).  Tolerances: 2e-2 max abs
on O, dQ, dK, dV; 1e-3 on LSE.  Each test prints the worst error per tensor
and its margin to the bar.
"""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as ora
from tests.gpu_helpers import TOL_LSE, TOL_OUT, f64, from_dev, map_heads, max_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_10_amd as fa
    fa.load_library()
    return fa


def log(msg):
    print(msg, flush=True)


def report(label, worst):
    """Print the worst error per tensor with its margin; assert the bars."""
    parts = []
    for name, err in worst.items():
        bar = TOL_LSE if name == "LSE" else TOL_OUT
        parts.append(f"{name} {err:.3e} ({100 * (1 - err / bar):.1f} % below the bar)")
    log(f"{label}: " + ", ".join(parts))
    for name, err in worst.items():
        assert err <= (TOL_LSE if name == "LSE" else TOL_OUT), f"{label}: {name} {err:.3e}"


def forward_all_heads(x, causal, O, L, label):
    """Max abs error of O and LSE over every (b, h) head."""
    B, H = O.shape[:2]

    def one(bh):
        b, hh = bh
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        ro, rl = ora.forward(f64(x["q"][sl]), f64(x["k"][sl]), f64(x["v"][sl]), fa_inputs.SCALE, causal)
        return max_err(O[sl], ro), max_err(L[sl], rl)

    errs = map_heads(one, [(b, hh) for b in range(B) for hh in range(H)], label)
    return {"O": max(e[0] for e in errs), "LSE": max(e[1] for e in errs)}


def run_forward(fa, entry, x, causal):
    import torch
    q, k, v = (to_dev(x[n], torch) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    entry(q, k, v, o, lse, fa_inputs.SCALE, causal)
    torch.cuda.synchronize()
    O, L = from_dev(o), from_dev(lse)
    assert np.isfinite(O).all() and np.isfinite(L).all()
    return O, L


def test_fwd_b1_h1_n512_full(fa):
    x = fa_inputs.make_workload("fwd_b1_h1_n512", with_do=False)
    O, L = run_forward(fa, fa.fa_fwd, x, False)
    ro, rl = ora.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), fa_inputs.SCALE, False)
    report("B1 H1 N512 (every element)", {"O": max_err(O, ro), "LSE": max_err(L, rl)})


@pytest.mark.timeout(900)
def test_fwd_b4_h32_n2048_every_head(fa):
    x = fa_inputs.make_workload("fwd_b4_h32_n2048", with_do=False)
    O, L = run_forward(fa, fa.fa_fwd, x, False)
    report("B4 H32 N2048 (every head)", forward_all_heads(x, False, O, L, "B4 H32 N2048"))


@pytest.mark.timeout(900)
def test_fwd_split_entry_b2_h16_n4096_every_head(fa):
    """The key-split kernel through its own entry point on a workload fa_fwd
    gives to the row-block kernel."""
    x = fa_inputs.make_workload("causal_b2_h16_n4096", with_do=False)
    O, L = run_forward(fa, fa.fa_fwd_split, x, True)
    report("B2 H16 N4096 causal through fa_fwd_split (every head)",
           forward_all_heads(x, True, O, L, "B2 H16 N4096 split"))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_fwd_causal_b1_h4_n2048_std4_every_head(fa, seed):
    """Q and K of standard deviation 4 (scores of standard deviation 16, rows
    dominated by a few keys) on a grid small enough that fa_fwd takes the
    key-split kernel; seed 1 is the input on which that kernel once exceeded
    the O bar (2.07e-2) before it divided O by the sum of the rounded P."""
    x = fa_inputs.make(1, 4, 2048, seed=seed, qk_std=4.0)
    for name, entry in (("fa_fwd", fa.fa_fwd), ("fa_fwd_split", fa.fa_fwd_split)):
        O, L = run_forward(fa, entry, x, True)
        report(f"B1 H4 N2048 causal std 4 seed {seed} through {name} (every head)",
               forward_all_heads(x, True, O, L, f"std4 {name}"))


def _c5_rows(N, n, seed):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 63, 64, 127, 128, N // 2, N - 129, N - 128, N - 2, N - 1]
    return np.unique(np.concatenate([fixed, rng.choice(N, n, replace=False)]))


@pytest.mark.timeout(900)
def test_fwd_causal_b1_h8_n32768_std4(fa):
    """B1 H8 N32768 causal, Q/K std 4, through both forward kernels: heads 0
    and 5 whole, and 100 sampled rows of every head."""
    name = "causal_b1_h8_n32768_std4"
    x = fa_inputs.make_workload(name, with_do=False)
    outs = {"fa_fwd": run_forward(fa, fa.fa_fwd, x, True),
            "fa_fwd_split": run_forward(fa, fa.fa_fwd_split, x, True)}

    def whole(hh):
        sl = (slice(0, 1), slice(hh, hh + 1))
        return ora.forward(f64(x["q"][sl]), f64(x["k"][sl]), f64(x["v"][sl]), fa_inputs.SCALE, True)

    heads = [0, 5]
    refs = map_heads(whole, heads, "N32768 whole heads", workers=2)
    rows = _c5_rows(32768, 100, 5)

    Q, K, V = (f64(x[n]) for n in "qkv")

    def sampled(hh):
        return ora.row_sample_forward(Q, K, V, fa_inputs.SCALE, True, 0, hh, rows)

    srefs = map_heads(sampled, list(range(8)), "N32768 sampled rows")
    for kname, (O, L) in outs.items():
        worst = {"O": 0.0, "LSE": 0.0}
        for hh, (ro, rl) in zip(heads, refs):
            worst["O"] = max(worst["O"], max_err(O[0, hh], ro[0, 0]))
            worst["LSE"] = max(worst["LSE"], max_err(L[0, hh], rl[0, 0]))
        for hh, (xo, xl) in enumerate(srefs):
            worst["O"] = max(worst["O"], max_err(O[0, hh, rows], xo))
            worst["LSE"] = max(worst["LSE"], max_err(L[0, hh, rows], xl))
        report(f"B1 H8 N32768 causal std 4 through {kname} (heads 0, 5 whole; sampled rows of all)",
               worst)


def _backward_every_head(fa, name, shape=None):
    """O, LSE, dQ, dK, dV of every head against the oracle: a named workload,
    or `shape` = (B, H, N, causal, seed) for another size."""
    import torch
    if shape is None:
        w = fa_inputs.WORKLOADS[name]
        x = fa_inputs.make_workload(name, with_do=True)
    else:
        B, H, N, causal, seed = shape
        w = {"B": B, "H": H, "N": N, "causal": causal}
        x = fa_inputs.make(B, H, N, seed=seed, with_do=True)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, fa_inputs.SCALE, w["causal"])
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, fa_inputs.SCALE, w["causal"])
    torch.cuda.synchronize()
    O, L = from_dev(o), from_dev(lse)
    G = [from_dev(t) for t in (dq, dk, dv)]
    for t in [O, L] + G:
        assert np.isfinite(t).all()
    del q, k, v, do, o, lse, dq, dk, dv

    def one(bh):
        b, hh = bh
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        Q, K, V, DO = (f64(x[n][sl]) for n in ("q", "k", "v", "do"))
        ro, rl = ora.forward(Q, K, V, fa_inputs.SCALE, w["causal"])
        rdq, rdk, rdv, _ = ora.backward(Q, K, V, ro, DO, fa_inputs.SCALE, w["causal"])
        return (max_err(O[sl], ro), max_err(L[sl], rl)) + tuple(
            max_err(g[sl], r) for g, r in zip(G, (rdq, rdk, rdv)))

    heads = [(b, hh) for b in range(w["B"]) for hh in range(w["H"])]
    errs = np.array(map_heads(one, heads, name))
    worst_head = [heads[i] for i in errs.argmax(axis=0)]
    names = ("O", "LSE", "dQ", "dK", "dV")
    log(f"{name}: worst head per tensor " + ", ".join(f"{n} {h}" for n, h in zip(names, worst_head)))
    report(f"{name} forward + backward (every head)", dict(zip(names, errs.max(axis=0))))


@pytest.mark.timeout(900)
def test_fwd_bwd_causal_b2_h16_n4096_every_head(fa):
    _backward_every_head(fa, "causal_b2_h16_n4096")


@pytest.mark.timeout(900)
def test_fwd_bwd_non_causal_b1_h8_n4096_every_head(fa):
    """The non-causal gradient kernels (their own instantiations, every tile
    unmasked but the tail) at a multi-tile size: every head."""
    _backward_every_head(fa, "non-causal B1 H8 N4096", shape=(1, 8, 4096, False, 9500))


@pytest.mark.timeout(1200)
def test_fwd_bwd_causal_b1_h64_n8192_every_head(fa):
    """The benchmark's workload: O, LSE, dQ, dK, dV on all 64 heads."""
    _backward_every_head(fa, "causal_b1_h64_n8192")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("scale", [-fa_inputs.SCALE, 0.0])
def test_fwd_bwd_other_scales_b2_h16_n4096(fa, scale):
    """A negative scale (the kernels fold its sign into the operand they hold
    in registers) and scale 0 (uniform attention over the visible keys) at a
    full workload size, causal, through the benchmark's launch configuration:
    O, LSE, dQ, dK, dV of two whole heads against the oracle."""
    import torch
    x = fa_inputs.make_workload("causal_b2_h16_n4096", with_do=True)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, scale, True)
    torch.cuda.synchronize()
    O, L = from_dev(o), from_dev(lse)
    G = [from_dev(t) for t in (dq, dk, dv)]
    for t in [O, L] + G:
        assert np.isfinite(t).all()

    def one(bh):
        b, hh = bh
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        Q, K, V, DO = (f64(x[n][sl]) for n in ("q", "k", "v", "do"))
        ro, rl = ora.forward(Q, K, V, scale, True)
        rdq, rdk, rdv, _ = ora.backward(Q, K, V, ro, DO, scale, True)
        return (max_err(O[sl], ro), max_err(L[sl], rl)) + tuple(
            max_err(g[sl], r) for g, r in zip(G, (rdq, rdk, rdv)))

    errs = np.array(map_heads(one, [(0, 0), (1, 15)], f"scale {scale}", workers=2))
    report(f"B2 H16 N4096 causal, scale {scale:+.4f}, heads (0, 0) and (1, 15)",
           dict(zip(("O", "LSE", "dQ", "dK", "dV"), errs.max(axis=0))))
