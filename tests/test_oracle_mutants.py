"""Planted mistakes in a copy of the oracle must each fail some pin.

A mutated copy of the oracle's source is built in memory (on the CPU) for
every plausible mistake below -- a dropped term, a wrong sign, an off-by-one
mask, a transposed operand -- and a compact set of the pins used in
test_oracle.py is run against it.  At least one pin must reject every mutant,
and the unmutated oracle must pass all of them.
"""
import math
import os
import types

import numpy as np
import pytest

SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "attention.py")).read()

MUTANTS = [
    ("scale dropped from scores", "s = scale * (qh[rows] @ kh.T)", "s = (qh[rows] @ kh.T)"),
    ("causal mask off by one", "rows[:, None] < keys[None, :]", "rows[:, None] <= keys[None, :]"),
    ("causal mask transposed", "rows[:, None] < keys[None, :]", "rows[:, None] > keys[None, :]"),
    ("max not subtracted consistently", "e = np.exp(s - m[:, None])\n                l = e.sum(axis=1)",
     "e = np.exp(s)\n                l = e.sum(axis=1) * 0 + np.exp(s - m[:, None]).sum(axis=1)"),
    ("LSE drops the max", "lse[b, h, rows] = m + np.log(l)", "lse[b, h, rows] = np.log(l)"),
    ("LSE in base 2", "lse[b, h, rows] = m + np.log(l)", "lse[b, h, rows] = m + np.log2(l)"),
    ("V rows reversed", "o[b, h, rows] = p @ v[b, h]", "o[b, h, rows] = p @ v[b, h][::-1]"),
    ("no normalisation", "p = e / l[:, None]\n                o[b, h, rows]",
     "p = e\n                o[b, h, rows]"),
    ("dV transposed operand", "dv[b, h] = p.T @ do[b, h]", "dv[b, h] = p @ do[b, h]"),
    ("dS sign of delta", "ds = p * (dp - D[:, None])", "ds = p * (dp + D[:, None])"),
    ("delta dropped", "ds = p * (dp - D[:, None])", "ds = p * dp"),
    ("dQ scale dropped", "dq[b, h] = scale * (ds @ k[b, h])", "dq[b, h] = (ds @ k[b, h])"),
    ("dK untransposed", "dk[b, h] = scale * (ds.T @ q[b, h])", "dk[b, h] = scale * (ds @ q[b, h])"),
    ("dP untransposed V", "dp = do[b, h] @ v[b, h].T", "dp = do[b, h] @ v[b, h]"),
    ("online rescale sign", "alpha = np.exp(m - base)", "alpha = np.exp(base - m)"),
    ("online NaN guard removed", "base = np.where(np.isneginf(m_new), 0.0, m_new)", "base = m_new"),
    ("online acc not rescaled", "acc = acc * alpha[:, None] + p @ v[b, h, cols]",
     "acc = acc + p @ v[b, h, cols]"),
]


def _load(src):
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _pins(mod):
    """Return the names of the pins that reject `mod`."""
    failed = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                ok = fn()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    # brute force (pure Python) on tiny inputs, causal and not
    def brute():
        N, d, scale = 4, 3, 0.8
        q, k, v = (_rand((1, 1, N, d), s) for s in (1, 2, 3))
        for causal in (False, True):
            o, lse = mod.forward(q, k, v, scale, causal)
            for i in range(N):
                keys = [j for j in range(N) if (not causal or j <= i)]
                w = {j: math.exp(scale * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d))) for j in keys}
                z = sum(w.values())
                for c in range(d):
                    if not abs(o[0, 0, i, c] - sum(w[j] * v[0, 0, j, c] for j in keys) / z) <= 1e-13:
                        return False
                if not abs(lse[0, 0, i] - math.log(z)) <= 1e-13:
                    return False
        return True

    def online():
        q, k, v = (_rand((1, 1, 23, 4), s) for s in (4, 5, 6))
        for causal in (False, True):
            for desc in (False, True):
                a = mod.forward(q, k, v, 0.5, causal)
                b = mod.online_forward(q, k, v, 0.5, causal, 3, desc)
                if not (np.abs(a[0] - b[0]).max() <= 1e-12 and np.abs(a[1] - b[1]).max() <= 1e-12):
                    return False
        return True

    def finite_diff():
        N, d = 5, 3
        q, k, v, do = (_rand((1, 1, N, d), s) for s in (7, 8, 9, 10))
        for causal in (False, True):
            o, _ = mod.forward(q, k, v, 0.6, causal)
            g = dict(zip("qkv", mod.backward(q, k, v, o, do, 0.6, causal)[:3]))
            for name in "qkv":
                for ix in np.ndindex(q.shape):
                    args = {"q": q, "k": k, "v": v}
                    xp, xm = args[name].copy(), args[name].copy()
                    xp[ix] += 1e-6
                    xm[ix] -= 1e-6
                    lp = np.sum(mod.forward(**{**args, name: xp}, scale=0.6, causal=causal)[0] * do)
                    lm = np.sum(mod.forward(**{**args, name: xm}, scale=0.6, causal=causal)[0] * do)
                    fd = (lp - lm) / 2e-6
                    if not abs(fd - g[name][ix]) <= 1e-7 + 1e-6 * abs(fd):
                        return False
        return True

    check("brute force", brute)
    check("online = full", online)
    check("finite differences", finite_diff)
    return failed


def test_unmutated_oracle_passes_compact_pins():
    assert _pins(_load(SRC)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_rejected(name, old, new):
    assert SRC.count(old) >= 1, f"mutation site for {name!r} not found"
    mutant = _load(SRC.replace(old, new, 1))
    assert _pins(mutant), f"no pin rejects the mutant {name!r}"
