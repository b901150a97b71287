"""Planted mistakes in a copy of the FP8 oracle must each fail some pin.

Like test_oracle_mutants.py for the exact oracle: a mutated copy of
oracle/fp8.py is built in memory for each plausible mistake (a rounding rule,
a butterfly sign, a forgotten factor of the rotation or of a scale) and a
compact set of the pins of test_oracle_fp8.py runs against it.
"""
import os
import types

import numpy as np
import pytest
import scipy.linalg

import fa_inputs
from oracle import attention as ora

SRC = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "fp8.py")).read()

MUTANTS = [
    ("ties round up", "n = np.rint(a / step)", "n = np.floor(a / step + 0.5)"),
    ("subnormal range one binade low", "np.maximum(E, -6.0), -6.0)", "np.maximum(E, -7.0), -6.0)"),
    ("butterfly difference reversed", "y[..., 1, :] = a - b", "y[..., 1, :] = b - a"),
    ("block exponent rule off by one", "e = np.where(f > 0.875, E - 8, E - 9)",
     "e = np.where(f > 0.875, E - 7, E - 8)"),
    ("block exponent boundary", "e = np.where(f > 0.875, E - 8, E - 9)",
     "e = np.where(f >= 0.875, E - 8, E - 9)"),
    ("un-rotation without 1/d", "o[b, h] = (op @ hm) / d * sg", "o[b, h] = (op @ hm) * sg"),
    ("un-rotation without signs", "o[b, h] = (op @ hm) / d * sg", "o[b, h] = (op @ hm) / d"),
    ("score gain of the rotation dropped", "gain = float(d) if rotate_first else 1.0", "gain = 1.0"),
    ("P scale not undone", "p8 = e4m3_decode(e4m3_encode(p * pscale)) / pscale",
     "p8 = e4m3_decode(e4m3_encode(p * pscale))"),
    ("rescale of l forgotten", "l[g] *= alpha\n", "l[g] *= 1.0\n"),
    ("dequantisation exponent sign", "return e4m3_decode(codes) * np.exp2(rows_e)[..., None]",
     "return e4m3_decode(codes) * np.exp2(-rows_e)[..., None]"),
    ("reference: score gain of the rotation dropped", "mult = scale / d if rotate_first else scale",
     "mult = scale"),
    ("reference: P scale not undone", "e4m3_encode(w * 256.0)) * (1.0 / 256.0)",
     "e4m3_encode(w * 256.0))"),
    ("reference: un-rotation without 1/d", "out = sg * (out @ hm) * (1.0 / d)", "out = sg * (out @ hm)"),
    ("reference: un-rotation without signs", "out = sg * (out @ hm) * (1.0 / d)",
     "out = (out @ hm) * (1.0 / d)"),
    ("reference: normalised by the rounded weights' count", "out = (wq @ vr[b, h]) / denom[:, None]",
     "out = (wq @ vr[b, h]) / w.shape[1]"),
    ("reference: P against the row sum instead of the maximum", "w = np.exp(s - m[:, None])",
     "w = np.exp(s - np.log(np.exp(s).sum(axis=1))[:, None])"),
    ("reference: output rounded toward zero", "r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16)",
     "r = ((u >> 16) << 16)"),
]


def _load(src):
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src, "fp8_mutant", "exec"), mod.__dict__)
    return mod


KNOWN = [(0.0, 0x00), (1.0, 0x38), (448.0, 0x7E), (2.0 ** -6, 0x08), (2.0 ** -9, 0x01),
         (1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (0.3, 0x2A)]


def _pins(mod):
    failed = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    check("codes", lambda: all(int(mod.e4m3_encode(np.array([v]))[0]) == c for v, c in KNOWN))

    def fwht():
        xi = np.random.default_rng(5).integers(-50, 50, (3, 128)).astype(np.float32)
        return np.array_equal(mod.fwht32(xi).astype(np.float64),
                              xi.astype(np.float64) @ scipy.linalg.hadamard(128))
    check("fwht", fwht)

    def bexp():
        for a in list(np.random.default_rng(7).uniform(1e-3, 1e3, 50)) + [448.0, 896.0, 224.0]:
            e = int(mod.block_exponent(a))
            if not (a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)):
                return False
        return True
    check("block exponent", bexp)

    x = fa_inputs.make(1, 1, 45, seed=345)
    q, k, v = (fa_inputs.bf16_bits_to_f64(x[n]) for n in "qkv")
    s = fa_inputs.rotation_signs(fa_inputs.FP8_SIGN_SEED)
    o_ref, lse_ref = ora.forward(q, k, v, fa_inputs.SCALE, True)

    # several tiles with growing maxima, so that the rescale runs
    x3 = fa_inputs.make(1, 1, 200, seed=346, qk_std=3.0)
    q3, k3, v3 = (fa_inputs.bf16_bits_to_f64(x3[n]) for n in "qkv")
    o3_ref, lse3_ref = ora.forward(q3, k3, v3, fa_inputs.SCALE, True)

    def exact():
        o, lse = mod.forward_emulated(q3, k3, v3, s, fa_inputs.SCALE, True, quantize=False)
        return np.abs(o - o3_ref).max() <= 1e-11 and np.abs(lse - lse3_ref).max() <= 1e-11
    check("exact without rounding", exact)

    def budget():
        o, lse = mod.forward_emulated(q, k, v, s, fa_inputs.SCALE, True)
        return np.abs(o - o_ref).max() <= 0.15 and np.abs(lse - lse_ref).max() <= 0.15
    check("error budget", budget)

    def ref_exact():
        o, lse = mod.forward_reference(q3, k3, v3, s, fa_inputs.SCALE, True, quantize=False)
        return np.abs(o - o3_ref).max() <= 1e-11 and np.abs(lse - lse3_ref).max() <= 1e-11
    check("reference exact without rounding", ref_exact)

    def ref_budget():
        o, lse = mod.forward_reference(q, k, v, s, fa_inputs.SCALE, True)
        return np.abs(o - o_ref).max() <= 0.15 and np.abs(lse - lse_ref).max() <= 0.15
    check("reference error budget", ref_budget)

    def ref_bf16():
        o, _ = mod.forward_reference(q, k, v, s, fa_inputs.SCALE, True)
        f = o.astype(np.float32)
        nearest = np.abs(o - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 0.15
        return np.all((f.view(np.uint32) & 0xFFFF) == 0) and np.all(nearest)
    check("reference bf16 output", ref_bf16)

    def ref_rne():
        # Uniform weights (scale 0) over two V rows a e_0 and b e_0 with a = 1
        # and b = 1.5 2^-8, both exact in one E4M3 block (exponent -8): every
        # step is exact in fp64 and O_00 = (a + b) / 2 = 0.5 (1 + 2^-8 + 2^-9),
        # which bf16 (ulp 2^-8 there) rounds to nearest as 0.5 (1 + 2^-7).
        qq = np.zeros((1, 1, 2, 128))
        vv = np.zeros((1, 1, 2, 128))
        vv[0, 0, 0, 0], vv[0, 0, 1, 0] = 1.0, 1.5 * 2.0 ** -8
        o, _ = mod.forward_reference(qq, qq, vv, s, 0.0, False)
        return o[0, 0, 0, 0] == 0.5 * (1 + 2.0 ** -7) and np.all(o[0, 0, :, 1:] == 0)
    check("reference rounding", ref_rne)

    def quant():
        codes, exps = mod.quantize_tensor(v, s)
        y = mod.rotate(v, s).astype(np.float64)
        back = mod._dequant(codes, exps)
        e_rows = np.repeat(exps, 64, axis=2)[:, :, :y.shape[2]][..., None]
        return np.all(np.abs(back - y) <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** (e_rows - 10)))
    check("quantisation error", quant)
    return failed


def test_unmutated_fp8_oracle_passes_every_pin():
    assert _pins(_load(SRC)) == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_fp8_mutant_is_caught(name, old, new):
    assert SRC.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    assert _pins(_load(SRC.replace(old, new))) != [], f"no pin rejects: {name}"
