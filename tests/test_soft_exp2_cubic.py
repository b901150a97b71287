"""The software exponential of "Interrogating the GPU, part 5: FlashAttention",
section "Why did Blackwell need FlashAttention-4?": 2^x = 2^n 2^f with
f in [0, 1) and 2^f from the cubic 1 + 0.6951 f + 0.2276 f^2 + 0.0771 f^3.

These CPU tests pin that reading of the page (the coefficients as printed
there, restated here) to what the mathematics fixes: the cubic's error
against 2^f, its end points, and the error of the whole composition in fp32
steps.  The bound they establish (relative error below 1.1e-4) is the one
the GPU tests of fa_fwd_soft_exp2 use: an LSE shift of at most about 1e-4
against the hardware exponential.  The GPU kernel's own coefficients are
checked there, against the fp64 oracle and against fa_fwd."""
import numpy as np

C1, C2, C3 = 0.6951, 0.2276, 0.0771


def cubic(f):
    return 1.0 + f * (C1 + f * (C2 + f * C3))


def test_cubic_relative_error_on_unit_interval():
    f = np.linspace(0.0, 1.0, 100001)
    rel = np.abs(cubic(f) / np.exp2(f) - 1.0)
    assert rel.max() < 1.1e-4
    assert rel.max() > 5e-5  # a cubic cannot do much better: the bound is not vacuous


def test_cubic_end_points():
    assert cubic(0.0) == 1.0
    assert abs(cubic(1.0) - 1.9998) < 1e-12  # the page's cubic sums to 1.9998 at f = 1
    # continuity across integers: 2 * E(0) against E(1) within the same bound
    assert abs(cubic(1.0) / 2.0 - cubic(0.0)) < 1.1e-4


def soft_exp2_f32(x):
    """The composition in fp32 steps: clamp at -126, n = floor, f = x - n, the
    cubic by fused multiply-adds, n added to the exponent field, 0 below -126."""
    x = np.asarray(x, np.float32)

    def fma32(a, b, c):
        return (np.float64(a) * np.float64(b) + np.float64(c)).astype(np.float32)

    with np.errstate(invalid="ignore"):
        xc = np.maximum(x, np.float32(-126.0))
    fl = np.floor(xc).astype(np.float32)
    f = (xc - fl).astype(np.float32)
    p = fma32(fma32(fma32(np.float32(C3), f, np.float32(C2)), f, np.float32(C1)), f, np.float32(1.0))
    r = (p.view(np.int32) + (fl.astype(np.int32) << 23)).view(np.float32)
    return np.where(x >= -126.0, r, np.float32(0.0))


def test_composition_in_fp32_steps():
    """Relative error below 1.1e-4 over the argument range the forward kernel
    produces (scores against a stale maximum: x <= 8), exactly 2^n at
    integers, and 0 below -126 (masked scores are -inf)."""
    rng = np.random.default_rng(11)
    x = rng.uniform(-126.0, 8.0, 200000).astype(np.float32)
    rel = np.abs(soft_exp2_f32(x).astype(np.float64) / np.exp2(x.astype(np.float64)) - 1.0)
    assert rel.max() < 1.1e-4
    ints = np.arange(-126, 9)
    assert np.array_equal(soft_exp2_f32(ints.astype(np.float32)).astype(np.float64), np.exp2(ints.astype(np.float64)))
    assert np.all(soft_exp2_f32(np.array([-126.5, -200.0, -np.inf], np.float32)) == 0.0)
