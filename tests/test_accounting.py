"""The FLOP/byte accounting reproduces the arithmetic printed on the pages."""
import json
import os

import pytest

from exact_io_aware_10_amd import accounting as acc

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_arithmetic.json")))


def item(what_prefix):
    for it in GOLD["items"]:
        if it["what"].startswith(what_prefix):
            return it
    raise KeyError(what_prefix)


def test_naive_intensity_tends_to_d_over_2():
    it = item("naive intensity")
    assert acc.naive_intensity(10**9, it["d"]) == pytest.approx(it["value"], rel=1e-6)
    assert acc.naive_intensity(8192, 128) == pytest.approx(63.0, abs=0.05)


def test_score_matrix_bytes():
    it = item("score matrix bytes")
    n = it["N"]
    assert 2 * n * n / 1e6 == pytest.approx(it["value_MB"], abs=0.5)
    it2 = item("scores per layer")
    assert 2 * n * n * it2["heads"] / 1e9 == pytest.approx(it2["value_GB"], abs=0.05)


def test_working_set():
    it = item("working set")
    br = bc = d = 128
    assert [br * d * 2 // 1024, bc * d * 2 // 1024, bc * d * 2 // 1024, br * bc * 4 // 1024] == it["value_KB"]


def test_flash_intensity():
    it = item("flash intensity")
    assert acc.flash_intensity(it["N"], 128) == it["value"]


def test_bytes_kept_per_head():
    it = item("bytes kept per head")
    N, d = 8192, 128
    kept = acc.fwd_bytes(1, 1, N, d) - 3 * N * d * 2  # O and LSE only
    assert kept == 2 * N * d + 4 * N
    assert kept / 1e6 == pytest.approx(it["value_MB"], abs=0.2)
    assert 5 * N * N / 1e6 == pytest.approx(item("textbook bytes kept")["value_MB"], abs=0.5)


def test_metric_conventions():
    # forward 4 N^2 d per head, halved when causal; backward 2.5x.
    assert acc.fwd_flops(1, 64, 8192, 128, True) == pytest.approx(1.0995e12, rel=1e-4)
    assert acc.bwd_flops(1, 64, 8192, 128, True) == pytest.approx(2.7488e12, rel=1e-4)
    assert acc.fwd_bytes(1, 64, 8192, 128) == 64 * (8 * 8192 * 128 + 4 * 8192)
    assert acc.bwd_bytes(2, 16, 4096, 128) == 32 * (16 * 4096 * 128 + 12 * 4096)


def test_fp8_byte_counts():
    # One E4M3 byte per element, an int32 exponent per 64-row block (65 rows
    # -> 2 blocks); the attention writes the same bf16 O and fp32 LSE.
    assert acc.fp8_quant_bytes(1, 1, 65, 128) == 65 * 128 * 3 + 2 * 4
    assert acc.fp8_fwd_bytes(1, 1, 64, 128) == 3 * 64 * 128 + 3 * 4 + 64 * 128 * 2 + 64 * 4
    assert acc.MI355X_FP8_DENSE_TFLOPS == pytest.approx(2 * acc.MI355X_BF16_DENSE_TFLOPS)
