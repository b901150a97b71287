"""The C-ABI library loads, exports every entry point include/fa.h declares,
and rejects bad arguments before touching the GPU (no compute call here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def fa():
    import exact_io_aware_10_amd as fa  # imports torch first: one HIP runtime per process
    if not os.path.exists(fa.LIB_PATH):
        pytest.skip("libfa.so not built")
    fa.load_library()
    return fa


def test_header_declares_the_boundary():
    names = declared()
    for n in ("fa_fwd", "fa_fwd_split", "fa_fwd_soft_exp2", "fa_fwd_pingpong", "fa_bwd_atomic_dq",
              "fa_bwd_atomic_workspace_size", "fa_bwd", "fa_bwd_workspace_size",
              "fa_strerror", "fa_bwd_preprocess", "fa_bwd_dkdv", "fa_bwd_dq"):
        assert n in names


def test_library_exports_every_declared_symbol(fa):
    lib = ctypes.CDLL(fa.LIB_PATH)
    for n in declared():
        assert hasattr(lib, n), n


def test_status_strings(fa):
    for st in range(6):
        assert fa.fa_strerror(st)
    assert "unknown" in fa.fa_strerror(99)
    assert "noalloc" in fa.fa_strerror(fa.FA_ERR_TOO_LARGE)


def test_workspace_size(fa):
    assert fa.fa_bwd_workspace_size(1, 64, 8192, 128, True) == 2 * 64 * 8192 * 4
    assert fa.fa_bwd_workspace_size(1, 1, 3, 128, False) == 256
    assert fa.fa_bwd_workspace_size(1, 1, 3, 64, False) == 0
    assert fa.fa_bwd_workspace_size(-1, 1, 3, 128, False) == 0
    assert fa.fa_bwd_workspace_size(0, 1, 3, 128, False) == 0


FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def fwd_entries(lib):
    """The forward entry points with fa_fwd's argument list (the software-exp2
    one at a quarter of its exponentials in software)."""
    return (lib.fa_fwd, lib.fa_fwd_split, lib.fa_fwd_pingpong,
            lambda *a: lib.fa_fwd_soft_exp2(*a[:-1], 8, a[-1]))


@pytest.mark.parametrize("args,expect", [
    # (B, H, N, d, scale, causal, misalign q) -> status
    ((1, 1, 16, 64, 0.1, 0, 0), 2),
    ((1, 1, 16, 128, float("nan"), 0, 0), 1),
    ((1, 1, 16, 128, float("inf"), 0, 0), 1),
    ((1, 1, 16, 128, float("-inf"), 0, 0), 1),
    # Any finite scale passes validation (shown on empty problems, which
    # return before touching a pointer); the kernels' results at scale 0 and
    # below are checked by the GPU tests.
    ((1, 1, 0, 128, 0.0, 0, 0), 0),
    ((1, 1, 0, 128, -0.5, 1, 0), 0),
    ((1, 1, 0, 128, -3e38, 0, 0), 0),
    ((1, 1, 16, 128, 0.1, 2, 0), 1),
    ((-1, 1, 16, 128, 0.1, 0, 0), 1),
    ((1, -1, 16, 128, 0.1, 0, 0), 1),
    ((1, 1, -16, 128, 0.1, 0, 0), 1),
    ((1, 1, 16, 128, 0.1, 0, 8), 2),
    ((64, 64, 4096, 128, 0.1, 0, 0), 2),  # B*H*N*d = 2^31: index overflow guard
])
def test_fwd_rejects_bad_arguments(fa, args, expect):
    B, H, N, d, scale, causal, mis = args
    lib = fa.load_library()
    for entry in fwd_entries(lib):
        assert entry(FAKE + mis, FAKE, FAKE, FAKE, FAKE, B, H, N, d, scale, causal, None) == expect


def test_fwd_rejects_null_pointers(fa):
    lib = fa.load_library()
    for entry in fwd_entries(lib):
        for i in range(5):
            ptrs = [FAKE] * 5
            ptrs[i] = None
            assert entry(*ptrs, 1, 1, 16, 128, 0.1, 0, None) == fa.FA_ERR_INVALID_ARG


def test_empty_problem_is_a_no_op(fa):
    lib = fa.load_library()
    assert lib.fa_fwd(None, None, None, None, None, 0, 4, 16, 128, 0.1, 0, None) == fa.FA_OK
    assert lib.fa_fwd(None, None, None, None, None, 1, 1, 0, 128, 0.1, 1, None) == fa.FA_OK
    assert lib.fa_fwd_split(None, None, None, None, None, 1, 1, 0, 128, 0.1, 1, None) == fa.FA_OK
    assert lib.fa_fwd_soft_exp2(None, None, None, None, None, 1, 1, 0, 128, 0.1, 1, 16, None) == fa.FA_OK
    assert lib.fa_fwd_pingpong(None, None, None, None, None, 1, 1, 0, 128, 0.1, 1, None) == fa.FA_OK


@pytest.mark.parametrize("share", [-1, 1, 4, 7, 12, 24, 31, 33, 64])
def test_soft_exp2_rejects_bad_shares(fa, share):
    """Only 0, 8, 16 or 32 of the 32 exponentials per tile may go through the
    software path; anything else is refused before any launch, also for an
    empty problem."""
    lib = fa.load_library()
    assert lib.fa_fwd_soft_exp2(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 128, 0.1, 1, share, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_soft_exp2(None, None, None, None, None, 1, 1, 0, 128, 0.1, 1, share, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd(*([None] * 9), 1, 0, 16, 128, 0.1, 0, None, 0, None) == fa.FA_OK


def test_atomic_dq_workspace(fa):
    """fa_bwd_atomic_dq needs the [-D | L log2 e] workspace (padded to 256
    bytes) plus an fp32 dQ buffer, and refuses anything smaller before any
    launch."""
    lib = fa.load_library()
    n = lib.fa_bwd_atomic_workspace_size(1, 2, 100, 128, 1)
    assert n == 1792 + 1 * 2 * 100 * 128 * 4  # 2*200 floats = 1600 bytes, padded to 1792
    assert lib.fa_bwd_atomic_workspace_size(1, 2, 0, 128, 1) == 0
    assert lib.fa_bwd_atomic_workspace_size(1, 2, 100, 64, 1) == 0
    p = [FAKE] * 9
    assert lib.fa_bwd_atomic_dq(*p, 1, 2, 100, 128, 0.1, 1, FAKE, n - 16, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd_atomic_dq(*p, 1, 2, 100, 128, 0.1, 1, None, n, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd_atomic_dq(*([None] * 9), 1, 2, 0, 128, 0.1, 1, None, 0, None) == fa.FA_OK
    assert lib.fa_bwd_atomic_dq(*([None] * 9), 1, 2, 16, 128, 0.1, 1, FAKE, n, None) == fa.FA_ERR_INVALID_ARG


def test_bwd_rejects_bad_workspace(fa):
    lib = fa.load_library()
    p = [FAKE] * 9
    assert lib.fa_bwd(*p, 1, 1, 16, 128, 0.1, 1, None, 1 << 20, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd(*p, 1, 1, 16, 128, 0.1, 1, FAKE, 16, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd(*p, 1, 1, 16, 128, 0.1, 1, FAKE + 4, 1 << 20, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd_preprocess(FAKE, FAKE, FAKE, FAKE, 8, 1, 1, 16, 128, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd_dkdv(FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, FAKE, 1, 1, 16, 128, 0.1, 0, None) == fa.FA_ERR_WORKSPACE
    assert lib.fa_bwd_dq(*([FAKE] * 6), FAKE, 8, FAKE, 1, 1, 16, 128, 0.1, 0, None) == fa.FA_ERR_WORKSPACE


def test_bwd_rejects_bad_shapes(fa):
    lib = fa.load_library()
    p = [FAKE] * 9
    assert lib.fa_bwd(*p, 1, 1, 16, 96, 0.1, 0, FAKE, 1 << 20, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_bwd(*p, 1, 1, 16, 128, float("nan"), 0, FAKE, 1 << 20, None) == fa.FA_ERR_INVALID_ARG
    p[3] = None
    assert lib.fa_bwd(*p, 1, 1, 16, 128, 0.1, 0, FAKE, 1 << 20, None) == fa.FA_ERR_INVALID_ARG


def test_binding_requires_device_tensors(fa):
    import torch
    t = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(t, t, t, 0.1, False)


def test_fp8_sizes(fa):
    assert fa.fa_fp8_codes_size(1, 2, 100, 128, fa.FA_FP8_ROWS) == 2 * 100 * 128
    assert fa.fa_fp8_codes_size(1, 2, 100, 128, fa.FA_FP8_VT) == 2 * 128 * 128  # 2 tiles of 64 keys
    assert fa.fa_fp8_codes_size(1, 2, 100, 128, 7) == 0
    assert fa.fa_fp8_codes_size(1, 2, 100, 96, fa.FA_FP8_ROWS) == 0
    assert fa.fa_fp8_exps_size(2, 3, 65, 128) == 2 * 3 * 2 * 4
    assert fa.fa_fp8_exps_size(0, 3, 65, 128) == 0


def test_fp8_entry_points_reject_bad_arguments(fa):
    lib = fa.load_library()
    assert lib.fa_fp8_quantize(FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 128, 2, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fp8_quantize(FAKE, None, FAKE, FAKE, 1, 1, 16, 128, 0, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fp8_quantize(FAKE, FAKE, FAKE + 4, FAKE, 1, 1, 16, 128, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fp8_quantize(FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 64, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fp8_quantize(None, None, None, None, 1, 0, 16, 128, 0, None) == fa.FA_OK
    p = [FAKE] * 9
    assert lib.fa_fwd_fp8(*p, 1, 1, 16, 128, 0.1, 3, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd_fp8(*p, 1, 1, 16, 128, float("nan"), 0, None) == fa.FA_ERR_INVALID_ARG
    for i in range(9):
        q = list(p)
        q[i] = None
        assert lib.fa_fwd_fp8(*q, 1, 1, 16, 128, 0.1, 0, None) == fa.FA_ERR_INVALID_ARG
        q[i] = FAKE + 8
        assert lib.fa_fwd_fp8(*q, 1, 1, 16, 128, 0.1, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fwd_fp8(*([None] * 9), 1, 1, 0, 128, 0.1, 0, None) == fa.FA_OK


def test_missing_library_fails_loudly():
    """No fallback: with the library absent, the binding raises instead of
    computing anything another way."""
    import subprocess
    import sys
    code = ("import exact_io_aware_10_amd as fa\n"
            "fa.LIB_PATH = '/nonexistent/libfa.so'\n"
            "try:\n"
            "    fa.load_library()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0 and "raised:" in r.stdout and "missing" in r.stdout


def test_noalloc_rejects_problems_beyond_its_scratch(fa):
    """fa_bwd_noalloc's fixed scratch holds the workspace of at most
    FA_NOALLOC_MAX_ROWS rows (B*H*N); one row more is rejected before any
    launch.  Its other argument checks are fa_bwd's."""
    lib = fa.load_library()
    p = [FAKE] * 9
    assert fa.NOALLOC_MAX_ROWS == 2097152
    assert lib.fa_bwd_noalloc(*p, 1, 1, fa.NOALLOC_MAX_ROWS + 1, 128, 0.1, 1, None) == fa.FA_ERR_TOO_LARGE
    assert lib.fa_bwd_noalloc(*p, 2, 4, fa.NOALLOC_MAX_ROWS // 8 + 1, 128, 0.1, 0, None) == fa.FA_ERR_TOO_LARGE
    assert lib.fa_bwd_noalloc(*p, 1, 1, 16, 64, 0.1, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_bwd_noalloc(*p, 1, 1, 16, 128, float("nan"), 0, None) == fa.FA_ERR_INVALID_ARG
    q = list(p)
    q[4] = None
    assert lib.fa_bwd_noalloc(*q, 1, 1, 16, 128, 0.1, 0, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_bwd_noalloc(*([None] * 9), 1, 0, 16, 128, 0.1, 0, None) == fa.FA_OK
