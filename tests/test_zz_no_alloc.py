"""fa_bwd_noalloc (the backward with its workspace in the library's fixed
per-GPU scratch) against fa_bwd with a caller-allocated workspace, through
the C ABI: bitwise equal gradients on two calls in a row, the second on a
smaller problem (the scratch then still holds the first call's workspace,
which the pre-pass must overwrite wherever the later kernels read), and the
largest problem the scratch holds."""
import pytest

import fa_inputs
from tests.gpu_helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_10_amd as fa
    fa.load_library()
    return fa


def _inputs(B, H, N, seed):
    import torch
    if B * H * N <= 1 << 16:
        x = fa_inputs.make(B, H, N, seed=seed, with_do=True)
        return [to_dev(x[n], torch) for n in ("q", "k", "v", "do")]
    # Large sizes: drawn on the device (both entry points see the same tensors).
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn((B, H, N, 128), generator=g, device="cuda", dtype=torch.float32)
            .to(torch.bfloat16) for _ in range(4)]


def _both(fa, B, H, N, causal, seed, scale=fa_inputs.SCALE):
    import torch
    q, k, v, do = _inputs(B, H, N, seed)
    o, lse = fa.forward(q, k, v, scale, causal)
    ref = [torch.empty_like(q) for _ in range(3)]
    ws = fa.workspace_for(B, H, N, causal, q.device)
    fa.fa_bwd(q, k, v, o, do, lse, *ref, scale, causal, ws)
    got = [torch.full_like(q, float("nan")) for _ in range(3)]
    fa.fa_bwd_noalloc(q, k, v, o, do, lse, *got, scale, causal)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"{name} differs (B{B} H{H} N{N} causal={causal})"
    print(f"fa_bwd_noalloc B{B} H{H} N{N} causal={causal}: dQ, dK, dV bitwise equal to fa_bwd",
          flush=True)


def test_noalloc_matches_fa_bwd_then_a_smaller_call(fa):
    _both(fa, 2, 8, 1000, True, 6100)
    _both(fa, 1, 3, 129, False, 6101)


def test_noalloc_at_its_largest_size(fa):
    # B*H*N = FA_NOALLOC_MAX_ROWS: the workspace fills the scratch exactly.
    assert 2 * 32 * 32768 == fa.NOALLOC_MAX_ROWS
    _both(fa, 2, 32, 32768, True, 6102)
    _both(fa, 1, 2, 77, True, 6103, scale=-0.3)


def test_noalloc_rejects_one_row_more(fa):
    import torch
    B, H, N = 1, 1, fa.NOALLOC_MAX_ROWS + 1
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")  # never read: rejected first
    lib = fa.load_library()
    p = t.data_ptr()
    assert lib.fa_bwd_noalloc(*([p] * 9), B, H, N, 128, 0.1, 1, None) == fa.FA_ERR_TOO_LARGE
    torch.cuda.synchronize()
