"""fa_fwd_pingpong: the forward scheduled as a ping-pong ("Interrogating the
GPU, part 5: FlashAttention", section "What did FlashAttention-3 do with
Hopper?": one group's softmax under the other group's matrix products).
The kernel performs the row-block kernel's arithmetic in the same order
(only the schedule differs), so its outputs equal fa_fwd's wherever fa_fwd
runs the row-block kernel, value for value; it is also held to the oracle's
tolerances on tails, masks, other scales and wide score ranges."""
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


def _run(fa, x, B, H, N, scale, causal, pingpong):
    import torch
    q, k, v = (to_dev(x[n], torch) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    (fa.fa_fwd_pingpong if pingpong else fa.fa_fwd)(q, k, v, o, lse, scale, causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("shape", [(2, 16, 4096, True), (1, 16, 2048, False), (1, 64, 8192, True)])
def test_equals_row_block_kernel(fa, shape):
    """At these sizes fa_fwd runs the row-block kernel: same values (float
    equality, so +0 and -0 compare equal)."""
    import torch
    B, H, N, causal = shape
    x = fa_inputs.make(B, H, N, seed=8500 + N)
    o0, l0 = _run(fa, x, B, H, N, fa_inputs.SCALE, causal, True)
    o1, l1 = _run(fa, x, B, H, N, fa_inputs.SCALE, causal, False)
    print(f"ping-pong vs row-block B{B} H{H} N{N} causal={causal}: "
          f"O max diff {float((o0.float() - o1.float()).abs().max()):.2e}, "
          f"LSE max diff {float((l0 - l1).abs().max()):.2e}", flush=True)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_small_against_oracle(fa, N, causal):
    B, H = 1, 3
    x = fa_inputs.make(B, H, N, seed=8600 + N + 7 * causal)
    scale = fa_inputs.SCALE
    o, lse = _run(fa, x, B, H, N, scale, causal, True)
    ro, rl = ora.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), scale, causal)
    eo, el = max_err(from_dev(o), ro), max_err(from_dev(lse), rl)
    print(f"ping-pong N={N} causal={causal}: O err {eo:.2e} LSE err {el:.2e}", flush=True)
    assert eo <= TOL_OUT and el <= TOL_LSE


@pytest.mark.parametrize("scale", [0.0, -fa_inputs.SCALE])
@pytest.mark.parametrize("causal", [False, True])
def test_other_scales(fa, scale, causal):
    B, H, N = 1, 2, 300
    x = fa_inputs.make(B, H, N, seed=8700 + causal)
    o, lse = _run(fa, x, B, H, N, scale, causal, True)
    ro, rl = ora.forward(f64(x["q"]), f64(x["k"]), f64(x["v"]), scale, causal)
    eo, el = max_err(from_dev(o), ro), max_err(from_dev(lse), rl)
    print(f"ping-pong scale {scale:+.4f} causal={causal}: O err {eo:.2e} LSE err {el:.2e}", flush=True)
    assert eo <= TOL_OUT and el <= TOL_LSE


def test_std4_scores_every_head(fa):
    """Q and K with standard deviation 4: new row maxima often, so the
    rescale carried from a softmax phase to the next MFMA phase is taken
    often; every head against the oracle."""
    B, H, N = 1, 4, 2048
    x = fa_inputs.make(B, H, N, seed=8800, qk_std=4.0)
    scale = fa_inputs.SCALE
    o, lse = _run(fa, x, B, H, N, scale, True, True)
    O, L = from_dev(o), from_dev(lse)

    def one(hh):
        sl = (slice(0, 1), slice(hh, hh + 1))
        ro, rl = ora.forward(f64(x["q"][sl]), f64(x["k"][sl]), f64(x["v"][sl]), scale, True)
        return max_err(O[sl], ro), max_err(L[sl], rl)

    errs = np.array(map_heads(one, range(H), "std4 ping-pong"))
    print(f"ping-pong std 4: worst O err {errs[:, 0].max():.2e}, LSE err {errs[:, 1].max():.2e}", flush=True)
    assert errs[:, 0].max() <= TOL_OUT and errs[:, 1].max() <= TOL_LSE
