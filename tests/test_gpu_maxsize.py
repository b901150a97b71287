"""The largest problems the ABI accepts: B * H * N * d just below 2^31
elements (4 GiB per bf16 tensor), so element offsets of the last heads pass
2^31 and byte offsets pass 2^32.

B = 2, H = 133152, N = 63: 2,147,475,456 elements.  The inputs are a pool of
32 seeded heads (fa_inputs) repeated over all 266,304 (batch, head) pairs on
the device, so head (b, h) holds pool head h % 32.  Every output head is
compared, on the device and chunk by chunk, with the fp64 oracle's result for
its pool head (the oracle runs on the 32 pool heads only).  A wrong offset
anywhere would put another head's values, or none, into some output head.
"""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as ora
from oracle import fp8 as ofp8
from tests.gpu_helpers import TOL_LSE, TOL_OUT, f64, to_dev

pytestmark = pytest.mark.gpu

B, H, N, POOL = 2, 133152, 63, 32
CHUNK = 8192  # heads per device-side comparison (a multiple of POOL)


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_10_amd as fa
    fa.load_library()
    assert 0 < 2 ** 31 - B * H * N * 128 <= 2 * N * 128  # within two heads of the limit
    return fa


@pytest.fixture(scope="module")
def pool():
    return fa_inputs.make(1, POOL, N, seed=9100, with_do=True)


def _tile(torch, bits):
    """[1, POOL, N, d] pool -> [B, H, N, d] device tensor, head h = pool head h % POOL."""
    small = to_dev(bits, torch)
    return small.repeat(B, H // POOL, 1, 1)


def _max_dev_err(torch, got, want_pool):
    """max |got - want| over every head, want_pool [1, POOL, ...] float64 numpy."""
    want = torch.from_numpy(np.ascontiguousarray(want_pool)).to("cuda", torch.float32)
    worst = 0.0
    for b in range(B):
        for h0 in range(0, H, CHUNK):
            h1 = min(H, h0 + CHUNK)
            g = got[b, h0:h1].float()
            w = want[0].repeat((h1 - h0) // POOL, *([1] * (want.dim() - 2)))
            worst = max(worst, float((g - w).abs().max()))
    return worst


@pytest.mark.parametrize("causal", [False, True])
def test_forward_every_kernel_at_the_largest_size(fa, pool, causal):
    import torch
    q, k, v = (_tile(torch, pool[n]) for n in "qkv")
    ro, rl = ora.forward(f64(pool["q"]), f64(pool["k"]), f64(pool["v"]), fa_inputs.SCALE, causal)
    soft16 = lambda *a: fa.fa_fwd_soft_exp2(*a, 16)  # noqa: E731  (half the exponentials in software)
    for name, entry in (("fa_fwd", fa.fa_fwd), ("fa_fwd_split", fa.fa_fwd_split),
                        ("fa_fwd_pingpong", fa.fa_fwd_pingpong), ("fa_fwd_soft_exp2", soft16)):
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        entry(q, k, v, o, lse, fa_inputs.SCALE, causal)
        torch.cuda.synchronize()
        eo, el = _max_dev_err(torch, o, ro), _max_dev_err(torch, lse, rl)
        print(f"{name} B{B} H{H} N{N} causal={causal}: O {eo:.2e} LSE {el:.2e} over every head", flush=True)
        assert eo <= TOL_OUT and el <= TOL_LSE
        del o, lse
    del q, k, v
    torch.cuda.empty_cache()


def test_backward_at_the_largest_size(fa, pool):
    import torch
    causal = True
    q, k, v, do = (_tile(torch, pool[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, fa_inputs.SCALE, causal)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, fa_inputs.SCALE, causal)
    torch.cuda.synchronize()
    Q, K, V, DO = (f64(pool[n]) for n in ("q", "k", "v", "do"))
    ro, _ = ora.forward(Q, K, V, fa_inputs.SCALE, causal)
    rdq, rdk, rdv, _ = ora.backward(Q, K, V, ro, DO, fa_inputs.SCALE, causal)
    e = [_max_dev_err(torch, g, r) for g, r in ((dq, rdq), (dk, rdk), (dv, rdv))]
    print(f"backward B{B} H{H} N{N}: dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e} over every head", flush=True)
    assert max(e) <= TOL_OUT
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_fp8_codes_at_the_largest_size(fa, pool):
    """E4M3 codes (row layout) and block exponents of every head equal the
    oracle's for its pool head, bit for bit."""
    import torch
    signs = torch.from_numpy(fa_inputs.rotation_signs(fa_inputs.FP8_SIGN_SEED)).cuda()
    want_c, want_e = ofp8.quantize_tensor(f64(pool["k"]), fa_inputs.rotation_signs(fa_inputs.FP8_SIGN_SEED))
    x = _tile(torch, pool["k"])
    codes, exps = fa.quantize_fp8(x, signs, fa.FA_FP8_ROWS)
    torch.cuda.synchronize()
    c = codes[:B * H * N * 128].view(B, H, N, 128)
    wc = torch.from_numpy(want_c).cuda()
    we = torch.from_numpy(want_e.astype(np.int32)).cuda()
    ex = exps[:B * H].view(B, H)  # one 64-row block per head at N = 63
    for b in range(B):
        for h0 in range(0, H, CHUNK):
            h1 = min(H, h0 + CHUNK)
            assert torch.equal(c[b, h0:h1], wc[0].repeat((h1 - h0) // POOL, 1, 1)), (b, h0)
            assert torch.equal(ex[b, h0:h1], we[0, :, 0].repeat((h1 - h0) // POOL)), (b, h0)
    print(f"fp8 codes B{B} H{H} N{N}: bit-exact over every head", flush=True)
    del x, codes, exps, c
    torch.cuda.empty_cache()
