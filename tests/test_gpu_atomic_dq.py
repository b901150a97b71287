"""fa_bwd_atomic_dq: the backward with dQ fused into the dK/dV pass through
fp32 atomics ("LLM flash attention", section "End-to-end flow").  Gradients
against the fp64 oracle at the usual tolerances (tails, both masks, other
scales, whole heads of B2 H16 N4096) and against fa_bwd; dK and dV repeat
bit for bit from run to run, dQ (summed in the order the atomics land) only
to within rounding."""
import numpy as np
import pytest

import fa_inputs
from oracle import attention as ora
from tests.gpu_helpers import TOL_OUT, f64, from_dev, map_heads, max_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_10_amd as fa
    fa.load_library()
    return fa


def _grads(fa, x, B, H, N, scale, causal, atomic):
    import torch
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, scale, causal)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if atomic:
        ws = torch.empty(max(fa.fa_bwd_atomic_workspace_size(B, H, N, 128, causal), 16), dtype=torch.uint8,
                         device=q.device)
        fa.fa_bwd_atomic_dq(q, k, v, o, do, lse, dq, dk, dv, scale, causal, ws)
    else:
        fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal, fa.workspace_for(B, H, N, causal, q.device))
    torch.cuda.synchronize()
    return dq, dk, dv


def _oracle(x, scale, causal, sl=None):
    sl = sl or (slice(None), slice(None))
    Q, K, V, DO = (f64(x[n][sl]) for n in ("q", "k", "v", "do"))
    ro, _ = ora.forward(Q, K, V, scale, causal)
    rdq, rdk, rdv, _ = ora.backward(Q, K, V, ro, DO, scale, causal)
    return rdq, rdk, rdv


@pytest.mark.parametrize("N", [1, 2, 31, 32, 33, 127, 128, 129, 300, 1000])
@pytest.mark.parametrize("causal", [False, True])
def test_small_against_oracle(fa, N, causal):
    B, H = 1, 2
    x = fa_inputs.make(B, H, N, seed=8900 + N + 7 * causal, with_do=True)
    scale = fa_inputs.SCALE
    got = [from_dev(t) for t in _grads(fa, x, B, H, N, scale, causal, True)]
    ref = _oracle(x, scale, causal)
    e = [max_err(g, r) for g, r in zip(got, ref)]
    print(f"atomic dQ N={N} causal={causal}: dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}", flush=True)
    assert max(e) <= TOL_OUT


@pytest.mark.parametrize("scale", [0.0, -fa_inputs.SCALE])
@pytest.mark.parametrize("causal", [False, True])
def test_other_scales(fa, scale, causal):
    B, H, N = 1, 2, 300
    x = fa_inputs.make(B, H, N, seed=9000 + causal, with_do=True)
    got = [from_dev(t) for t in _grads(fa, x, B, H, N, scale, causal, True)]
    ref = _oracle(x, scale, causal)
    e = [max_err(g, r) for g, r in zip(got, ref)]
    print(f"atomic dQ scale {scale:+.4f} causal={causal}: dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}", flush=True)
    assert max(e) <= TOL_OUT
    if scale == 0.0:
        assert not np.any(got[0]) and not np.any(got[1])  # dQ = dK = 0 exactly


def test_b2_h16_n4096_causal(fa):
    """Four whole heads against the oracle; every head against fa_bwd; dK and
    dV bitwise repeatable, dQ repeatable to within rounding."""
    import torch
    name = "causal_b2_h16_n4096"
    w = fa_inputs.WORKLOADS[name]
    B, H, N = w["B"], w["H"], w["N"]
    x = fa_inputs.make_workload(name, with_do=True)
    scale = fa_inputs.SCALE
    a1 = _grads(fa, x, B, H, N, scale, True, True)
    a2 = _grads(fa, x, B, H, N, scale, True, True)
    ref = _grads(fa, x, B, H, N, scale, True, False)
    assert torch.equal(a1[1].view(torch.int16), a2[1].view(torch.int16))
    assert torch.equal(a1[2].view(torch.int16), a2[2].view(torch.int16))
    rep = float((a1[0].float() - a2[0].float()).abs().max())
    vs_bwd = [float((a.float() - r.float()).abs().max()) for a, r in zip(a1, ref)]
    G = [from_dev(t) for t in a1]

    def one(bh):
        b, hh = bh
        sl = (slice(b, b + 1), slice(hh, hh + 1))
        r = _oracle(x, scale, True, sl)
        return [max_err(g[sl], rr) for g, rr in zip(G, r)]

    errs = np.array(map_heads(one, [(0, 0), (0, 7), (1, 8), (1, 15)], "atomic dQ heads", workers=4))
    print(f"atomic dQ B2 H16 N4096: vs oracle (4 heads) dQ {errs[:, 0].max():.2e} dK {errs[:, 1].max():.2e} "
          f"dV {errs[:, 2].max():.2e}; vs fa_bwd dQ {vs_bwd[0]:.2e} dK {vs_bwd[1]:.2e} dV {vs_bwd[2]:.2e}; "
          f"dQ run to run {rep:.2e}", flush=True)
    assert errs.max() <= TOL_OUT and max(vs_bwd) <= TOL_OUT and rep <= 1e-2
