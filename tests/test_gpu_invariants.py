"""GPU checks that need no oracle run: closed forms the mathematics fixes,
gradient identities, bitwise determinism, untouched guard bands, error paths
with real device tensors, and non-default streams.  All through the C ABI."""
import math

import numpy as np
import pytest

import fa_inputs
from tests.gpu_helpers import TOL_LSE, TOL_OUT, f64, from_dev, max_err, to_dev

pytestmark = pytest.mark.gpu
SCALE = fa_inputs.SCALE


@pytest.fixture(scope="module")
def fa():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_io_aware_10_amd as fa
    fa.load_library()
    return fa


def dev_bf16(a, torch):
    return to_dev(fa_inputs.f32_to_bf16_bits(np.asarray(a, np.float32)), torch)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 77, 1000])
def test_zero_q_uniform_attention(fa, causal, N):
    import torch
    x = fa_inputs.make(1, 2, N, seed=9100 + N)
    q = torch.zeros((1, 2, N, 128), dtype=torch.bfloat16, device="cuda")
    k, v = to_dev(x["k"], torch), to_dev(x["v"], torch)
    o, lse = fa.forward(q, k, v, SCALE, causal)
    torch.cuda.synchronize()
    V = f64(x["v"])
    if causal:
        ref = np.cumsum(V, axis=2) / np.arange(1, N + 1)[:, None]
        rl = np.broadcast_to(np.log(np.arange(1, N + 1)), (1, 2, N))
    else:
        ref = np.broadcast_to(V.mean(axis=2, keepdims=True), V.shape)
        rl = np.full((1, 2, N), math.log(N))
    assert max_err(from_dev(o), ref) <= TOL_OUT
    assert max_err(from_dev(lse), rl) <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_rows(fa, causal):
    import torch
    N = 700
    x = fa_inputs.make(1, 3, N, seed=9200)
    row = fa_inputs.bf16_bits_to_f64(fa_inputs.gaussian_bf16(9201, (128,)))
    v = dev_bf16(np.broadcast_to(row, (1, 3, N, 128)), torch)
    o, _ = fa.forward(to_dev(x["q"], torch), to_dev(x["k"], torch), v, SCALE, causal)
    torch.cuda.synchronize()
    assert max_err(from_dev(o), np.broadcast_to(row, (1, 3, N, 128))) <= TOL_OUT


def test_causal_row_zero(fa):
    import torch
    N = 513
    x = fa_inputs.make(2, 2, N, seed=9300)
    o, lse = fa.forward(*(to_dev(x[n], torch) for n in "qkv"), SCALE, True)
    torch.cuda.synchronize()
    Q, K, V = (f64(x[n]) for n in "qkv")
    assert max_err(from_dev(o)[:, :, 0], V[:, :, 0]) <= TOL_OUT
    assert max_err(from_dev(lse)[:, :, 0], SCALE * np.sum(Q[:, :, 0] * K[:, :, 0], -1)) <= TOL_LSE


def test_dominant_score_selects_row(fa):
    import torch
    N = 128
    c = 12.0  # bf16-exact; score margin scale * c^2 = 12.7
    perm = np.random.default_rng(9400).permutation(N)
    K = np.zeros((1, 1, N, 128))
    K[0, 0, np.arange(N), np.arange(N)] = c
    Q = np.zeros((1, 1, N, 128))
    Q[0, 0, np.arange(N), perm] = c
    x = fa_inputs.make(1, 1, N, seed=9401)
    o, _ = fa.forward(dev_bf16(Q, torch), dev_bf16(K, torch), to_dev(x["v"], torch), SCALE, False)
    torch.cuda.synchronize()
    V = f64(x["v"])
    margin = SCALE * c * c
    bound = 2 * (N - 1) * math.exp(-margin) * np.abs(V).max()
    assert max_err(from_dev(o)[0, 0], V[0, 0, perm]) <= bound + TOL_OUT


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(fa, causal):
    """K_j <- K_j + u for every key leaves O unchanged and moves LSE_i by
    scale q_i . u.  K is drawn on a 1/8 grid in [-4, 4] so K + u is exact in bf16."""
    import torch
    N = 640
    x = fa_inputs.make(1, 2, N, seed=9500)
    K = np.clip(np.round(8 * f64(x["k"])) / 8, -4, 4)
    u = np.zeros(128)
    u[3], u[77] = 0.5, -0.25
    q, v = to_dev(x["q"], torch), to_dev(x["v"], torch)
    k1, k2 = dev_bf16(K, torch), dev_bf16(K + u, torch)
    assert np.array_equal(from_dev(k2), K + u)
    o1, l1 = fa.forward(q, k1, v, SCALE, causal)
    o2, l2 = fa.forward(q, k2, v, SCALE, causal)
    torch.cuda.synchronize()
    shift = SCALE * (f64(x["q"]) @ u)
    assert max_err(from_dev(l2) - from_dev(l1), shift) <= 2 * TOL_LSE
    assert max_err(from_dev(o1), from_dev(o2)) <= TOL_OUT


@pytest.mark.parametrize("causal", [False, True])
def test_gradient_identities(fa, causal):
    import torch
    N = 1000
    x = fa_inputs.make(1, 2, N, seed=9600, with_do=True)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, SCALE, causal)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, SCALE, causal)
    torch.cuda.synchronize()
    DK, DV, DO = from_dev(dk), from_dev(dv), f64(x["do"])
    tol = TOL_OUT * math.sqrt(N)
    assert np.abs(DK.sum(axis=2)).max() <= tol
    assert np.abs(DV.sum(axis=2) - DO.sum(axis=2)).max() <= tol


def test_constant_v_gives_zero_qk_gradients(fa):
    import torch
    N = 600
    x = fa_inputs.make(1, 2, N, seed=9700, with_do=True)
    row = fa_inputs.bf16_bits_to_f64(fa_inputs.gaussian_bf16(9701, (128,)))
    v = dev_bf16(np.broadcast_to(row, (1, 2, N, 128)), torch)
    q, k, do = (to_dev(x[n], torch) for n in ("q", "k", "do"))
    o, lse = fa.forward(q, k, v, SCALE, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, SCALE, True)
    torch.cuda.synchronize()
    assert np.abs(from_dev(dq)).max() <= TOL_OUT
    assert np.abs(from_dev(dk)).max() <= TOL_OUT


@pytest.mark.parametrize("causal", [False, True])
def test_bitwise_deterministic(fa, causal):
    import torch
    N = 1100
    x = fa_inputs.make(2, 3, N, seed=9800, with_do=True)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    outs = []
    for _ in range(2):
        o, lse = fa.forward(q, k, v, SCALE, causal)
        dq, dk, dv = fa.backward(q, k, v, o, do, lse, SCALE, causal)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16).cpu().numpy() if t.dtype == torch.bfloat16
                     else t.view(torch.int32).cpu().numpy() for t in (o, lse, dq, dk, dv)])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
def test_outputs_stay_inside_their_buffers(fa, causal):
    """Guard bands around every output keep their sentinel bytes."""
    import torch
    B, H, N = 1, 2, 333
    n = B * H * N * 128
    pad = 4096
    x = fa_inputs.make(B, H, N, seed=9900, with_do=True)
    q, k, v, do = (to_dev(x[nm], torch) for nm in ("q", "k", "v", "do"))

    def guarded(count, dtype, fill):
        buf = torch.full((count + 2 * pad,), fill, dtype=dtype, device="cuda")
        return buf, buf[pad:pad + count]

    sent_bf = torch.tensor([-12345], dtype=torch.int16).view(torch.bfloat16).item()
    ob, o = guarded(n, torch.bfloat16, sent_bf)
    lb, lse = guarded(B * H * N, torch.float32, -7.25)
    o, lse = o.view(B, H, N, 128), lse.view(B, H, N)
    fa.fa_fwd(q, k, v, o, lse, SCALE, causal)
    grads = [guarded(n, torch.bfloat16, sent_bf) for _ in range(3)]
    wsz = fa.fa_bwd_workspace_size(B, H, N, 128, causal)
    wb, ws = guarded(wsz, torch.uint8, 0xA5)
    dq, dk, dv = (g[1].view(B, H, N, 128) for g in grads)
    fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, SCALE, causal, ws)
    torch.cuda.synchronize()
    for buf in [ob, lb, wb] + [g[0] for g in grads]:
        head, tail = buf[:pad], buf[-pad:]
        ref = buf[:1].clone().fill_(buf[0].item())
        assert torch.equal(head, ref.expand_as(head)) and torch.equal(tail, ref.expand_as(tail))
    assert torch.isfinite(o.float()).all() and torch.isfinite(dq.float()).all()


def test_non_default_stream(fa):
    import torch
    N = 500
    x = fa_inputs.make(1, 2, N, seed=9950)
    q, k, v = (to_dev(x[n], torch) for n in "qkv")
    ref_o, ref_l = fa.forward(q, k, v, SCALE, True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = fa.forward(q, k, v, SCALE, True, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


@pytest.mark.parametrize("entry", ["fa_fwd", "fa_fwd_split"])
def test_graph_replays_match_eager(fa, entry):
    """The forward captured in a HIP graph (as bench.py times the forward-only
    workloads): every replay, with eager work and synchronisations between
    them, equals the eager result bit for bit (the kernels are deterministic)."""
    import torch
    B, H, N = 2, 128, 300  # fa_fwd takes the row-block kernel at this size
    x = fa_inputs.make(B, H, N, seed=9960)
    q, k, v = (to_dev(x[n], torch) for n in "qkv")
    run = getattr(fa, entry)
    ref_o, ref_l = torch.empty_like(q), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    run(q, k, v, ref_o, ref_l, SCALE, True)
    o, lse = torch.empty_like(q), torch.empty_like(ref_l)
    graph = torch.cuda.CUDAGraph()
    gs = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(gs):
        with torch.cuda.graph(graph, stream=gs):
            run(q, k, v, o, lse, SCALE, True)
    for i in range(3):
        o.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        run(q, k, v, ref_o, ref_l, SCALE, True)  # eager work between the replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(1, 3, 300), (2, 16, 4096)])
def test_staged_backward_equals_fa_bwd(fa, shape):
    """fa_bwd_dq -> fa_bwd_dkdv (the calls bench.py times) give exactly fa_bwd's
    gradients; fa_bwd_preprocess writes the workspace bit for bit as
    fa_bwd_dq does, so preprocess -> dkdv -> dq gives them too (every path
    is deterministic)."""
    import torch
    B, H, N = shape
    x = fa_inputs.make(B, H, N, seed=9970 + N, with_do=True)
    q, k, v, do = (to_dev(x[n], torch) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, SCALE, True)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, SCALE, True)
    ws = fa.workspace_for(B, H, N, True, q.device)
    ws2 = fa.workspace_for(B, H, N, True, q.device)
    rows = B * H * N
    dq2, dk2, dv2 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    fa.fa_bwd_dq(q, k, v, o, do, lse, ws, dq2, SCALE, True)
    fa.fa_bwd_dkdv(q, k, v, do, ws, dk2, dv2, SCALE, True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    dq3, dk3, dv3 = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    fa.fa_bwd_preprocess(o, do, lse, ws2)
    torch.cuda.synchronize()
    assert torch.equal(ws2[: 8 * rows], ws[: 8 * rows])
    fa.fa_bwd_dkdv(q, k, v, do, ws2, dk3, dv3, SCALE, True)
    fa.fa_bwd_dq(q, k, v, o, do, lse, ws2, dq3, SCALE, True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq3) and torch.equal(dk, dk3) and torch.equal(dv, dv3)


def test_error_paths_with_device_tensors(fa):
    import torch
    N = 64
    x = fa_inputs.make(1, 1, N, seed=9990)
    q, k, v = (to_dev(x[n], torch) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((1, 1, N), dtype=torch.float32, device="cuda")
    lib = fa.load_library()
    p = lambda t: t.data_ptr()  # noqa: E731
    assert lib.fa_fwd(p(q) + 2, p(k), p(v), p(o), p(lse), 1, 1, N, 128, SCALE, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fwd(p(q), p(k), p(v), p(o), p(lse), 1, 1, N, 64, SCALE, 0, None) == fa.FA_ERR_UNSUPPORTED
    assert lib.fa_fwd(p(q), p(k), p(v), p(o), p(lse), 1, 1, N, 128, float("nan"), 0, None) == fa.FA_ERR_INVALID_ARG
    assert lib.fa_fwd(p(q), p(k), p(v), p(o), p(lse), 1, 1, N, 128, SCALE, 3, None) == fa.FA_ERR_INVALID_ARG
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FAError) as ei:
        fa.fa_bwd(q, k, v, o, q, lse, o, o, o, SCALE, False, ws)
    assert ei.value.status == fa.FA_ERR_WORKSPACE
    # Empty problem: nothing launched, success.
    assert lib.fa_fwd(None, None, None, None, None, 1, 1, 0, 128, SCALE, 0, None) == fa.FA_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [100, 1000])
def test_tail_reads_stay_inside_each_head(fa, causal, N):
    """Rows past N of a head must read as zero, never as the next head's rows
    or memory past the tensor: fill head 1 and a tail guard band with NaN and
    check that head 0 (forward and backward) is finite and matches the same
    problem run on its own."""
    import torch
    x = fa_inputs.make(1, 1, N, seed=9970 + N, with_do=True)
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16)
    t = {}
    for nm in ("q", "k", "v", "do"):
        buf = torch.full((1, 3, N, 128), nan, dtype=torch.bfloat16, device="cuda")
        buf[:, 0] = to_dev(x[nm], torch)[:, 0]
        t[nm] = buf[:, :2]  # head 1 and the third (guard) head hold NaN
    # Views of the first two heads of 3-head buffers: contiguous, with a NaN
    # guard head right after them in memory.
    q2, k2, v2, do2 = (t[nm] for nm in ("q", "k", "v", "do"))
    assert q2.is_contiguous()
    o2, l2 = fa.forward(q2, k2, v2, SCALE, causal)
    q1, k1, v1, do1 = (to_dev(x[nm], torch) for nm in ("q", "k", "v", "do"))
    o1, l1 = fa.forward(q1, k1, v1, SCALE, causal)
    g1 = fa.backward(q1, k1, v1, o1, do1, l1, SCALE, causal)
    o2h = o2[:, :1].contiguous()
    l2h = l2[:, :1].contiguous()
    torch.cuda.synchronize()
    assert torch.equal(o2h, o1) and torch.equal(l2h, l1)
    # backward of head 0 with NaN neighbours: only head 0's rows are inputs to it
    o2[:, 1] = 0
    l2[:, 1] = 0
    g2 = fa.backward(q2, k2, v2, o2, do2, l2, SCALE, causal)
    torch.cuda.synchronize()
    for a, b in zip(g2, g1):
        assert torch.equal(a[:, :1].contiguous(), b)
