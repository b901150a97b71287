"""Pins for the fp64 oracle, independent of the oracle's own formulas.

Each test checks the oracle against something the pages or the mathematics fix:
the pages' printed worked example, closed forms, invariants, central finite
differences, a pure-Python brute force on tiny inputs, and a library routine
(torch's CPU float64 scaled_dot_product_attention with autograd).
"""
import json
import math
import os

import numpy as np
import pytest

import fa_inputs
from oracle import attention as ora

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


# ---------------------------------------------------------------------------
# The worked example printed on the datarekha page (online vs full softmax)
# ---------------------------------------------------------------------------
def _page_example_inputs(meta):
    """The page's inputs: one query row, then K, then V, from one generator."""
    rng = np.random.default_rng(meta["seed"])
    N, d = meta["N"], meta["d"]
    Q = rng.standard_normal((1, d))
    K = rng.standard_normal((N, d))
    V = rng.standard_normal((N, d))
    return Q[None, None], K[None, None], V[None, None]


def test_worked_example_online_equals_full():
    """The page streams one query over eight keys in tiles of two and prints
    the largest difference between the tiled and the whole-row result.  The
    oracle's two forms, given the same single query row, reproduce that
    printed number exactly (it is one rounding of fp64, so any change in the
    order of the oracle's operations moves it), and both stay within the
    1e-12 acceptance bar of the online form."""
    meta = json.load(open(os.path.join(GOLD, "online_softmax_worked_example.json")))
    q, k, v = _page_example_inputs(meta)
    scale = 1.0 / math.sqrt(meta["d"])
    o_full, lse_full = ora.forward(q, k, v, scale, causal=False)
    o_onl, lse_onl = ora.online_forward(q, k, v, scale, causal=False, block=meta["tile"])
    diff = float(np.abs(o_full[0, 0, 0] - o_onl[0, 0, 0]).max())
    assert diff == meta["printed_max_abs_difference_full_vs_online"]
    assert diff <= 1e-12
    assert abs(lse_full[0, 0, 0] - lse_onl[0, 0, 0]) <= 1e-12


def test_cross_lengths_match_square_rows():
    """Fewer queries than keys (non-causal) gives exactly the rows of the
    square problem that share those queries."""
    rng = np.random.default_rng(11)
    q = rng.standard_normal((1, 2, 20, 8))
    k = rng.standard_normal((1, 2, 20, 8))
    v = rng.standard_normal((1, 2, 20, 8))
    o, lse = ora.forward(q, k, v, 0.3, False)
    o5, lse5 = ora.forward(q[:, :, 3:8], k, v, 0.3, False)
    assert np.abs(o5 - o[:, :, 3:8]).max() <= 1e-15
    assert np.abs(lse5 - lse[:, :, 3:8]).max() <= 1e-15
    with pytest.raises(ValueError):
        ora.forward(q[:, :, :5], k, v, 0.3, True)


@pytest.mark.parametrize("block", [1, 2, 3, 7, 16, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("descending", [False, True])
def test_online_equals_full_every_block(block, causal, descending):
    N, d = 150, 16
    q, k, v = (rand((1, 2, N, d), s) for s in (1, 2, 3))
    scale = 1 / math.sqrt(d)
    o_full, lse_full = ora.forward(q, k, v, scale, causal)
    o_onl, lse_onl = ora.online_forward(q, k, v, scale, causal, block, descending)
    assert np.isfinite(o_onl).all()
    assert np.abs(o_full - o_onl).max() <= 1e-12
    assert np.abs(lse_full - lse_onl).max() <= 1e-12


def test_online_descending_causal_needs_nan_guard():
    # Descending order with causal masking starts every low row with a block
    # of masked scores; the guard must keep those rows finite.
    N, d = 9, 4
    q, k, v = (rand((1, 1, N, d), s) for s in (4, 5, 6))
    o, lse = ora.online_forward(q, k, v, 0.5, True, block=2, descending=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all()


# ---------------------------------------------------------------------------
# Closed forms of the forward
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_constant_v_rows_give_that_row(causal):
    N, d = 40, 8
    q, k = rand((2, 2, N, d), 7), rand((2, 2, N, d), 8)
    row = rand((d,), 9)
    v = np.broadcast_to(row, (2, 2, N, d)).copy()
    o, _ = ora.forward(q, k, v, 0.3, causal)
    assert np.abs(o - row).max() <= 1e-12


def test_zero_q_gives_column_mean_noncausal():
    N, d = 33, 8
    q = np.zeros((1, 2, N, d))
    k, v = rand((1, 2, N, d), 10), rand((1, 2, N, d), 11)
    o, lse = ora.forward(q, k, v, 0.7, False)
    assert np.abs(o - v.mean(axis=2, keepdims=True)).max() <= 1e-12
    assert np.abs(lse - math.log(N)).max() <= 1e-12


def test_zero_q_gives_prefix_mean_causal():
    N, d = 33, 8
    q = np.zeros((1, 1, N, d))
    k, v = rand((1, 1, N, d), 12), rand((1, 1, N, d), 13)
    o, lse = ora.forward(q, k, v, 0.7, True)
    prefix = np.cumsum(v[0, 0], axis=0) / np.arange(1, N + 1)[:, None]
    assert np.abs(o[0, 0] - prefix).max() <= 1e-12
    assert np.abs(lse[0, 0] - np.log(np.arange(1, N + 1))).max() <= 1e-12


def test_dominant_score_selects_its_v_row():
    # K_j = c e_j, Q_i = c e_pi(i): score scale*c^2 on key pi(i), 0 elsewhere.
    N = d = 16
    c, scale = 10.0, 0.5  # margin = 50
    perm = np.random.default_rng(14).permutation(N)
    k = (c * np.eye(d))[None, None]
    q = (c * np.eye(d)[perm])[None, None]
    v = rand((1, 1, N, d), 15)
    o, lse = ora.forward(q, k, v, scale, False)
    margin = scale * c * c
    bound = 2 * (N - 1) * math.exp(-margin) * np.abs(v).max()
    assert np.abs(o[0, 0] - v[0, 0, perm]).max() <= max(bound, 1e-15)
    assert np.abs(lse[0, 0] - margin).max() <= 1e-12


def test_causal_row_zero():
    N, d = 20, 8
    q, k, v = (rand((1, 3, N, d), s) for s in (16, 17, 18))
    scale = 0.4
    o, lse = ora.forward(q, k, v, scale, True)
    assert np.abs(o[:, :, 0] - v[:, :, 0]).max() <= 1e-15
    assert np.abs(lse[:, :, 0] - scale * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1)).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_key_shift_invariance(causal):
    N, d = 30, 8
    q, k, v = (rand((1, 2, N, d), s) for s in (19, 20, 21))
    u = rand((d,), 22)
    scale = 0.35
    o1, l1 = ora.forward(q, k, v, scale, causal)
    o2, l2 = ora.forward(q, k + u, v, scale, causal)
    assert np.abs(o1 - o2).max() <= 1e-12
    assert np.abs((l2 - l1) - scale * (q @ u)).max() <= 1e-12


def test_permutation_noncausal():
    N, d = 25, 8
    q, k, v = (rand((1, 1, N, d), s) for s in (23, 24, 25))
    pk = np.random.default_rng(26).permutation(N)
    pq = np.random.default_rng(27).permutation(N)
    o, l = ora.forward(q, k, v, 0.5, False)
    o2, l2 = ora.forward(q[:, :, pq], k[:, :, pk], v[:, :, pk], 0.5, False)
    assert np.abs(o2 - o[:, :, pq]).max() <= 1e-12
    assert np.abs(l2 - l[:, :, pq]).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_lse_normalises_rows(causal):
    N, d = 37, 8
    q, k, v = (rand((1, 1, N, d), s, 3.0) for s in (28, 29, 30))
    scale = 0.5
    _, lse = ora.forward(q, k, v, scale, causal)
    s = scale * q[0, 0] @ k[0, 0].T
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    assert np.abs(np.exp(s - lse[0, 0][:, None]).sum(axis=1) - 1).max() <= 1e-14


def test_row_sample_matches_full_rows():
    N, d = 70, 16
    q, k, v = (rand((2, 2, N, d), s) for s in (31, 32, 33))
    o, lse = ora.forward(q, k, v, 0.25, True, row_block=16)
    rows = [0, 5, 17, 69]
    so, sl = ora.row_sample_forward(q, k, v, 0.25, True, 1, 0, rows)
    assert np.array_equal(so, o[1, 0, rows]) or np.abs(so - o[1, 0, rows]).max() <= 1e-15
    assert np.abs(sl - lse[1, 0, rows]).max() <= 1e-15


def test_row_block_does_not_change_result():
    N, d = 70, 8
    q, k, v = (rand((1, 1, N, d), s) for s in (34, 35, 36))
    a = ora.forward(q, k, v, 0.3, True, row_block=7)
    b = ora.forward(q, k, v, 0.3, True, row_block=4096)
    assert np.abs(a[0] - b[0]).max() <= 1e-15 and np.abs(a[1] - b[1]).max() <= 1e-15


# ---------------------------------------------------------------------------
# Brute force on tiny inputs (pure Python, scalar loops)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    N, d, scale = 4, 3, 0.8
    q, k, v = (rand((1, 1, N, d), s) for s in (37, 38, 39))
    o, lse = ora.forward(q, k, v, scale, causal)
    for i in range(N):
        keys = [j for j in range(N) if (not causal or j <= i)]
        w = {j: math.exp(scale * sum(q[0, 0, i, c] * k[0, 0, j, c] for c in range(d))) for j in keys}
        z = sum(w.values())
        for c in range(d):
            ref = sum(w[j] * v[0, 0, j, c] for j in keys) / z
            assert abs(o[0, 0, i, c] - ref) <= 1e-13
        assert abs(lse[0, 0, i] - math.log(z)) <= 1e-13


# ---------------------------------------------------------------------------
# Backward: central finite differences of loss = sum(O * dO)
# ---------------------------------------------------------------------------
def _loss(q, k, v, do, scale, causal):
    o, _ = ora.forward(q, k, v, scale, causal)
    return float(np.sum(o * do))


@pytest.mark.parametrize("N,d", [(1, 4), (2, 4), (3, 16), (5, 4), (8, 16), (16, 4), (16, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_finite_differences(N, d, causal):
    seed = 100 * N + d + int(causal)
    q, k, v, do = (rand((1, 2, N, d), seed + s) for s in range(4))
    scale = 1 / math.sqrt(d)
    o, _ = ora.forward(q, k, v, scale, causal)
    dq, dk, dv, _ = ora.backward(q, k, v, o, do, scale, causal)
    h = 1e-6
    rng = np.random.default_rng(seed)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        idx = list(np.ndindex(x.shape))
        if len(idx) > 48:
            idx = [idx[i] for i in rng.choice(len(idx), 48, replace=False)]
        for ix in idx:
            xp, xm = x.copy(), x.copy()
            xp[ix] += h
            xm[ix] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = {"q": q, "k": k, "v": v}
            args_p[name], args_m[name] = xp, xm
            fd = (_loss(args_p["q"], args_p["k"], args_p["v"], do, scale, causal)
                  - _loss(args_m["q"], args_m["k"], args_m["v"], do, scale, causal)) / (2 * h)
            assert abs(fd - g[ix]) <= 1e-7 + 1e-6 * abs(fd), (name, ix, fd, g[ix])


@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    N, d = 24, 8
    q, k, v, do = (rand((1, 2, N, d), s) for s in (40, 41, 42, 43))
    scale = 0.4
    o, lse = ora.forward(q, k, v, scale, causal)
    dq, dk, dv, D = ora.backward(q, k, v, o, do, scale, causal)
    # D equals sum_j P_ij dP_ij
    s = scale * q @ np.swapaxes(k, -1, -2)
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    p = np.exp(s - lse[..., None])
    dp = do @ np.swapaxes(v, -1, -2)
    assert np.abs(D - np.sum(p * dp, axis=-1)).max() <= 1e-12
    # column sums of dS vanish row-wise -> sum_j dK_j = 0
    assert np.abs(dk.sum(axis=2)).max() <= 1e-12
    # P rows sum to one -> sum_j dV_j = sum_i dO_i
    assert np.abs(dv.sum(axis=2) - do.sum(axis=2)).max() <= 1e-12


def test_backward_constant_v_has_no_q_k_gradient():
    N, d = 20, 8
    q, k, do = (rand((1, 1, N, d), s) for s in (44, 45, 46))
    v = np.broadcast_to(rand((d,), 47), (1, 1, N, d)).copy()
    o, _ = ora.forward(q, k, v, 0.5, True)
    dq, dk, dv, _ = ora.backward(q, k, v, o, do, 0.5, True)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_zero_q_dv_closed_form(causal):
    N, d = 18, 8
    q = np.zeros((1, 1, N, d))
    k, v, do = (rand((1, 1, N, d), s) for s in (48, 49, 50))
    o, _ = ora.forward(q, k, v, 0.5, causal)
    _, _, dv, _ = ora.backward(q, k, v, o, do, 0.5, causal)
    if causal:
        w = do[0, 0] / np.arange(1, N + 1)[:, None]
        ref = np.cumsum(w[::-1], axis=0)[::-1]  # dV_j = sum_{i >= j} dO_i / (i + 1)
    else:
        ref = np.broadcast_to(do[0, 0].mean(axis=0), (N, d))
    assert np.abs(dv[0, 0] - ref).max() <= 1e-12


# ---------------------------------------------------------------------------
# A library routine computing the same definition
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_against_torch_cpu_float64(causal):
    torch = pytest.importorskip("torch")
    N, d = 45, 16
    q, k, v, do = (rand((2, 3, N, d), s) for s in (51, 52, 53, 54))
    scale = 1 / math.sqrt(d)
    o, lse = ora.forward(q, k, v, scale, causal)
    dq, dk, dv, _ = ora.backward(q, k, v, o, do, scale, causal)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    to.backward(torch.tensor(do))
    assert np.abs(to.detach().numpy() - o).max() <= 1e-12
    for mine, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.abs(t.grad.numpy() - mine).max() <= 1e-12
    tl = torch.logsumexp(scale * tq.detach() @ tk.detach().transpose(-1, -2)
                         + (torch.triu(torch.full((N, N), -math.inf, dtype=torch.float64), 1) if causal else 0),
                         dim=-1)
    assert np.abs(tl.numpy() - lse).max() <= 1e-12


# ---------------------------------------------------------------------------
# Input generator: bf16 rounding is round-to-nearest-even
# ---------------------------------------------------------------------------
def test_bf16_rounding_rne():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(55).standard_normal(100000).astype(np.float32) * 7
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32) + 0x3F000000
    x = np.concatenate([x, ties.view(np.float32)])
    bits = fa_inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = fa_inputs.bf16_bits_to_f64(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).double().numpy())
