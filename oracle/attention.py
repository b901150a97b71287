"""fp64 CPU oracle for exact softmax attention -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
calls it, and it shares no code with that path: it is plain numpy float64 on
the CPU, written from the definitions on the pages, with S and P materialised.

Sources (cited by page title and section):
  [P1] "Interrogating the GPU, part 5: FlashAttention" (vaibhav016.github.io)
  [P2] "FlashAttention versions" (worksonmygpu.com)
  [P3] "FlashAttention" (datarekha.com)
  [P4] "LLM flash attention" (aicassindra.com)

Readings adopted where the pages are silent or ambiguous:
  * the softmax is taken over scale * Q K^T, with `scale` a caller argument
    (P1's textbook section writes S = Q K^T; P4's end-to-end flow divides by
    sqrt(d));
  * the saved statistic is the natural log-sum-exp of the *scaled* scores,
    L_i = m_i + ln(l_i), so that P_ij = exp(S_ij - L_i) (P1, backward section);
  * causal masking keeps key j only when j <= query i (equal lengths);
  * delta in dS = P o (dP - delta) is D_i = sum_k dO_ik O_ik, the row sum of
    dO o O, which equals sum_j P_ij dP_ij when O is exact;
  * dQ = scale * dS K and dK = scale * dS^T Q follow from the chain rule
    (the pages state only dV and dS).

Parity: every function here is pinned by tests that do not use this module's
own formulas (closed forms, invariants, finite differences, the pages'
worked example, a pure-Python brute force and a library routine).
"""
from __future__ import annotations

import numpy as np

__all__ = ["forward", "backward", "online_forward", "row_sample_forward"]


def _check(q, k, v, causal):
    """q [B, H, Nq, d], k and v [B, H, Nk, d].  Nq may differ from Nk only
    without the causal mask (a query row attends to every key, as in [P3]'s
    worked example, which streams one query over eight keys); the causal mask
    is defined for equal lengths."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if q.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if causal and q.shape[2] != k.shape[2]:
        raise ValueError("the causal mask needs as many queries as keys")
    return q, k, v


def _head_scores(qh, kh, scale, causal, rows):
    """S = scale * Q K^T for the given query rows of one head; masked -> -inf.

    [P1] "Why is the textbook algorithm memory-bound?" (S = Q K^T);
    [P4] "End-to-end flow" (division by sqrt(d), causal skipping of the future).
    """
    s = scale * (qh[rows] @ kh.T)
    if causal:
        keys = np.arange(kh.shape[0])
        s[rows[:, None] < keys[None, :]] = -np.inf
    return s


def forward(q, k, v, scale, causal, row_block=2048):
    """Plain softmax attention: O = softmax(scale Q K^T) V and LSE per row.

    For each (batch, head) and each query row, the whole row of scores is
    materialised, its maximum m subtracted before exponentiating, the row sum
    l formed, P = E / l, O = P V, and LSE = m + ln l.
    [P1] "Why is the textbook algorithm memory-bound?" (S, P, O);
    [P1] "What does the backward pass do without P?" (L_i = m_i + log l_i).
    Rows are independent, so they are processed `row_block` at a time only to
    bound memory; no sum is split.

    Returns (O [B,H,Nq,d] float64, LSE [B,H,Nq] float64).
    """
    q, k, v = _check(q, k, v, causal)
    B, H, N, d = q.shape
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                s = _head_scores(q[b, h], k[b, h], scale, causal, rows)
                m = s.max(axis=1)
                e = np.exp(s - m[:, None])
                l = e.sum(axis=1)
                p = e / l[:, None]
                o[b, h, rows] = p @ v[b, h]
                lse[b, h, rows] = m + np.log(l)
    return o, lse


def row_sample_forward(q, k, v, scale, causal, b, h, rows):
    """`forward` restricted to the listed query rows of head (b, h).

    The definition is per row, so a sample of rows is computed exactly as the
    full forward computes them.  Returns (O [len(rows), d], LSE [len(rows)]).
    """
    qh = np.asarray(q[b, h], dtype=np.float64)
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    s = _head_scores(qh, kh, scale, causal, rows)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return (e / l[:, None]) @ vh, m + np.log(l)


def backward(q, k, v, o, do, scale, causal):
    """Gradients of attention by the chain rule, with P materialised.

    [P1] "What does the backward pass do without P?": dV = P^T dO and
    dS = P o (dP - delta); here dP = dO V^T, delta_i = D_i = sum_k dO_ik O_ik,
    and the chain rule through S = scale Q K^T gives dQ = scale dS K,
    dK = scale dS^T Q.  Masked scores have P = 0 and hence dS = 0.
    `o` is the forward output used for D (the oracle's own fp64 O in parity
    tests).

    Returns (dQ, dK, dV [B,H,N,d], D [B,H,N]) in float64.
    """
    q, k, v = _check(q, k, v, causal)
    if q.shape != k.shape:
        raise ValueError("the backward takes as many queries as keys")
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, d = q.shape
    dq = np.empty_like(q)
    dk = np.empty_like(q)
    dv = np.empty_like(q)
    dD = np.empty((B, H, N), dtype=np.float64)
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            s = _head_scores(q[b, h], k[b, h], scale, causal, rows)
            m = s.max(axis=1)
            e = np.exp(s - m[:, None])
            p = e / e.sum(axis=1)[:, None]
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            D = np.sum(do[b, h] * o[b, h], axis=1)
            ds = p * (dp - D[:, None])
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
            dD[b, h] = D
    return dq, dk, dv, dD


def online_forward(q, k, v, scale, causal, block, descending=False):
    """The streaming (online) softmax, used only to check `forward`.

    Keys are visited `block` at a time.  Per query row the state is the running
    maximum m, the running sum l = sum e^(s - m) and the unnormalised output
    acc = sum e^(s - m) v.  A block with new maximum m' rescales the old state
    by e^(m - m') before adding its own terms taken relative to m'; at the end
    O = acc / l and LSE = m + ln l.
    [P1] "How can you softmax a row you never see whole?" (the update rule);
    [P2] "FlashAttention (2022)" (one streaming step);
    [P3] "The online softmax -- why it's exact" (worked example);
    [P4] "End-to-end flow" (m starts at -inf, l and the accumulator at 0).
    When every score seen so far is masked (m' = -inf) the subtraction base is
    taken as 0 so that e^(-inf - (-inf)) never forms a NaN.
    """
    q, k, v = _check(q, k, v, causal)
    B, H, N, d = q.shape
    Nk = k.shape[2]
    o = np.empty_like(q)
    lse = np.empty((B, H, N), dtype=np.float64)
    starts = list(range(0, Nk, block))
    if descending:
        starts.reverse()
    rows = np.arange(N)
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for t0 in starts:
                cols = np.arange(t0, min(Nk, t0 + block))
                s = scale * (q[b, h] @ k[b, h, cols].T)
                if causal:
                    s[rows[:, None] < cols[None, :]] = -np.inf
                m_new = np.maximum(m, s.max(axis=1))
                base = np.where(np.isneginf(m_new), 0.0, m_new)
                alpha = np.exp(m - base)
                p = np.exp(s - base[:, None])
                l = l * alpha + p.sum(axis=1)
                acc = acc * alpha[:, None] + p @ v[b, h, cols]
                m = m_new
            o[b, h] = acc / l[:, None]
            lse[b, h] = m + np.log(l)
    return o, lse
