"""fp64 CPU oracle for the FP8 forward with incoherent processing -- test
infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the HIP library never calls it and shares no code with
it.  Plain numpy, written from the pages and from the published definition of
the OCP FP8 E4M3 format.

Sources:
  [P1] "Interrogating the GPU, part 5: FlashAttention", section "What did
       FlashAttention-3 do with Hopper?": FP8 keys and values with one scale
       per block, preceded by a random orthogonal (Hadamard) mixing of the
       head dimension so that a few large features no longer set a whole
       block's scale; the page reports the error of that scheme against
       plain FP8 (a factor 2.6).
  [P2] "FlashAttention versions", section "FlashAttention-3": per-block
       scales with this "incoherent processing", contrasted with one scale
       per tensor.
  [P1] section "How can you softmax a row you never see whole?" and the
       FlashAttention-4 section (conditional rescale) for the online softmax.

Two functions compute the FP8 forward:
  * forward_reference follows only the pages and the readings below that the
    pages force (rotation, per-block E4M3, P in E4M3): no tiles, no stale
    maxima, P taken against each row's true maximum.  Tests compare the GPU's
    error against exact attention with this function's error, and check the
    pages' claim (the rotation lowers the error on outlier features) on GPU
    output against it.
  * forward_emulated additionally makes the choices of one tiled schedule
    (TILE keys per step, the conditional rescale with threshold TAU decided
    for WAVE_ROWS query rows at once, P scaled by 2^(8 - TAU) before its
    rounding), so that its E4M3 roundings of P fall where a kernel with that
    schedule rounds them; it is the tight parity check of such a kernel.
    These choices are readings of this oracle, not of the pages (which fix
    no tile size, threshold or scaling of P).

Readings adopted where the pages are silent:
  * the rotation is R = diag(sigma) H over the head dimension d = 128, with H
    the Sylvester Hadamard matrix (entries +-1, H H = d I) and sigma a random
    sign vector supplied by the caller; Q, K and V are all rotated:
    Q' = (Q o sigma) H, K' = (K o sigma) H, V' = (V o sigma) H, so that
    Q' K'^T = d Q K^T and O = ((P V') H / d) o sigma -- exact in real
    arithmetic; the rotation is computed in float32 as a fast Walsh-Hadamard
    transform, stage s = 0..6 pairing entries i and i + 2^s (bit s of i clear)
    into (a + b, a - b);
  * blocks are 64 consecutive rows of one head (the last block of a head may
    be shorter); a block's scale is the power of two 2^e with e the smallest
    integer such that amax <= 448 * 2^e (448 is E4M3's largest finite value),
    and its codes are E4M3(x * 2^-e) with round-to-nearest-even;
  * P enters the P V' product in E4M3 as well: P~ * 2^(8 - tau) is rounded to
    E4M3, with P~ = 2^(S log2 e - m) taken against the running reference
    maximum m; m follows the conditional rescale with threshold tau (log2
    units): when any row of a group of 32 query rows (one GPU wavefront) sees
    its tile maximum exceed m + tau, every row of the group moves m to
    max(m, tile maximum); the row sum l accumulates the unrounded P~.
"""
from __future__ import annotations

import numpy as np

__all__ = ["e4m3_decode", "e4m3_encode", "fwht32", "rotate", "block_exponent",
           "quantize_rows", "quantize_tensor", "forward_emulated", "forward_reference",
           "TAU", "TILE", "QBLOCK"]

TAU = 2.0        # conditional-rescale threshold (log2 units) of the FP8 path
TILE = 64        # keys per tile (and rows per quantisation block)
QBLOCK = 64      # rows per quantisation block
WAVE_ROWS = 32   # query rows that share one rescale decision
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """OCP FP8 E4M3 code (uint8) -> value: 1 sign bit, 4 exponent bits (bias 7),
    3 mantissa bits; exponent field 0 holds subnormals m/8 * 2^-6; the codes
    0x7F / 0xFF are NaN; there are no infinities."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """Round values with |x| <= 448 to the nearest E4M3 code, ties to even.

    Within a binade [2^E, 2^(E+1)) (E >= -6) the representable values are
    spaced 2^(E-3); below 2^-6 the subnormals are spaced 2^-9.  Rounding
    x / spacing to the nearest integer (ties to even) picks the code; an
    integer of 16 in a binade is the first value of the next one."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(a)) or np.any(a > E4M3_MAX):
        raise ValueError("E4M3 encoding needs finite |x| <= 448")
    with np.errstate(divide="ignore"):
        E = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    E = np.where(a > 0, np.maximum(E, -6.0), -6.0)  # zero lies in the subnormal range
    step = np.exp2(E - 3.0)
    n = np.rint(a / step)  # a / step is exact: step is a power of two
    # n in [0, 16]; n = 16 carries into the next binade
    carry = n >= 16
    E = np.where(carry, E + 1, E)
    n = np.where(carry, 8.0, n)
    sub = (E == -6) & (n < 8)
    exp_field = np.where(sub, 0, E + 7).astype(np.int64)
    mant = np.where(sub, n, n - 8).astype(np.int64)
    code = (exp_field << 3) | mant
    code = np.where(np.signbit(x), code | 0x80, code)
    return code.astype(np.uint8)


def fwht32(x):
    """Fast Walsh-Hadamard transform of the last axis (length 128) in float32.

    Stage s = 0..6 replaces each pair (x_i, x_{i + 2^s}), bit s of i clear, by
    (x_i + x_{i+2^s}, x_i - x_{i+2^s}).  The result is x H with H the Sylvester
    Hadamard matrix; every add is one IEEE float32 operation in this order."""
    y = np.array(x, dtype=np.float32, copy=True)
    n = y.shape[-1]
    s = 1
    while s < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * s), 2, s))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (n,))
        s *= 2
    return y


def rotate(x, signs):
    """x' = (x o sigma) H in float32 (x: bf16-exact values, any leading shape)."""
    x32 = np.asarray(x, dtype=np.float32)
    sg = np.asarray(signs, dtype=np.float32)
    return fwht32(x32 * sg)


def block_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (amax > 0); -127 for amax = 0.

    With amax = f 2^E, f in [0.5, 1), and 448 = 0.875 * 2^9: e = E - 9 when
    f <= 0.875 and E - 8 otherwise."""
    a = np.asarray(amax, dtype=np.float64)
    f, E = np.frexp(a)
    e = np.where(f > 0.875, E - 8, E - 9)
    return np.where(a > 0, e, -127).astype(np.int64)


def quantize_rows(y):
    """One block of rotated rows (float32, [rows, 128]) -> (E4M3 codes, e)."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)
    amax = np.max(np.abs(y)) if y.size else 0.0
    e = int(block_exponent(amax))
    return e4m3_encode(y * np.exp2(-e)), e


def quantize_tensor(x, signs, rotate_first=True):
    """[B, H, N, 128] -> codes [B, H, N, 128] (uint8), exponents [B, H, ceil(N/64)].

    rotate_first=False quantises the unrotated tensor (plain block FP8), used
    only to compare against incoherent processing."""
    x = np.asarray(x, dtype=np.float64)
    B, H, N, d = x.shape
    y = rotate(x, signs) if rotate_first else x.astype(np.float32)
    nb = (N + QBLOCK - 1) // QBLOCK
    codes = np.zeros((B, H, N, d), dtype=np.uint8)
    exps = np.zeros((B, H, nb), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for j in range(nb):
                r0, r1 = j * QBLOCK, min(N, (j + 1) * QBLOCK)
                c, e = quantize_rows(y[b, h, r0:r1])
                codes[b, h, r0:r1] = c
                exps[b, h, j] = e
    return codes, exps


def _dequant(codes, exps):
    B, H, N, d = codes.shape
    rows_e = np.repeat(exps, QBLOCK, axis=2)[:, :, :N]
    return e4m3_decode(codes) * np.exp2(rows_e)[..., None]


def forward_emulated(q, k, v, signs, scale, causal, quantize=True, rotate_first=True, tau=TAU):
    """The FP8 path in float64: rotate, quantise per block, online softmax with
    E4M3 P, un-rotate.  Returns (O, LSE) with LSE the natural log-sum-exp of
    the scaled scores the path computes.

    quantize=False skips every E4M3 rounding (Q', K', V' and P stay exact);
    the result is then exact attention, which ties this emulation to the
    plain oracle.  rotate_first=False quantises without the rotation."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if quantize:
        qc, qe = quantize_tensor(q, signs, rotate_first)
        kc, ke = quantize_tensor(k, signs, rotate_first)
        vc, ve = quantize_tensor(v, signs, rotate_first)
        qd, kd, vd = _dequant(qc, qe), _dequant(kc, ke), _dequant(vc, ve)
    elif rotate_first:
        sg = np.asarray(signs, dtype=np.float64)
        hm = fwht32(np.eye(d, dtype=np.float32)).astype(np.float64)  # H
        qd, kd, vd = (q * sg) @ hm, (k * sg) @ hm, (v * sg) @ hm
    else:
        qd, kd, vd = q, k, v
    gain = float(d) if rotate_first else 1.0   # Q' K'^T = d Q K^T
    sl2 = scale / gain * np.log2(np.e)         # log2-domain multiplier of Q' K'^T
    pscale = 2.0 ** (8 - tau)
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            rows = np.arange(N)
            for t0 in range(0, N, TILE):
                cols = np.arange(t0, min(N, t0 + TILE))
                s2 = sl2 * (qd[b, h] @ kd[b, h, cols].T)      # log2 units
                if causal:
                    s2[rows[:, None] < cols[None, :]] = -np.inf
                tmax = s2.max(axis=1)
                for g0 in range(0, N, WAVE_ROWS):
                    g = slice(g0, min(N, g0 + WAVE_ROWS))
                    if np.any(tmax[g] > m[g] + tau):
                        mnew = np.maximum(m[g], tmax[g])
                        alpha = np.where(np.isneginf(mnew), 1.0,
                                         np.exp2(m[g] - np.where(np.isneginf(mnew), 0.0, mnew)))
                        l[g] *= alpha
                        acc[g] *= alpha[:, None]
                        m[g] = mnew
                base = np.where(np.isneginf(m), 0.0, m)
                p = np.exp2(s2 - base[:, None])
                l += p.sum(axis=1)
                if quantize:
                    p8 = e4m3_decode(e4m3_encode(p * pscale)) / pscale
                else:
                    p8 = p
                acc += p8 @ vd[b, h, cols]
            op = acc / l[:, None]
            if rotate_first:
                sg = np.asarray(signs, dtype=np.float64)
                hm = fwht32(np.eye(d, dtype=np.float32)).astype(np.float64)
                o[b, h] = (op @ hm) / d * sg
            else:
                o[b, h] = op
            lse[b, h] = (m + np.log2(l)) * np.log(2.0)
    return o, lse


def forward_reference(q, k, v, signs, scale, causal, rotate_first=True, quantize=True,
                      row_block=1024):
    """FP8 attention as the pages describe it, with no schedule: rotate Q, K
    and V (unless rotate_first is False: plain per-block FP8), quantise each
    64-row block to E4M3, form every score of a row from the dequantised
    codes, take the softmax against the row's true maximum, round P times 2^8
    (so that the largest weight, 1, lands on the E4M3 value 256) to E4M3 for
    the P V' product, divide by the row sum of the unrounded weights, undo
    the rotation, and round O to bf16 as the GPU path stores it.

    quantize=False skips every E4M3 rounding and the bf16 rounding of O: the
    result is then exact attention.  Returns (O, LSE), LSE the natural
    log-sum-exp of the scores it forms."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    sg = np.asarray(signs, dtype=np.float64)
    hm = fwht32(np.eye(d, dtype=np.float32)).astype(np.float64)  # Sylvester H, H H = d I
    if quantize:
        qr, kr, vr = (_dequant(*quantize_tensor(x, signs, rotate_first)) for x in (q, k, v))
    elif rotate_first:
        qr, kr, vr = ((x * sg) @ hm for x in (q, k, v))
    else:
        qr, kr, vr = q, k, v
    # with the rotation, q'.k' = d q.k; the score multiplier takes the d out
    mult = scale / d if rotate_first else scale
    o = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    keys = np.arange(N)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, row_block):
                rows = np.arange(r0, min(N, r0 + row_block))
                s = mult * (qr[b, h, rows] @ kr[b, h].T)
                if causal:
                    s[rows[:, None] < keys[None, :]] = -np.inf
                m = s.max(axis=1)
                w = np.exp(s - m[:, None])
                denom = w.sum(axis=1)
                wq = e4m3_decode(e4m3_encode(w * 256.0)) * (1.0 / 256.0) if quantize else w
                out = (wq @ vr[b, h]) / denom[:, None]
                if rotate_first:
                    out = sg * (out @ hm) * (1.0 / d)  # (x H / d) o sigma undoes the rotation
                o[b, h, rows] = out
                lse[b, h, rows] = m + np.log(denom)
    if not quantize:
        return o, lse
    # round to bf16, nearest even, as the output is stored
    u = o.astype(np.float32).view(np.uint32).astype(np.uint64)
    r = (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32)
    return r.view(np.float32).astype(np.float64), lse
