"""FLOP and byte accounting for the attention hot path (host-side arithmetic).

Conventions (the metric's): forward = 4 N^2 d per (batch, head), backward =
2.5x forward, both halved when causal.  Algorithmic bytes count what the
method itself must move through HBM -- Q, K, V read once, O and LSE written
once -- since the N x N scores never leave the chip and K/V re-reads are cache
hits ("Interrogating the GPU, part 5: FlashAttention", section "How does tiling
remove the traffic?").
"""
from __future__ import annotations

FP8 = 1
BF16 = 2
FP32 = 4


def fwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Two matmuls of 2 N^2 d each per head (S = Q K^T and O = P V)."""
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def bwd_flops(B: int, H: int, N: int, d: int, causal: bool) -> float:
    """Five matmuls per head: the recomputed S plus four gradient products
    ("Interrogating the GPU, part 5", backward section: about 2.5x forward)."""
    return 2.5 * fwd_flops(B, H, N, d, causal)


def fwd_bytes(B: int, H: int, N: int, d: int) -> float:
    """Read Q, K, V; write O (bf16) and LSE (fp32): 8 N d + 4 N per head."""
    return float(B * H * (4 * N * d * BF16 + N * FP32))


def bwd_bytes(B: int, H: int, N: int, d: int) -> float:
    """Read Q, K, V, O, dO, LSE; write dQ, dK, dV; write and read D:
    16 N d + 12 N bytes per head."""
    return float(B * H * (8 * N * d * BF16 + 3 * N * FP32))


def bwd_pre_bytes(B: int, H: int, N: int, d: int) -> float:
    """D = rowsum(dO * O) and L log2(e): read O, dO and L, write D and
    L log2(e): 4 N d + 12 N bytes per head."""
    return float(B * H * (2 * N * d * BF16 + 3 * N * FP32))


def fp8_quant_bytes(B: int, H: int, N: int, d: int) -> float:
    """Rotate and quantise one tensor: read it in bf16, write one E4M3 byte
    per element and one int32 exponent per 64-row block."""
    return float(B * H * (N * d * (BF16 + FP8) + -(-N // 64) * FP32))


def fp8_fwd_bytes(B: int, H: int, N: int, d: int) -> float:
    """FP8 attention: read the Q, K, V codes and their block exponents, write
    O (bf16) and LSE (fp32)."""
    return float(B * H * (3 * N * d * FP8 + 3 * -(-N // 64) * FP32 + N * d * BF16 + N * FP32))


def naive_intensity(N: int, d: int) -> float:
    """Textbook three-kernel attention: 4 N^2 d FLOPs over 8 N^2 + 8 N d bytes
    ("Interrogating the GPU, part 5", textbook section, intensity equation)."""
    return 4.0 * N * N * d / (8.0 * N * N + 8.0 * N * d)


def flash_intensity(N: int, d: int) -> float:
    """FLOPs over the 8 N d bytes of Q, K, V, O: N / 2."""
    return 4.0 * N * N * d / (8.0 * N * d)


# MI355X published peaks used as roofline denominators.
MI355X_BF16_DENSE_TFLOPS = 2516.6   # 256 CU x 4096 FLOP/clk x 2.4 GHz
MI355X_FP8_DENSE_TFLOPS = 5033.2    # 256 CU x 8192 FLOP/clk x 2.4 GHz
MI355X_HBM_GBPS = 8000.0
