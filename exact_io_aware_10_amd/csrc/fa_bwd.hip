// Backward kernels: gradients of exact attention with P recomputed on chip.
//
// "Interrogating the GPU, part 5: FlashAttention", section "What does the
// backward pass do without P?": only L_i = m_i + ln l_i is kept, and each
// tile of P is rebuilt as exp(S_ij - L_i) from Q, K and L; dV = P^T dO and
// dS = P o (dP - delta).  Here dP = dO V^T, delta_i = D_i = sum_k dO_ik O_ik
// (computed once by a pre-pass), and the chain rule through S = scale Q K^T
// gives dQ = scale dS K and dK = scale dS^T Q ("LLM flash attention",
// section "End-to-end flow": recompute each block's weights, then its
// contribution to the Q, K and V gradients).
//
// Three launches, no atomics (bitwise deterministic):
//   bwd_pre   D = rowsum(dO o O)                       streaming, HBM-bound
//   bwd_dkdv  per key block: K, V held in registers; query tiles of Q, dO,
//             L, D stream through LDS; dV^T += dO^T P and dK^T += Q^T dS
//   bwd_dq    per query block: Q, dO, L, D held in registers; K, V tiles
//             stream through LDS; dQ^T += K^T dS^T
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik: 16 threads per row, 8 elements (16 bytes) each.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta, int rows) {
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid >> 4;
  const int part = gid & 15;
  float s = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * kD + part * 8;
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + off);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dO + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a0 = __uint_as_float(a[j] << 16), a1 = __uint_as_float(a[j] & 0xffff0000u);
      const float b0 = __uint_as_float(b[j] << 16), b1 = __uint_as_float(b[j] & 0xffff0000u);
      s = __builtin_fmaf(a0, b0, s);
      s = __builtin_fmaf(a1, b1, s);
    }
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) s += __shfl_xor(s, w, 16);
  if (row < rows && part == 0) delta[row] = s;
}

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
constexpr int KV_BK = 128;               // keys per workgroup
constexpr int KV_WAVES = 4;              // 32 keys per wave
constexpr int KV_BQ = 64;                // queries per streamed tile
constexpr int KV_TILE = KV_BQ * kRowBytes;  // 16 KiB (Q or dO)
constexpr int KV_STAGE = 2 * KV_TILE + 2 * KV_BQ * 4;  // Q, dO, L*log2e, D
constexpr int KV_THREADS = KV_WAVES * 64;
constexpr int KV_LOADS = KV_TILE / 16 / KV_THREADS;

template <bool CAUSAL>
__global__ __launch_bounds__(KV_THREADS) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int BH, int N, float sl2, float scale) {
  __shared__ __attribute__((aligned(16))) char smem[2 * KV_STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // Causal: the first key blocks see the most queries; issue them first.
  const int id = blockIdx.x;
  const int kb = id / BH;
  const int bh = id % BH;
  const int k0 = kb * KV_BK;
  const int kw = k0 + wave * 32;
  const int krow = kw + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const char* qh = reinterpret_cast<const char*>(q + head);
  const char* kh = reinterpret_cast<const char*>(k + head);
  const char* vh = reinterpret_cast<const char*>(v + head);
  const char* doh = reinterpret_cast<const char*>(dO + head);
  const float* lseh = lse + (size_t)bh * N;
  const float* dh = delta + (size_t)bh * N;

  // K^T and V^T as B operands: lane holds row krow, dims 16 kc + 8 h .. + 7.
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    const size_t off = (size_t)krow * kRowBytes + (2 * kc + h) * 16;
    kf[kc] = __builtin_bit_cast(bf16x8, load16_or_zero(kh + off, krow < N));
    vf[kc] = __builtin_bit_cast(bf16x8, load16_or_zero(vh + off, krow < N));
  }

  const int t0 = CAUSAL ? (k0 / KV_BQ) : 0;
  const int ntiles = (N + KV_BQ - 1) / KV_BQ;

  const int ld_row = tid >> 4;
  const int ld_chunk = tid & 15;
  u32x4 qr[KV_LOADS], dr[KV_LOADS];
  float lr = 0.f, drr = 0.f;
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < KV_LOADS; ++i) {
      const int qi = t * KV_BQ + ld_row + 16 * i;
      const size_t off = (size_t)qi * kRowBytes + ld_chunk * 16;
      qr[i] = load16_or_zero(qh + off, qi < N);
      dr[i] = load16_or_zero(doh + off, qi < N);
    }
    if (tid < KV_BQ) {
      const int qi = t * KV_BQ + tid;
      // Rows past N get L = +inf, hence P = 0: they contribute nothing.
      lr = qi < N ? lseh[qi] * kLog2e : INFINITY;
      drr = qi < N ? dh[qi] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
    char* base = smem + buf * KV_STAGE;
#pragma unroll
    for (int i = 0; i < KV_LOADS; ++i) {
      const int off = tile_off(ld_row + 16 * i, ld_chunk);
      lds_write16(base, off, qr[i]);
      lds_write16(base + KV_TILE, off, dr[i]);
    }
    if (tid < KV_BQ) {
      reinterpret_cast<float*>(base + 2 * KV_TILE)[tid] = lr;
      reinterpret_cast<float*>(base + 2 * KV_TILE + KV_BQ * 4)[tid] = drr;
    }
  };

  f32x16 dka[4], dva[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dka[mb][i] = 0.f;
      dva[mb][i] = 0.f;
    }

  const int tr_s = lane & 15;
  const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
  const int tr_row = 4 * h + (tr_s >> 2);

  if (t0 < ntiles) {
    gload(t0);
    swrite(0);
  }
  __syncthreads();

  for (int t = t0; t < ntiles; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const char* qb = smem + buf * KV_STAGE;
    const char* dob = qb + KV_TILE;
    const float* lsb = reinterpret_cast<const float*>(qb + 2 * KV_TILE);
    const float* dsb = lsb + KV_BQ;
#pragma unroll
    for (int sub = 0; sub < KV_BQ / 32; ++sub) {
      const int qs = t * KV_BQ + 32 * sub;
      const bool active = !CAUSAL || (qs + 31 >= kw);
      if (!active) continue;
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const int off = tile_off(32 * sub + col, 2 * kc + h);
        s = mfma32(__builtin_bit_cast(bf16x8, lds_read16(qb, off)), kf[kc], s);
        dp = mfma32(__builtin_bit_cast(bf16x8, lds_read16(dob, off)), vf[kc], dp);
      }
      const bool need_mask = CAUSAL && (qs < kw + 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = 32 * sub + 8 * g + 4 * h;  // tile-local query row of element 4g
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lsb + r);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dsb + r);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = 4 * g + j;
          float p = fast_exp2(__builtin_fmaf(s[i], sl2, -l4[j]));
          if (need_mask && krow > t * KV_BQ + r + j) p = 0.f;
          s[i] = p;
          dp[i] = p * (dp[i] - d4[j]);
        }
      }
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = 8 * u;
        pb[u] = pack8(s[b], s[b + 1], s[b + 2], s[b + 3], s[b + 4], s[b + 5], s[b + 6], s[b + 7]);
        sb[u] = pack8(dp[b], dp[b + 1], dp[b + 2], dp[b + 3], dp[b + 4], dp[b + 5], dp[b + 6],
                      dp[b + 7]);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int dim = 32 * mb + tr_dim;
        const int chunk = dim >> 3;
        const int half = (dim >> 2) & 1;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 32 * sub + 16 * u + tr_row;
          const bf16x8 a_do = join(lds_read_tr(dob + tile_off8(r, chunk, half)),
                                   lds_read_tr(dob + tile_off8(r + 8, chunk, half)));
          dva[mb] = mfma32(a_do, pb[u], dva[mb]);
          const bf16x8 a_q = join(lds_read_tr(qb + tile_off8(r, chunk, half)),
                                  lds_read_tr(qb + tile_off8(r + 8, chunk, half)));
          dka[mb] = mfma32(a_q, sb[u], dka[mb]);
        }
      }
    }
    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  if (krow < N) {
    char* dkrow = reinterpret_cast<char*>(dk + head) + (size_t)krow * kRowBytes;
    char* dvrow = reinterpret_cast<char*>(dv + head) + (size_t)krow * kRowBytes;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = 4 * g;
        const int off = (32 * mb + 8 * g + 4 * h) * 2;
        u32x2 wk = {pack_bf16(dka[mb][i] * scale, dka[mb][i + 1] * scale),
                    pack_bf16(dka[mb][i + 2] * scale, dka[mb][i + 3] * scale)};
        u32x2 wv = {pack_bf16(dva[mb][i], dva[mb][i + 1]), pack_bf16(dva[mb][i + 2], dva[mb][i + 3])};
        *reinterpret_cast<u32x2*>(dkrow + off) = wk;
        *reinterpret_cast<u32x2*>(dvrow + off) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int DQ_BQ = 128;   // queries per workgroup
constexpr int DQ_WAVES = 4;  // 32 queries per wave
constexpr int DQ_BC = 64;    // keys per streamed tile
constexpr int DQ_TILE = DQ_BC * kRowBytes;
constexpr int DQ_THREADS = DQ_WAVES * 64;
constexpr int DQ_LOADS = DQ_TILE / 16 / DQ_THREADS;

template <bool CAUSAL>
__global__ __launch_bounds__(DQ_THREADS) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ delta,
    uint16_t* __restrict__ dq, int BH, int N, int nqb, float sl2, float scale) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * DQ_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  const int id = blockIdx.x;
  const int qblk = CAUSAL ? (nqb - 1 - id / BH) : (id / BH);
  const int bh = id % BH;
  const int q0 = qblk * DQ_BQ;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const char* qh = reinterpret_cast<const char*>(q + head);
  const char* kh = reinterpret_cast<const char*>(k + head);
  const char* vh = reinterpret_cast<const char*>(v + head);
  const char* doh = reinterpret_cast<const char*>(dO + head);

  bf16x8 qf[8], df[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    const size_t off = (size_t)qrow * kRowBytes + (2 * kc + h) * 16;
    qf[kc] = __builtin_bit_cast(bf16x8, load16_or_zero(qh + off, qrow < N));
    df[kc] = __builtin_bit_cast(bf16x8, load16_or_zero(doh + off, qrow < N));
  }
  const float l2 = qrow < N ? lse[(size_t)bh * N + qrow] * kLog2e : INFINITY;
  const float Dq = qrow < N ? delta[(size_t)bh * N + qrow] : 0.f;

  const int kend = CAUSAL ? min(N, q0 + DQ_BQ) : N;
  const int ntiles = (kend + DQ_BC - 1) / DQ_BC;

  const int ld_row = tid >> 4;
  const int ld_chunk = tid & 15;
  u32x4 kr[DQ_LOADS], vr[DQ_LOADS];
  auto gload = [&](int t) {
#pragma unroll
    for (int i = 0; i < DQ_LOADS; ++i) {
      const int key = t * DQ_BC + ld_row + 16 * i;
      const size_t off = (size_t)key * kRowBytes + ld_chunk * 16;
      kr[i] = load16_or_zero(kh + off, key < N);
      vr[i] = load16_or_zero(vh + off, key < N);
    }
  };
  auto swrite = [&](int buf) {
    char* kb = smem + buf * 2 * DQ_TILE;
    char* vb = kb + DQ_TILE;
#pragma unroll
    for (int i = 0; i < DQ_LOADS; ++i) {
      const int off = tile_off(ld_row + 16 * i, ld_chunk);
      lds_write16(kb, off, kr[i]);
      lds_write16(vb, off, vr[i]);
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;

  const int tr_s = lane & 15;
  const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
  const int tr_row = 4 * h + (tr_s >> 2);

  gload(0);
  swrite(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int k0 = t * DQ_BC;
    const bool active = !CAUSAL || (k0 <= q0w + 31);
    if (active) {
      const char* kb = smem + buf * 2 * DQ_TILE;
      const char* vb = kb + DQ_TILE;
      f32x16 s[2], dp[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[st][i] = 0.f;
          dp[st][i] = 0.f;
        }
#pragma unroll
        for (int kc = 0; kc < 8; ++kc) {
          const int off = tile_off(32 * st + col, 2 * kc + h);
          s[st] = mfma32(__builtin_bit_cast(bf16x8, lds_read16(kb, off)), qf[kc], s[st]);
          dp[st] = mfma32(__builtin_bit_cast(bf16x8, lds_read16(vb, off)), df[kc], dp[st]);
        }
      }
      const bool need_mask = (CAUSAL && (k0 + DQ_BC - 1 > q0w)) || (k0 + DQ_BC > N);
      bf16x8 sb[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float p = fast_exp2(__builtin_fmaf(s[st][i], sl2, -l2));
          if (need_mask) {
            const int key = k0 + 32 * st + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
          }
          dp[st][i] = p * (dp[st][i] - Dq);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int b = 8 * u;
          sb[st][u] = pack8(dp[st][b], dp[st][b + 1], dp[st][b + 2], dp[st][b + 3], dp[st][b + 4],
                            dp[st][b + 5], dp[st][b + 6], dp[st][b + 7]);
        }
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int dim = 32 * mb + tr_dim;
        const int chunk = dim >> 3;
        const int half = (dim >> 2) & 1;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int r = 32 * st + 16 * u + tr_row;
            const bf16x8 a = join(lds_read_tr(kb + tile_off8(r, chunk, half)),
                                  lds_read_tr(kb + tile_off8(r + 8, chunk, half)));
            acc[mb] = mfma32(a, sb[st][u], acc[mb]);
          }
      }
    }
    if (t + 1 < ntiles) swrite(buf ^ 1);
    __syncthreads();
  }

  if (qrow < N) {
    char* row = reinterpret_cast<char*>(dq + head) + (size_t)qrow * kRowBytes;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = 4 * g;
        u32x2 w = {pack_bf16(acc[mb][i] * scale, acc[mb][i + 1] * scale),
                   pack_bf16(acc[mb][i + 2] * scale, acc[mb][i + 3] * scale)};
        *reinterpret_cast<u32x2*>(row + (32 * mb + 8 * g + 4 * h) * 2) = w;
      }
  }
}

hipError_t launch_bwd_pre(const void* o, const void* dO, float* delta, int B, int H, int N,
                          hipStream_t stream) {
  const int rows = B * H * N;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO),
                     delta, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* lse, const float* delta, void* dk, void* dv, int B, int H,
                           int N, float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const float sl2 = scale * kLog2e;
  const int nkb = (N + KV_BK - 1) / KV_BK;
  dim3 grid((unsigned)(nkb * BH)), block(KV_THREADS);
  auto kern = causal ? bwd_dkdv_kernel<true> : bwd_dkdv_kernel<false>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dO), lse, delta, static_cast<uint16_t*>(dk),
                     static_cast<uint16_t*>(dv), BH, N, sl2, scale);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* delta, void* dq, int B, int H, int N,
                         float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const float sl2 = scale * kLog2e;
  const int nqb = (N + DQ_BQ - 1) / DQ_BQ;
  dim3 grid((unsigned)(nqb * BH)), block(DQ_THREADS);
  auto kern = causal ? bwd_dq_kernel<true> : bwd_dq_kernel<false>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dO), lse, delta, static_cast<uint16_t*>(dq), BH,
                     N, nqb, sl2, scale);
  return hipGetLastError();
}

}  // namespace fa
