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
//   bwd_pre   workspace <- [D = rowsum(dO o O) | L log2(e)]   HBM-bound
//   bwd_dkdv  per key block: K, V held in registers; query tiles of Q, dO,
//             L log2(e), D stream through LDS; dV^T += dO^T P, dK^T += Q^T dS
//   bwd_dq    per query block: Q, dO, L, D held in registers; K, V tiles
//             stream through LDS; dQ^T += K^T dS^T
// Tiles reach LDS through LDS-direct buffer loads; rows past N read as zero,
// which makes their P finite and their dO, dP, D and dS zero, so they add
// nothing to any gradient.
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
// 4 bytes per lane straight into LDS: lane i writes lds_base + 4 i.
__device__ __forceinline__ void buf_load4_lds(rsrc_t r, char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4,
                                           voff, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Pre-pass: D_i = sum_k dO_ik O_ik and L_i log2(e), 16 threads per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ ws, int rows) {
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
  if (row < rows && part == 0) {
    ws[row] = s;
    ws[(size_t)rows + row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK / dV
//
// A workgroup owns KV_BK = 128 keys of one head and runs 8 waves: wave w
// holds keys 32 (w % 4) .. + 31 and the query half w / 4 of every streamed
// 64-query tile, so the two waves of a key group split the queries and their
// partial dK, dV are summed through LDS at the end.  K and V of the block sit
// in LDS for the whole kernel; this keeps a wave at about 200 registers, two
// waves per SIMD, so one wave's softmax arithmetic overlaps the other's MFMA.
// ---------------------------------------------------------------------------
constexpr int KV_BK = 128;                  // keys per workgroup
constexpr int KV_WAVES = 8;
constexpr int KV_BQ = 64;                   // queries per streamed tile
constexpr int KV_TILE = KV_BQ * kRowBytes;  // 16 KiB (Q or dO)
constexpr int KV_BLOCK = KV_BK * kRowBytes;  // 32 KiB (K or V block)
constexpr int KV_STAGE = 2 * KV_TILE + 2 * KV_BQ * 4;  // Q, dO, L log2(e), D
constexpr int KV_SMEM = 2 * KV_BLOCK + 2 * KV_STAGE;   // 130 KiB
constexpr int KV_THREADS = KV_WAVES * 64;

template <bool CAUSAL>
__global__ __launch_bounds__(KV_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
                     const float* __restrict__ ws, uint16_t* __restrict__ dk,
                     uint16_t* __restrict__ dv, int BH, int N, float sl2, float scale) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* kblk = smem;
  char* vblk = smem + KV_BLOCK;
  char* stage0 = smem + 2 * KV_BLOCK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kg = wave & 3;   // key group of 32
  const int qh = wave >> 2;  // query half of each tile
  const int h = lane >> 5;
  const int col = lane & 31;

  // Causal: the first key blocks see the most queries; issue them first.
  int kb, bh;
  block_head(blockIdx.x, (N + KV_BK - 1) / KV_BK, BH, false, &kb, &bh);
  const int k0 = kb * KV_BK;
  const int kw = k0 + kg * 32;
  const int krow = kw + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const size_t rows = (size_t)BH * N;
  const rsrc_t rD = make_rsrc(ws + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rL = make_rsrc(ws + rows + (size_t)bh * N, (uint32_t)N * 4);

  const int ld_sub = lane >> 4;
  const int ld_pc = lane & 15;
  // K and V of the block: 128 rows each, 4 one-KiB loads per wave per tensor.
#pragma unroll
  for (int n = 0; n < KV_BK / 32; ++n) {
    const int row0 = 32 * n + 4 * wave;
    const int row = row0 + ld_sub;
    const uint32_t voff = (uint32_t)(k0 + row) * kRowBytes + ((ld_pc ^ swz(row)) << 4);
    buf_load16_lds(rk, kblk + row0 * kRowBytes, voff);
    buf_load16_lds(rv, vblk + row0 * kRowBytes, voff);
  }

  const int t0 = CAUSAL ? (k0 / KV_BQ) : 0;
  const int ntiles = (N + KV_BQ - 1) / KV_BQ;

  auto issue_tile = [&](int t, int buf) {
    char* base = stage0 + buf * KV_STAGE;
#pragma unroll
    for (int n = 0; n < KV_BQ / 32; ++n) {
      const int row0 = 32 * n + 4 * wave;
      const int row = row0 + ld_sub;
      const uint32_t voff = (uint32_t)(t * KV_BQ + row) * kRowBytes + ((ld_pc ^ swz(row)) << 4);
      buf_load16_lds(rq, base + row0 * kRowBytes, voff);
      buf_load16_lds(rdo, base + KV_TILE + row0 * kRowBytes, voff);
    }
    if (wave == 0) buf_load4_lds(rL, base + 2 * KV_TILE, (uint32_t)(t * KV_BQ + lane) * 4);
    if (wave == 1) buf_load4_lds(rD, base + 2 * KV_TILE + KV_BQ * 4, (uint32_t)(t * KV_BQ + lane) * 4);
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

  if (t0 < ntiles) issue_tile(t0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = t0; t < ntiles; ++t) {
    const int buf = (t - t0) & 1;
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    const char* qb = stage0 + buf * KV_STAGE;
    const char* dob = qb + KV_TILE;
    const float* lsb = reinterpret_cast<const float*>(qb + 2 * KV_TILE);
    const float* dsb = lsb + KV_BQ;
    const int qs = t * KV_BQ + 32 * qh;
    const bool active = !CAUSAL || (qs + 31 >= kw);
    if (active) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const int qoff = tile_off(32 * qh + col, 2 * kc + h);
        const int koff = tile_off(32 * kg + col, 2 * kc + h);
        s = mfma32(__builtin_bit_cast(bf16x8, lds_read16(qb, qoff)),
                   __builtin_bit_cast(bf16x8, lds_read16(kblk, koff)), s);
        dp = mfma32(__builtin_bit_cast(bf16x8, lds_read16(dob, qoff)),
                    __builtin_bit_cast(bf16x8, lds_read16(vblk, koff)), dp);
      }
      const bool need_mask = CAUSAL && (qs < kw + 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r = 32 * qh + 8 * g + 4 * h;  // tile-local query row of element 4g
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
          const int r = 32 * qh + 16 * u + tr_row;
          const bf16x8 a_do = join(lds_read_tr(dob + tile_off8(r, chunk, half)),
                                   lds_read_tr(dob + tile_off8(r + 8, chunk, half)));
          dva[mb] = mfma32(a_do, pb[u], dva[mb]);
          const bf16x8 a_q = join(lds_read_tr(qb + tile_off8(r, chunk, half)),
                                  lds_read_tr(qb + tile_off8(r + 8, chunk, half)));
          dka[mb] = mfma32(a_q, sb[u], dka[mb]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // Sum the two query halves: waves 4..7 park their partials in LDS (the loop
  // is over, every buffer is free), waves 0..3 add them and store.
  float* red = reinterpret_cast<float*>(smem) + kg * 2 * 64 * 64;  // 32 KiB per key group
  if (qh == 1) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[(mb * 16 + i) * 64 + lane] = dka[mb][i];
        red[64 * 64 + (mb * 16 + i) * 64 + lane] = dva[mb][i];
      }
  }
  __syncthreads();
  if (qh == 0) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dka[mb][i] += red[(mb * 16 + i) * 64 + lane];
        dva[mb][i] += red[64 * 64 + (mb * 16 + i) * 64 + lane];
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
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
constexpr int DQ_BQ = 128;   // queries per workgroup
constexpr int DQ_WAVES = 4;  // 32 queries per wave
constexpr int DQ_BC = 64;    // keys per streamed tile (two 32-key halves)
constexpr int DQ_TILE = DQ_BC * kRowBytes;
constexpr int DQ_THREADS = DQ_WAVES * 64;
constexpr int DQ_LOADS = DQ_TILE / 1024 / DQ_WAVES;

template <bool CAUSAL>
__global__ __launch_bounds__(DQ_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
                   const float* __restrict__ ws, uint16_t* __restrict__ dq, int BH, int N, int nqb,
                   float sl2, float scale) {
  __shared__ __attribute__((aligned(16))) char smem[2 * 2 * DQ_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  int qblk, bh;
  block_head(blockIdx.x, nqb, BH, CAUSAL, &qblk, &bh);
  const int q0 = qblk * DQ_BQ;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const size_t rows = (size_t)BH * N;
  const rsrc_t rD = make_rsrc(ws + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rL = make_rsrc(ws + rows + (size_t)bh * N, (uint32_t)N * 4);

  bf16x8 qf[8], df[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) {
    const uint32_t off = (uint32_t)qrow * kRowBytes + (2 * kc + h) * 16;
    qf[kc] = __builtin_bit_cast(bf16x8, buf_load16(rq, off));
    df[kc] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
  }
  const float l2 = buf_load_f32(rL, (uint32_t)qrow * 4);
  const float Dq = buf_load_f32(rD, (uint32_t)qrow * 4);

  const int kend = CAUSAL ? min(N, q0 + DQ_BQ) : N;
  const int ntiles = (kend + DQ_BC - 1) / DQ_BC;

  const int ld_sub = lane >> 4;
  const int ld_pc = lane & 15;
  auto issue_tile = [&](int t, int buf) {
    char* kb = smem + buf * 2 * DQ_TILE;
    char* vb = kb + DQ_TILE;
#pragma unroll
    for (int n = 0; n < DQ_LOADS; ++n) {
      const int row0 = 16 * n + 4 * wave;
      const int row = row0 + ld_sub;
      const uint32_t voff = (uint32_t)(t * DQ_BC + row) * kRowBytes + ((ld_pc ^ swz(row)) << 4);
      buf_load16_lds(rk, kb + row0 * kRowBytes, voff);
      buf_load16_lds(rv, vb + row0 * kRowBytes, voff);
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

  issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) issue_tile(t + 1, buf ^ 1);
    const int k0 = t * DQ_BC;
    const char* kb = smem + buf * 2 * DQ_TILE;
    const char* vb = kb + DQ_TILE;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int ks = k0 + 32 * st;
      const bool active = !CAUSAL || (ks <= q0w + 31);
      if (!active) continue;
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[i] = 0.f;
        dp[i] = 0.f;
      }
#pragma unroll
      for (int kc = 0; kc < 8; ++kc) {
        const int off = tile_off(32 * st + col, 2 * kc + h);
        s = mfma32(__builtin_bit_cast(bf16x8, lds_read16(kb, off)), qf[kc], s);
        dp = mfma32(__builtin_bit_cast(bf16x8, lds_read16(vb, off)), df[kc], dp);
      }
      const bool need_mask = (CAUSAL && (ks + 31 > q0w)) || (ks + 32 > N);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = fast_exp2(__builtin_fmaf(s[i], sl2, -l2));
        if (need_mask) {
          const int key = ks + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key >= N || (CAUSAL && key > qrow)) p = 0.f;
        }
        dp[i] = p * (dp[i] - Dq);
      }
      bf16x8 sb[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = 8 * u;
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
          const int r = 32 * st + 16 * u + tr_row;
          const bf16x8 a = join(lds_read_tr(kb + tile_off8(r, chunk, half)),
                                lds_read_tr(kb + tile_off8(r + 8, chunk, half)));
          acc[mb] = mfma32(a, sb[u], acc[mb]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
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

hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ws, int B, int H,
                          int N, hipStream_t stream) {
  const int rows = B * H * N;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), lse,
                     ws, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* ws, void* dk, void* dv, int B, int H, int N, float scale,
                           int causal, hipStream_t stream) {
  const int BH = B * H;
  const float sl2 = scale * kLog2e;
  const int nkb = (N + KV_BK - 1) / KV_BK;
  dim3 grid((unsigned)(nkb * BH)), block(KV_THREADS);
  auto kern = causal ? bwd_dkdv_kernel<true> : bwd_dkdv_kernel<false>;
  static bool attr_set[2] = {false, false};
  if (!attr_set[causal]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, KV_SMEM);
    if (e != hipSuccess) return e;
    attr_set[causal] = true;
  }
  hipLaunchKernelGGL(kern, grid, block, KV_SMEM, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dO), ws, static_cast<uint16_t*>(dk),
                     static_cast<uint16_t*>(dv), BH, N, sl2, scale);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* ws, void* dq, int B, int H, int N, float scale, int causal,
                         hipStream_t stream) {
  const int BH = B * H;
  const float sl2 = scale * kLog2e;
  const int nqb = (N + DQ_BQ - 1) / DQ_BQ;
  dim3 grid((unsigned)(nqb * BH)), block(DQ_THREADS);
  auto kern = causal ? bwd_dq_kernel<true> : bwd_dq_kernel<false>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dO), ws, static_cast<uint16_t*>(dq), BH, N, nqb,
                     sl2, scale);
  return hipGetLastError();
}

}  // namespace fa
