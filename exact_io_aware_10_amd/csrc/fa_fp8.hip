// FP8 forward with incoherent processing: Q, K and V rotated by a random
// Hadamard transform over the head dimension, quantised per block of 64 rows
// to OCP E4M3 with power-of-two scales, and attended with gfx950's FP8 MFMA:
// the FP8 scheme of "Interrogating the GPU, part 5: FlashAttention", section
// "What did FlashAttention-3 do with Hopper?", and of "FlashAttention
// versions", section "FlashAttention-3", built for this GPU.
//
// With sigma a random sign vector and H the 128 x 128 Sylvester Hadamard
// matrix (entries +-1, H H = 128 I):
//   Q' = (Q o sigma) H,  K' = (K o sigma) H,  V' = (V o sigma) H
//   S  = scale Q K^T = (scale / 128) Q' K'^T
//   O  = ((P V') H / 128) o sigma
// exactly in real arithmetic; only the E4M3 roundings of Q', K', V' and of P
// make the result approximate.
//
// fp8_quant_kernel   one wavefront per 64-row block: each lane rotates one
//                    row in float32 (fast Walsh-Hadamard transform, stage s
//                    pairing entries i and i + 2^s into (a + b, a - b)), the
//                    block's largest magnitude sets the exponent e (the
//                    smallest with amax <= 448 2^e), and the codes are
//                    E4M3(y 2^-e), round to nearest even.  V is written
//                    transposed per 64-key tile, keys in the order the P V'
//                    MFMA pairs them with P.
// fwd_fp8_kernel     the bf16 forward's structure (4 wavefronts x 32 queries,
//                    64-key tiles through LDS, online softmax with the
//                    conditional rescale) with 32x32x64 FP8 MFMAs: 4 for
//                    S^T = K8 Q8^T and 4 for O'^T = V8^T P8^T per tile, the
//                    per-block exponents folded into the softmax multiplier
//                    (Q, K) and the MFMA's scale operand (V); the epilogue
//                    undoes the rotation in registers.
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

typedef int i32x8 __attribute__((ext_vector_type(8)));
template <int V>
using ic8 = std::integral_constant<int, V>;

constexpr int F8_BLK = 64;                  // rows per quantisation block = keys per tile
constexpr int F8_ROWB = kD;                 // bytes per E4M3 row
constexpr int F8_TILE = F8_BLK * F8_ROWB;   // 8 KiB: one K tile or one transposed V tile
constexpr int F8_BR = 128;                  // queries per workgroup
constexpr int F8_WAVES = 4;
constexpr int F8_THREADS = F8_WAVES * 64;
// Conditional-rescale threshold (log2 units), and the power of two P~ is
// multiplied by before it is rounded to E4M3: P~ <= 2^tau, so P~ 2^6 <= 256
// stays below E4M3's largest value 448 while small P keep normal precision.
constexpr float kTauF8 = 2.f;
constexpr float kPShiftF8 = 6.f;

// Position of block-local key r inside a transposed V tile row: lane half h
// of the P V' MFMA holds, as its bytes j = 0..31, the P of keys
// 32 (j / 16) + 8 ((j % 16) / 4) + 4 h + j % 4 (the S^T accumulator layout of
// the two 32-key groups), so that key is stored at 32 h + j.
__device__ __forceinline__ int vt_pos(int r) {
  return 32 * ((r >> 2) & 1) + 16 * (r >> 5) + 4 * ((r >> 3) & 3) + (r & 3);
}

// E4M3 codes of four floats packed into one dword, a in byte 0
// (v_cvt_pk_fp8_f32: OCP E4M3, round to nearest even).
__device__ __forceinline__ int cvt_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// ---------------------------------------------------------------------------
// Quantisation
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void fp8_quant_kernel(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ signs,
                                                       uint8_t* __restrict__ codes,
                                                       int* __restrict__ exps, int N, int nblk,
                                                       int layout) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[F8_TILE];  // transposed V staging
  const int bh = blockIdx.x / nblk;
  const int blk = blockIdx.x - bh * nblk;
  const int r = threadIdx.x;
  const int row = blk * F8_BLK + r;
  const bool valid = row < N;

  // The row, widened to float32, with the signs applied (exact).
  float y[kD];
  const uint16_t* src = x + ((size_t)bh * N + (valid ? row : 0)) * kD;
#pragma unroll
  for (int c = 0; c < kD / 8; ++c) {
    u32x4 w = {0u, 0u, 0u, 0u};
    if (valid) w = *reinterpret_cast<const u32x4*>(src + 8 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y[8 * c + 2 * j] = __uint_as_float(w[j] << 16) * signs[8 * c + 2 * j];
      y[8 * c + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u) * signs[8 * c + 2 * j + 1];
    }
  }
  // Fast Walsh-Hadamard transform, stages in increasing stride.
#pragma unroll
  for (int s = 1; s < kD; s <<= 1)
#pragma unroll
    for (int i = 0; i < kD; ++i)
      if ((i & s) == 0) {
        const float a = y[i], b = y[i + s];
        y[i] = a + b;
        y[i + s] = a - b;
      }

  float am = 0.f;
#pragma unroll
  for (int i = 0; i < kD; ++i) am = fmaxf(am, fabsf(y[i]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  // amax = f 2^E, f in [0.5, 1); 448 = 0.875 2^9.
  int e = -127;
  if (am > 0.f) {
    int E;
    const float f = frexpf(am, &E);
    e = f > 0.875f ? E - 8 : E - 9;
  }

  uint32_t w[kD / 4];
#pragma unroll
  for (int i = 0; i < kD / 4; ++i) {
    w[i] = (uint32_t)cvt_fp8x4(ldexpf(y[4 * i], -e), ldexpf(y[4 * i + 1], -e),
                               ldexpf(y[4 * i + 2], -e), ldexpf(y[4 * i + 3], -e));
  }
  if (r == 0) exps[blockIdx.x] = e;

  if (layout == 0) {
    if (valid) {
      uint8_t* dst = codes + ((size_t)bh * N + row) * F8_ROWB;
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<u32x4*>(dst + 16 * c) = u32x4{w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]};
    }
  } else {
    // Transposed tile: dimension rows of 64 bytes, this key at vt_pos(r).
    const int p = vt_pos(r);
#pragma unroll
    for (int i = 0; i < kD; ++i) tile[i * F8_BLK + p] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    __syncthreads();
    uint8_t* dst = codes + ((size_t)bh * nblk + blk) * F8_TILE;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int off = (c * 64 + r) * 16;
      *reinterpret_cast<u32x4*>(dst + off) = *reinterpret_cast<const u32x4*>(tile + off);
    }
  }
}

// ---------------------------------------------------------------------------
// Attention
// ---------------------------------------------------------------------------
// LDS chunk swizzles (16-byte chunks), conflict-free for the operand reads:
// K tile rows are 128 bytes (8 chunks), V tile rows 64 bytes (4 chunks).
__device__ __forceinline__ int kswz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int vswz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ i32x8 join8(u32x4 a, u32x4 b) {
  return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
}

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, 127);
}

// Three workgroups per CU (one wave of each per SIMD, at most 168 VGPRs and
// 32 KiB of LDS apiece): a third wave per SIMD keeps the matrix pipe fed
// while the other two exponentiate, which two waves do not.
template <bool CAUSAL>
__global__ __launch_bounds__(F8_THREADS) __attribute__((amdgpu_waves_per_eu(3, 3)))
void fwd_fp8_kernel(const uint8_t* __restrict__ q8, const int* __restrict__ qexp,
                    const uint8_t* __restrict__ k8, const int* __restrict__ kexp,
                    const uint8_t* __restrict__ v8, const int* __restrict__ vexp,
                    const float* __restrict__ signs, uint16_t* __restrict__ o,
                    float* __restrict__ lse, int BH, int N, int nqb, float sl2base,
                    uint32_t qkeep, uint32_t qflip) {
  __shared__ __attribute__((aligned(16))) char k_lds0[F8_TILE];
  __shared__ __attribute__((aligned(16))) char k_lds1[F8_TILE];
  __shared__ __attribute__((aligned(16))) char v_lds0[F8_TILE];
  __shared__ __attribute__((aligned(16))) char v_lds1[F8_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  int qb, bh;
  block_head(blockIdx.x, nqb, BH, CAUSAL, CAUSAL, &qb, &bh);
  const int q0 = qb * F8_BR;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + col;
  const int nkt = (N + F8_BLK - 1) / F8_BLK;

  const rsrc_t rq = make_rsrc(q8 + (size_t)bh * N * F8_ROWB, (uint32_t)N * F8_ROWB);
  const rsrc_t rk = make_rsrc(k8 + (size_t)bh * N * F8_ROWB, (uint32_t)N * F8_ROWB);
  const rsrc_t rv = make_rsrc(v8 + (size_t)bh * nkt * F8_TILE, (uint32_t)nkt * F8_TILE);
  const int* ke = kexp + (size_t)bh * nkt;
  const int* ve = vexp + (size_t)bh * nkt;

  // Q codes as the B operand of S^T = K Q^T: lane holds Q8[qrow][64 kk + 32 h .. + 31]
  // (zero past N).  The wave's 32 queries share one quantisation block.
  i32x8 qf[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const uint32_t off = (uint32_t)qrow * F8_ROWB + 64 * kk + 32 * h;
    qf[kk] = join8(signed_operand(buf_load16(rq, off), qkeep, qflip),
                   signed_operand(buf_load16(rq, off + 16), qkeep, qflip));
  }
  const int qe = qexp[(size_t)bh * nkt + min(q0w / F8_BLK, nkt - 1)];
  const float sl2q = ldexpf(sl2base, qe);

  const int kend = CAUSAL ? min(N, q0 + F8_BR) : N;
  const int ntiles = (kend + F8_BLK - 1) / F8_BLK;

  // Tile loader (LDS-direct, 1 KiB per instruction, lane i -> byte 16 i).
  // Instruction I = 2 wave + n: K rows 8 I .. + 7 (lane i: row 8 I + i / 8,
  // physical chunk i % 8), V dimension rows 16 I .. + 15 (lane i: row
  // 16 I + i / 4, physical chunk i % 4); each lane fetches the logical chunk
  // the swizzle stores there.
  uint32_t k_voff[2], v_voff[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int I = 2 * wave + n;
    const int kr = 8 * I + (lane >> 3);
    k_voff[n] = (uint32_t)kr * F8_ROWB + (((lane & 7) ^ kswz(kr)) << 4);
    const int vr = 16 * I + (lane >> 2);
    v_voff[n] = (uint32_t)vr * F8_BLK + (((lane & 3) ^ vswz(vr)) << 4);
  }
  auto issue_tile = [&](int t, auto bufc) {
    char* kb = decltype(bufc)::value ? k_lds1 : k_lds0;
    char* vb = decltype(bufc)::value ? v_lds1 : v_lds0;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int I = 2 * wave + n;
      buf_load16_lds(rk, kb + 1024 * I, k_voff[n] + (uint32_t)t * F8_TILE);
      buf_load16_lds(rv, vb + 1024 * I, v_voff[n] + (uint32_t)t * F8_TILE);
    }
  };

  // Per-lane LDS offsets of the operand reads (tile-relative, two 16-byte
  // halves each): K row 32 st + col, dimensions 64 kk + 32 h + 16 u;
  // V dimension row 32 mb + col, key positions 32 h + 16 u.
  int koff[2][2][2], voff[4][2];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int kr = 32 * st + col;
        koff[st][kk][u] = kr * F8_ROWB + (((4 * kk + 2 * h + u) ^ kswz(kr)) << 4);
      }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vr = 32 * mb + col;
      voff[mb][u] = vr * F8_BLK + (((2 * h + u) ^ vswz(vr)) << 4);
    }

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m = -INFINITY;  // reference maximum (log2 units of the scaled scores)
  float l = 0.f;        // this lane's half of the row sum of P~ 2^6

  auto step = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < ntiles) issue_tile(t + 1, ic8<BUF ^ 1>{});
    const int k0 = t * F8_BLK;
    const bool active = !CAUSAL || (k0 <= q0w + 31);
    if (active) {
      const char* kb = BUF ? k_lds1 : k_lds0;
      const char* vb = BUF ? v_lds1 : v_lds0;
      const float sl2 = ldexpf(sl2q, ke[t]);
      const int vscale = ve[t] + 127;  // E8M0 exponent of the V block

      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const i32x8 a = join8(lds_read16(kb, koff[st][kk][0]), lds_read16(kb, koff[st][kk][1]));
          s[st] = mfma_f8(a, qf[kk], s[st], 127);
        }

      const bool need_mask = (CAUSAL && (k0 + F8_BLK - 1 > q0w)) || (k0 + F8_BLK > N);
      if (need_mask) {
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * st + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[st][i] = -INFINITY;
          }
      }

      float mx = s[0][0];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[st][i]);
      mx = halves_max(mx);
      const float mcand = mx * sl2;
      if (__builtin_amdgcn_ballot_w64(mcand > m + kTauF8) != 0) {
        const float mnew = fmaxf(m, mcand);
        const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
      }
      const float mu = (m == -INFINITY) ? 0.f : m;

      // P~ 2^6 = 2^(S log2 e - m + 6), written over S, and its row sum.
      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[st][i], sl2, kPShiftF8 - mu));
          s[st][i] = p;
          rs += p;
        }
      l += rs;

      // E4M3 P as the B operand of O'^T = V'^T P^T: byte j = element
      // (j / 16, j % 16) of s.
      i32x8 pb;
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const int st = wd >> 2, i0 = 4 * (wd & 3);
        pb[wd] = cvt_fp8x4(s[st][i0], s[st][i0 + 1], s[st][i0 + 2], s[st][i0 + 3]);
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const i32x8 a = join8(lds_read16(vb, voff[mb][0]), lds_read16(vb, voff[mb][1]));
        acc[mb] = mfma_f8(a, pb, acc[mb], vscale);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue_tile(0, ic8<0>{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(t, ic8<0>{});
    if (t + 1 < ntiles) step(t + 1, ic8<1>{});
  }

  // Undo the rotation: O = (O' H / 128) o sigma with O' = acc / (row sum).
  // Lane (query, h) holds dimension 32 mb + 8 (i / 4) + 4 h + i % 4 in
  // acc[mb][i]; the Walsh-Hadamard stages over dimension bits 0, 1, 3, 4, 5, 6
  // pair registers of the lane, the stage over bit 2 pairs lane l with l ^ 32.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int bit = 1; bit <= 8; bit <<= 1)  // element bits 0, 1 (dims 1, 2), 2, 3 (dims 8, 16)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if ((i & bit) == 0) {
          const float x = acc[mb][i], y = acc[mb][i + bit];
          acc[mb][i] = x + y;
          acc[mb][i + bit] = x - y;
        }
#pragma unroll
  for (int bit = 1; bit <= 2; bit <<= 1)  // dims 32, 64
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      if ((mb & bit) == 0)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = acc[mb][i], y = acc[mb + bit][i];
          acc[mb][i] = x + y;
          acc[mb + bit][i] = x - y;
        }
  // dim bit 2: half 0 (x0) keeps x0 + x1, half 1 (x1) gets x0 - x1.
  const float hs = h ? -1.f : 1.f;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float other = __shfl_xor(acc[mb][i], 32);
      acc[mb][i] = __builtin_fmaf(acc[mb][i], hs, other);
    }

  const float lt = halves_sum(l);
  if (qrow < N) {
    const float inv = 1.f / (lt * (float)kD);
    char* orow = reinterpret_cast<char*>(o + (size_t)bh * N * kD) + (size_t)qrow * kRowBytes;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = 4 * g;
        const int dim = 32 * mb + 8 * g + 4 * h;
        const f32x4 sg = *reinterpret_cast<const f32x4*>(signs + dim);
        u32x2 w = {pack_bf16(acc[mb][i] * inv * sg[0], acc[mb][i + 1] * inv * sg[1]),
                   pack_bf16(acc[mb][i + 2] * inv * sg[2], acc[mb][i + 3] * inv * sg[3])};
        *reinterpret_cast<u32x2*>(orow + dim * 2) = w;
      }
    if (h == 0) lse[(size_t)bh * N + qrow] = (m + __log2f(lt) - kPShiftF8) * kLn2;
  }
}

hipError_t launch_fp8_quant(const void* x, const float* signs, void* codes, int* exps, int B, int H,
                            int N, int layout, hipStream_t stream) {
  const int nblk = (N + F8_BLK - 1) / F8_BLK;
  const unsigned grid = (unsigned)(B * H * nblk);
  hipLaunchKernelGGL(fp8_quant_kernel, dim3(grid), dim3(64), 0, stream,
                     static_cast<const uint16_t*>(x), signs, static_cast<uint8_t*>(codes), exps, N,
                     nblk, layout);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const void* q8, const int* qexp, const void* k8, const int* kexp,
                          const void* v8, const int* vexp, const float* signs, void* o, float* lse,
                          int B, int H, int N, float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const int nqb = (N + F8_BR - 1) / F8_BR;
  // |scale|; the sign (or a zero scale) is folded into the Q codes, whose
  // sign bits are flipped (or cleared) as they are loaded.
  const signed_scale sc = split_scale(scale, kSignBitsFp8);
  const float sl2base = sc.mag * kLog2e / (float)kD;  // Q' K'^T = 128 Q K^T
  dim3 grid((unsigned)(nqb * BH)), block(F8_THREADS);
  auto kern = causal ? fwd_fp8_kernel<true> : fwd_fp8_kernel<false>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<const uint8_t*>(q8), qexp,
                     static_cast<const uint8_t*>(k8), kexp, static_cast<const uint8_t*>(v8), vexp,
                     signs, static_cast<uint16_t*>(o), lse, BH, N, nqb, sl2base, sc.keep, sc.flip);
  return hipGetLastError();
}

}  // namespace fa
