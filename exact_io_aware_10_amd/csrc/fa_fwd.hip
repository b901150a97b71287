// Forward kernel: exact softmax attention by tiling with an online softmax.
//
// One workgroup owns FWD_BR = 256 query rows of one (batch, head) and streams
// the head's keys and values through LDS in tiles of FWD_BC = 64 rows; each
// of its 8 wavefronts (two per SIMD) owns 32 of the query rows
// ("Interrogating the GPU, part 5: FlashAttention", sections "How does tiling
// remove the traffic?" and "What did FlashAttention-2 fix?": queries split
// across warps, outer loop over query blocks, grid over query blocks x
// heads).  Each K/V tile brought into LDS serves 256 queries: half the L2 and
// fabric traffic of 128-row blocks, which at the board's power cap is worth
// more than the freedom of two independent workgroups per CU.
//
// Per tile and wave:
//   S^T = K_j Q_i^T         bf16 MFMA 32x32x16, fp32 accumulate (C: key rows,
//                           query columns; each lane owns one query)
//   online softmax          m' = max(m, rowmax S), alpha = 2^(m - m'),
//                           P = 2^(S log2e scale - m'), l = alpha l + rowsum P
//                           ("How can you softmax a row you never see whole?",
//                           update rule; exp2 with log2(e) folded into scale)
//   O^T = alpha O^T + V_j^T P^T   bf16 MFMA; V read transposed from LDS
// and after the last tile O = O / l (one division per row) and
// LSE = ln2 (m + log2 l) ("What does the backward pass do without P?").
// Causal: key tiles wholly after the workgroup's last query are never loaded,
// tiles wholly after a wave's last query are skipped by that wave, and the
// diagonal tiles are masked element-wise ("LLM flash attention", section
// "End-to-end flow").
#include <type_traits>

#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

constexpr int FWD_BR = 256;
constexpr int FWD_WAVES = 8;
constexpr int FWD_QW = FWD_BR / FWD_WAVES;  // 32 query rows per wave
constexpr int FWD_BC = 64;
constexpr int FWD_TILE = FWD_BC * kRowBytes;  // 16 KiB per K or V tile
constexpr int FWD_THREADS = FWD_WAVES * 64;
constexpr int FWD_LOADS = FWD_TILE / 1024 / FWD_WAVES;  // 1 KiB LDS-direct loads per wave
static_assert(FWD_QW == 32 && 4 * FWD_WAVES * FWD_LOADS == FWD_BC,
              "the tile loader's rows 4 FWD_WAVES n + 4 w + lane / 16 cover one tile exactly");

// Rows whose running maximum grows by less than this (log2 units) keep the
// stale maximum: P is then bounded by 2^kTau and the O / l rescale is skipped
// ("Interrogating the GPU, part 5", FlashAttention-4 section: the rescale
// becomes conditional; exact in real arithmetic since O and l share the
// reference maximum that LSE records).
constexpr float kTau = 8.f;

template <int V>
using ic = std::integral_constant<int, V>;

// 2^x on the FMA path instead of the transcendental unit ("Interrogating the
// GPU, part 5: FlashAttention", section "Why did Blackwell need
// FlashAttention-4?": part of the exponentials evaluated in software):
// x = n + f with n = floor(x) and f in [0, 1), 2^f from the page's cubic
// 1 + 0.6951 f + 0.2276 f^2 + 0.0771 f^3 (relative error about 1e-4 on
// [0, 1)), and n added to the exponent field of the result.  Arguments here
// are at most kTau (the stale maximum bounds the scores), so 2^n stays
// normal; below -126 (masked scores are -inf) the result is 0.  Ten
// full-rate VALU instructions against one v_exp_f32.
__device__ __forceinline__ float soft_exp2(float x) {
  const float xc = fmaxf(x, -126.f);
  const float fl = __builtin_floorf(xc);
  const float f = xc - fl;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(0.0771f, f, 0.2276f), f, 0.6951f), f, 1.f);
  const float r = __int_as_float(__float_as_int(p) + ((int)fl << 23));
  return x >= -126.f ? r : 0.f;
}

// SW of a lane's 32 exponentials per tile (0, 8, 16 or 32) go through
// soft_exp2, spread evenly over the tile: element e = 16 st + i when
// e % (32 / SW) == 0.
template <int SW>
__device__ __forceinline__ constexpr bool soft_elem(int e) {
  return SW > 0 && e % (32 / SW) == 0;
}

template <bool CAUSAL, int SW = 0>
__global__ __launch_bounds__(FWD_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                float* __restrict__ lse, int BH, int N, int nqb, float sl2, uint32_t qkeep,
                uint32_t qflip) {
  // [buffer][K | V] tiles, each 64 rows x 256 bytes, swizzled (tile_off).
  __shared__ __attribute__((aligned(16))) char k_lds0[FWD_TILE];
  __shared__ __attribute__((aligned(16))) char k_lds1[FWD_TILE];
  __shared__ __attribute__((aligned(16))) char v_lds0[FWD_TILE];
  __shared__ __attribute__((aligned(16))) char v_lds1[FWD_TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // Causal: issue the longest query blocks first.
  int qb, bh;
  block_head(blockIdx.x, nqb, BH, CAUSAL, CAUSAL, &qb, &bh);
  const int q0 = qb * FWD_BR;
  const int q0w = q0 + wave * FWD_QW;
  const int qrow = q0w + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);

  // Q^T as the B operand: lane holds Q[qrow][16 kc + 8 h .. + 7] (zero past N),
  // negated for a negative scale and cleared for scale 0 (sl2 is |scale| log2 e).
  bf16x8 qf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    qf[kc] = __builtin_bit_cast(
        bf16x8, signed_operand(buf_load16(rq, (uint32_t)qrow * kRowBytes + (2 * kc + h) * 16), qkeep, qflip));

  const int kend = CAUSAL ? min(N, q0 + FWD_BR) : N;
  const int ntiles = (kend + FWD_BC - 1) / FWD_BC;

  // Tile loader: LDS-direct buffer loads.  Instruction n of wave w fills rows
  // 32 n + 4 w .. + 3 (1 KiB, lane-linear in LDS); lane i lands on physical
  // chunk i % 16 of its row and so fetches the logical chunk stored there.
  // The tile's row offset is added to the per-lane offset, the part the
  // hardware range-checks, so rows past N read as zero.
  uint32_t ld_voff[FWD_LOADS];
#pragma unroll
  for (int n = 0; n < FWD_LOADS; ++n) {
    const int row = 4 * FWD_WAVES * n + 4 * wave + (lane >> 4);
    ld_voff[n] = (uint32_t)row * kRowBytes + (((lane & 15) ^ swz(row)) << 4);
  }
  auto issue_tile = [&](int t, auto bufc) {
    char* kb = decltype(bufc)::value ? k_lds1 : k_lds0;
    char* vb = decltype(bufc)::value ? v_lds1 : v_lds0;
    const uint32_t toff = (uint32_t)t * FWD_TILE;
#pragma unroll
    for (int n = 0; n < FWD_LOADS; ++n) {
      const int row0 = 4 * FWD_WAVES * n + 4 * wave;
      buf_load16_lds(rk, kb + row0 * kRowBytes, ld_voff[n] + toff);
      buf_load16_lds(rv, vb + row0 * kRowBytes, ld_voff[n] + toff);
    }
  };

  // Per-lane LDS offsets, fixed for the whole kernel (tile-relative):
  //   K rows for S^T: row col (+ 32 st), logical chunk 2 kc + h;
  //   V transpose reads: row 4 h + (lane % 16) / 4 (+ 8, + 16 u, + 32 st),
  //   dims 32 mb + 16 ((lane / 16) % 2) + 4 (lane % 4).
  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = tile_off(col, 2 * kc + h);
  int voff[4][2];
  {
    const int tr_s = lane & 15;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
    const int tr_row = 4 * h + (tr_s >> 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int dim = 32 * mb + tr_dim;
#pragma unroll
      for (int e = 0; e < 2; ++e) voff[mb][e] = tile_off8(tr_row + 8 * e, dim >> 3, (dim >> 2) & 1);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m = -INFINITY;  // reference maximum, log2 domain of the scaled scores
  float l = 0.f;        // running sum of P over this lane's half of each tile (for LSE)
  float lr = 0.f;       // the same sum of P as rounded to bf16 for the P V product
  // O is divided by lr: normalised by exactly the weights it was built from,
  // O stays a convex combination of V rows, and on rows dominated by one key
  // (large score ranges, where the stale reference maximum leaves that key's
  // P anywhere in [1, 2^kTau] and its bf16 rounding would otherwise move O by
  // up to 2^-9 |V|) the rounding cancels.  LSE keeps the fp32 sum l.

  auto step = [&](int t, auto bufc) {
    constexpr int BUF = decltype(bufc)::value;
    if (t + 1 < ntiles) issue_tile(t + 1, ic<BUF ^ 1>{});
    const int k0 = t * FWD_BC;
    const bool active = !CAUSAL || (k0 <= q0w + FWD_QW - 1);
    if (active) {
      const char* kb = BUF ? k_lds1 : k_lds0;
      const char* vb = BUF ? v_lds1 : v_lds0;

      f32x16 s[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[st][i] = 0.f;
#pragma unroll
      for (int kc = 0; kc < 8; ++kc)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, lds_read16(kb + st * 32 * kRowBytes, koff[kc]));
          s[st] = mfma32(a, qf[kc], s[st]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < 10; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);

      const bool need_mask = (CAUSAL && (k0 + FWD_BC - 1 > q0w)) || (k0 + FWD_BC > N);
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
      if (__builtin_amdgcn_ballot_w64(mcand > m + kTau) != 0) {
        const float mnew = fmaxf(m, mcand);
        const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
        m = mnew;
        l *= alpha;
        lr *= alpha;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
      }
      const float mu = (m == -INFINITY) ? 0.f : m;  // no (-inf) - (-inf)

      float rs = 0.f;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = __builtin_fmaf(s[st][i], sl2, -mu);
          const float p = soft_elem<SW>(16 * st + i) ? soft_exp2(x) : fast_exp2(x);
          s[st][i] = p;
          rs += p;
        }
      l += rs;

      bf16x8 pb[2][2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int b = 8 * u;
          pb[st][u] = pack8(s[st][b], s[st][b + 1], s[st][b + 2], s[st][b + 3], s[st][b + 4],
                            s[st][b + 5], s[st][b + 6], s[st][b + 7]);
          const u32x4 pw = __builtin_bit_cast(u32x4, pb[st][u]);
#pragma unroll
          for (int e = 0; e < 4; ++e) lr = add_bf16_pair(pw[e], lr);
        }

#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            const char* rb = vb + (32 * st + 16 * u) * kRowBytes;
            const i16x4 lo = lds_read_tr(rb + voff[mb][0]);
            const i16x4 hi = lds_read_tr(rb + voff[mb][1]);
            acc[mb] = mfma32(join(lo, hi), pb[st][u], acc[mb]);
          }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  issue_tile(0, ic<0>{});
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int t = 0; t < ntiles; t += 2) {
    step(t, ic<0>{});
    if (t + 1 < ntiles) step(t + 1, ic<1>{});
  }

  const float lt = halves_sum(l);
  const float lrt = halves_sum(lr);
  if (qrow < N) {
    const float inv = 1.f / lrt;
    char* orow = reinterpret_cast<char*>(o + head) + (size_t)qrow * kRowBytes;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = 4 * g;
        u32x2 w = {pack_bf16(acc[mb][i] * inv, acc[mb][i + 1] * inv),
                   pack_bf16(acc[mb][i + 2] * inv, acc[mb][i + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + (32 * mb + 8 * g + 4 * h) * 2) = w;
      }
    if (h == 0) lse[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Ping-pong forward ("Interrogating the GPU, part 5", section "What did
// FlashAttention-3 do with Hopper?", and "FlashAttention versions", section
// "FlashAttention-3": one group's softmax on the vector units while the other
// group's matrix products run).  Same tiles, numerics and results contract as
// fwd_kernel; what differs is the schedule.  Waves w and w + 4 of the
// workgroup share a SIMD.  Each wave alternates an MFMA phase (O^T += V^T P^T
// of the previous tile, then S^T of this tile) with a softmax phase (mask,
// running maximum and conditional rescale, P, row sums); waves 4..7 run one
// phase behind waves 0..3 and a workgroup barrier ends every phase, so on
// every SIMD one wave's MFMAs meet the other wave's exponentials.  K/V tiles
// stream through three LDS stages (tile t - 1's V is still read while tile t
// is used and tile t + 1 loads).
// ---------------------------------------------------------------------------
constexpr int PP_STAGES = 3;
__device__ __forceinline__ int opaque_int(int x) {
  asm volatile("" : "+v"(x));
  return x;
}
constexpr int PP_STAGE = 2 * FWD_TILE;  // K tile, then V tile

template <bool CAUSAL>
__global__ __launch_bounds__(FWD_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                   float* __restrict__ lse, int BH, int N, int nqb, float sl2, uint32_t qkeep,
                   uint32_t qflip) {
  __shared__ __attribute__((aligned(16))) char smem[PP_STAGES * PP_STAGE];
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: leads, 1: one phase behind
  const int h = lane >> 5;
  const int col = lane & 31;

  int qb, bh;
  block_head(blockIdx.x, nqb, BH, CAUSAL, CAUSAL, &qb, &bh);
  const int q0 = qb * FWD_BR;
  const int q0w = q0 + wave * FWD_QW;
  const int qrow = q0w + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);

  bf16x8 qf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    qf[kc] = __builtin_bit_cast(
        bf16x8, signed_operand(buf_load16(rq, (uint32_t)qrow * kRowBytes + (2 * kc + h) * 16), qkeep, qflip));
  // Q has arrived (in the compiler's view too) before any LDS-direct load,
  // which the compiler does not track, is in flight.
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) asm volatile("" : : "v"(qf[kc]));

  const int kend = CAUSAL ? min(N, q0 + FWD_BR) : N;
  const int T = (kend + FWD_BC - 1) / FWD_BC;

  uint32_t ld_voff[FWD_LOADS];
#pragma unroll
  for (int n = 0; n < FWD_LOADS; ++n) {
    const int row = 4 * FWD_WAVES * n + 4 * wave + (lane >> 4);
    ld_voff[n] = (uint32_t)row * kRowBytes + (((lane & 15) ^ swz(row)) << 4);
  }
  auto issue_tile = [&](int t) {
    const uint32_t st = smem_lds + (uint32_t)(t % PP_STAGES) * PP_STAGE;
    const uint32_t toff = (uint32_t)t * FWD_TILE;
#pragma unroll
    for (int n = 0; n < FWD_LOADS; ++n) {
      const uint32_t dst = st + (uint32_t)(4 * FWD_WAVES * n + 4 * wave) * kRowBytes;
      dma16(rk, dst, ld_voff[n] + toff);
      dma16(rv, dst + FWD_TILE, ld_voff[n] + toff);
    }
  };

  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = tile_off(col, 2 * kc + h);
  int voff[4][2];
  {
    const int tr_s = lane & 15;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
    const int tr_row = 4 * h + (tr_s >> 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int dim = 32 * mb + tr_dim;
#pragma unroll
      for (int e = 0; e < 2; ++e) voff[mb][e] = tile_off8(tr_row + 8 * e, dim >> 3, (dim >> 2) & 1);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m = -INFINITY, l = 0.f, lr = 0.f;  // as in fwd_kernel
  f32x16 sc[2];     // S^T of the tile whose softmax phase is next
  bf16x8 pb[2][2];  // P^T of the tile whose P V product is next
  // A rescale decided in a softmax phase reaches O^T at the start of the
  // next MFMA phase, before that tile's P V product (the accumulators are
  // touched only in MFMA phases).
  bool rescale = false;
  float alpha_pending = 1.f;

  // MFMA phase of tile tm: O^T += V^T P^T of tile tm - 1, then S^T of tile tm.
  // Operands are read PP_AHEAD MFMAs ahead of their use (sched_barrier keeps
  // the compiler to that depth: hoisting every read of the phase would not
  // fit two waves' registers).
  constexpr int PP_AHEAD = 2;
  auto mfma_phase = [&](int tm) {
    if (rescale) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha_pending;
      rescale = false;
    }
    if (tm > 0) {
      // The stage offset through a register the compiler cannot follow, so
      // that it forms eight lane addresses per phase instead of keeping
      // every stage's addresses live across the loop.
      const char* vb = smem + opaque_int(((tm - 1) % PP_STAGES) * PP_STAGE) + FWD_TILE;
      bf16x8 va[PP_AHEAD + 1];
      auto rdv = [&](int j) {  // j = 8 st + 4 u + mb
        const char* rb = vb + (32 * (j >> 3) + 16 * ((j >> 2) & 1)) * kRowBytes;
        va[j % (PP_AHEAD + 1)] = join(lds_read_tr(rb + voff[j & 3][0]), lds_read_tr(rb + voff[j & 3][1]));
      };
#pragma unroll
      for (int j = 0; j < PP_AHEAD; ++j) rdv(j);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j + PP_AHEAD < 16) rdv(j + PP_AHEAD);
        acc[j & 3] = mfma32(va[j % (PP_AHEAD + 1)], pb[j >> 3][(j >> 2) & 1], acc[j & 3]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (tm < T) {
      const char* kb = smem + opaque_int((tm % PP_STAGES) * PP_STAGE);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[st][i] = 0.f;
      bf16x8 ka[PP_AHEAD + 1];
      auto rdk = [&](int j) {  // j = 2 kc + st
        ka[j % (PP_AHEAD + 1)] = __builtin_bit_cast(bf16x8, lds_read16(kb + (j & 1) * 32 * kRowBytes, koff[j >> 1]));
      };
#pragma unroll
      for (int j = 0; j < PP_AHEAD; ++j) rdk(j);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j + PP_AHEAD < 16) rdk(j + PP_AHEAD);
        sc[j & 1] = mfma32(ka[j % (PP_AHEAD + 1)], qf[j >> 1], sc[j & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Softmax phase of tile tv (the same steps as fwd_kernel's).
  auto softmax_phase = [&](int tv) {
    const int k0 = tv * FWD_BC;
    const bool need_mask = (CAUSAL && (k0 + FWD_BC - 1 > q0w)) || (k0 + FWD_BC > N);
    if (need_mask) {
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * st + 8 * (i >> 2) + 4 * h + (i & 3);
          if (key >= N || (CAUSAL && key > qrow)) sc[st][i] = -INFINITY;
        }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[st][i]);
    mx = halves_max(mx);
    const float mcand = mx * sl2;
    if (__builtin_amdgcn_ballot_w64(mcand > m + kTau) != 0) {
      const float mnew = fmaxf(m, mcand);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
      lr *= alpha;
      alpha_pending = alpha;
      rescale = true;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sc[st][i], sl2, -mu));
        sc[st][i] = p;
        rs += p;
      }
    l += rs;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int b = 8 * u;
        pb[st][u] = pack8(sc[st][b], sc[st][b + 1], sc[st][b + 2], sc[st][b + 3], sc[st][b + 4],
                          sc[st][b + 5], sc[st][b + 6], sc[st][b + 7]);
        const u32x4 pw = __builtin_bit_cast(u32x4, pb[st][u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) lr = add_bf16_pair(pw[e], lr);
      }
  };

  issue_tile(0);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" : : : "memory");

  // Slot s: waves 0..3 run phase s, waves 4..7 phase s - 1; phase 2t is the
  // MFMA phase of tile t, phase 2t + 1 its softmax phase.  Tile t + 1 is
  // requested at the start of slot 2t and waited for at the end of slot
  // 2t + 1; its stage last held tile t - 2, whose V was last read in slot
  // 2t - 1 (the trailing waves' MFMA phase of tile t - 1).  Every wave runs
  // the same 2T + 2 slots and barriers.
  for (int s = 0; s < 2 * T + 2; ++s) {
    if ((s & 1) == 0 && (s >> 1) + 1 < T) issue_tile((s >> 1) + 1);
    const int ph = s - grp;
    if (ph >= 0 && ph <= 2 * T) {
      if ((ph & 1) == 0)
        mfma_phase(ph >> 1);
      else if ((ph >> 1) < T)
        softmax_phase(ph >> 1);
    }
    if (s & 1)
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" : : : "memory");
    else
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" : : : "memory");
  }

  const float lt = halves_sum(l);
  const float lrt = halves_sum(lr);
  if (qrow < N) {
    const float inv = 1.f / lrt;
    char* orow = reinterpret_cast<char*>(o + head) + (size_t)qrow * kRowBytes;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int i = 4 * g;
        u32x2 w = {pack_bf16(acc[mb][i] * inv, acc[mb][i + 1] * inv),
                   pack_bf16(acc[mb][i + 2] * inv, acc[mb][i + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + (32 * mb + 8 * g + 4 * h) * 2) = w;
      }
    if (h == 0) lse[(size_t)bh * N + qrow] = (m + __log2f(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Key-split forward, for grids too small to occupy the chip.
// ---------------------------------------------------------------------------
// With few (batch, head) pairs and a short sequence, one workgroup per 128
// query rows leaves most CUs idle and each wave walks every key tile in turn,
// waiting on memory at each ("Interrogating the GPU, part 5", FlashAttention-2
// section: batch x heads alone does not fill the GPU).  Here a workgroup owns
// 32 query rows and its 4 waves split the keys: wave w takes the 32-key tiles
// w, w + 4, w + 8, ... into LDS of its own (double-buffered, no barrier in the
// loop) and keeps its own online-softmax state (m_w, l_w, O_w).  At the end
// the four partial states merge by the rescale rule of the online softmax:
//   M = max_w m_w,  L = sum_w 2^(m_w - M) l_w,
//   O = sum_w 2^(m_w - M) O_w / L',  LSE = ln2 (M + log2 L),
// where L' merges the same way the sums of P as rounded to bf16 for the P V
// products (so that O is normalised by exactly the weights it was built from),
// through LDS, each wave producing 32 of the 128 output dimensions.
constexpr int SPL_QW = 32;                         // query rows per workgroup
constexpr int SPL_WAVES = 4;
constexpr int SPL_BC = 32;                         // keys per tile
constexpr int SPL_TILE = SPL_BC * kRowBytes;       // 8 KiB (K or V)
constexpr int SPL_WAVE_LDS = 4 * SPL_TILE;         // [buffer][K | V] per wave
constexpr int SPL_SMEM = SPL_WAVES * SPL_WAVE_LDS;  // 128 KiB
constexpr int SPL_LOADS = SPL_TILE / 1024;         // 1 KiB LDS-direct loads per tile and tensor
constexpr int SPL_PART = 64 * 16;                  // floats in one O^T block (64 lanes x 16)
static_assert((SPL_WAVES * SPL_WAVES * SPL_PART + 3 * SPL_WAVES * SPL_QW) * 4 <= SPL_SMEM,
              "the merge buffers must fit the tile buffers they reuse");

template <bool CAUSAL>
__global__ __launch_bounds__(SPL_WAVES * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fwd_split_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                      float* __restrict__ lse, int BH, int N, int nqb, float sl2, uint32_t qkeep,
                      uint32_t qflip) {
  __shared__ __attribute__((aligned(16))) char smem[SPL_SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  int qb, bh;
  block_head(blockIdx.x, nqb, BH, CAUSAL, CAUSAL, &qb, &bh);
  const int q0 = qb * SPL_QW;
  const int qrow = q0 + col;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);

  bf16x8 qf[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc)
    qf[kc] = __builtin_bit_cast(
        bf16x8, signed_operand(buf_load16(rq, (uint32_t)qrow * kRowBytes + (2 * kc + h) * 16), qkeep, qflip));

  const int kend = CAUSAL ? min(N, q0 + SPL_QW) : N;
  const int ntiles = (kend + SPL_BC - 1) / SPL_BC;
  const int nmine = ntiles > wave ? (ntiles - wave + SPL_WAVES - 1) / SPL_WAVES : 0;

  // This wave's LDS: buffer b holds K at b * 2 * SPL_TILE and V after it.
  char* const wlds = smem + wave * SPL_WAVE_LDS;
  const uint32_t wlds_addr = lds_addr(wlds);
  // Load n of a tile fills rows 4 n .. 4 n + 3 (1 KiB, lane-linear); lane i
  // lands on physical chunk i % 16 of its row and fetches the logical chunk
  // the swizzle stores there.  Rows past N read as zero.
  uint32_t ld_voff[SPL_LOADS];
#pragma unroll
  for (int n = 0; n < SPL_LOADS; ++n) {
    const int row = 4 * n + (lane >> 4);
    ld_voff[n] = (uint32_t)row * kRowBytes + (((lane & 15) ^ swz(row)) << 4);
  }
  auto issue = [&](int j, int b) {
    const uint32_t toff = (uint32_t)(wave + SPL_WAVES * j) * SPL_TILE;
    const uint32_t kb = wlds_addr + b * 2 * SPL_TILE;
#pragma unroll
    for (int n = 0; n < SPL_LOADS; ++n) {
      dma16(rk, kb + 1024 * n, ld_voff[n] + toff);
      dma16(rv, kb + SPL_TILE + 1024 * n, ld_voff[n] + toff);
    }
  };

  int koff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) koff[kc] = tile_off(col, 2 * kc + h);
  int voff[4][2];
  {
    const int tr_s = lane & 15;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
    const int tr_row = 4 * h + (tr_s >> 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int dim = 32 * mb + tr_dim;
#pragma unroll
      for (int e = 0; e < 2; ++e) voff[mb][e] = tile_off8(tr_row + 8 * e, dim >> 3, (dim >> 2) & 1);
    }
  }

  f32x16 acc[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mb][i] = 0.f;
  float m = -INFINITY;
  float l = 0.f;   // row sum of P in fp32: the LSE's
  float lr = 0.f;  // row sum of P as rounded to bf16 for the P V product: O's divisor
  // Dividing O by the sum of the same rounded weights that the P V product
  // used keeps O a convex combination of V rows: on rows dominated by one or
  // two keys (large score ranges) the rounding of the dominant P then cancels
  // instead of moving O by up to 2^-9 |V|.

  if (nmine > 0) issue(0, 0);
  for (int j = 0; j < nmine; ++j) {
    const int b = j & 1;
    // Tile j + 1 goes into the other buffer, whose reads (tile j - 1) are
    // complete; then wait for tile j alone.
    if (j + 1 < nmine) {
      issue(j + 1, b ^ 1);
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(2 * SPL_LOADS) : "memory");
    } else {
      dma_drain();
    }
    const char* kb = wlds + b * 2 * SPL_TILE;
    const char* vb = kb + SPL_TILE;
    const int k0 = (wave + SPL_WAVES * j) * SPL_BC;

    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      s = mfma32(__builtin_bit_cast(bf16x8, lds_read16(kb, koff[kc])), qf[kc], s);

    if ((CAUSAL && k0 + SPL_BC - 1 > q0) || k0 + SPL_BC > N) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key >= N || (CAUSAL && key > qrow)) s[i] = -INFINITY;
      }
    }

    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = halves_max(mx);
    const float mcand = mx * sl2;
    if (__builtin_amdgcn_ballot_w64(mcand > m + kTau) != 0) {
      const float mnew = fmaxf(m, mcand);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
      lr *= alpha;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mb][i] *= alpha;
    }
    const float mu = (m == -INFINITY) ? 0.f : m;
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(__builtin_fmaf(s[i], sl2, -mu));
      s[i] = p;
      rs += p;
    }
    l += rs;

#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pb = pack8(s[8 * u], s[8 * u + 1], s[8 * u + 2], s[8 * u + 3], s[8 * u + 4],
                              s[8 * u + 5], s[8 * u + 6], s[8 * u + 7]);
      const u32x4 pw = __builtin_bit_cast(u32x4, pb);
#pragma unroll
      for (int e = 0; e < 4; ++e) lr = add_bf16_pair(pw[e], lr);
      const char* rb = vb + 16 * u * kRowBytes;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb] = mfma32(join(lds_read_tr(rb + voff[mb][0]), lds_read_tr(rb + voff[mb][1])), pb, acc[mb]);
    }
  }

  // Merge.  Every wave's reads and loads are done before the tile buffers
  // are reused: part[w][mb] holds wave w's O^T block mb (element group g of
  // lane x at float4 index 64 g + x), stats[w] its m and row sum per query.
  const float lt = halves_sum(l);
  const float lrt = halves_sum(lr);
  __syncthreads();
  float* part = reinterpret_cast<float*>(smem);
  float* stats = part + SPL_WAVES * SPL_WAVES * SPL_PART;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 w4 = {acc[mb][4 * g], acc[mb][4 * g + 1], acc[mb][4 * g + 2], acc[mb][4 * g + 3]};
      *reinterpret_cast<f32x4*>(part + (wave * SPL_WAVES + mb) * SPL_PART + 4 * (64 * g + lane)) = w4;
    }
  if (h == 0) {
    stats[(3 * wave) * SPL_QW + col] = m;
    stats[(3 * wave + 1) * SPL_QW + col] = lt;
    stats[(3 * wave + 2) * SPL_QW + col] = lrt;
  }
  __syncthreads();

  float mw[SPL_WAVES], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < SPL_WAVES; ++w) {
    mw[w] = stats[(3 * w) * SPL_QW + col];
    M = fmaxf(M, mw[w]);
  }
  float L = 0.f, Lr = 0.f, cw[SPL_WAVES];
#pragma unroll
  for (int w = 0; w < SPL_WAVES; ++w) {
    cw[w] = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);  // a wave without keys adds nothing
    L += cw[w] * stats[(3 * w + 1) * SPL_QW + col];
    Lr += cw[w] * stats[(3 * w + 2) * SPL_QW + col];
  }
  const float inv = 1.f / Lr;
  // This wave writes output dimensions 32 wave .. 32 wave + 31 (block mb = wave).
  f32x16 ob;
#pragma unroll
  for (int i = 0; i < 16; ++i) ob[i] = 0.f;
#pragma unroll
  for (int w = 0; w < SPL_WAVES; ++w)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x4 = *reinterpret_cast<const f32x4*>(part + (w * SPL_WAVES + wave) * SPL_PART +
                                                       4 * (64 * g + lane));
#pragma unroll
      for (int e = 0; e < 4; ++e) ob[4 * g + e] += cw[w] * x4[e];
    }
  if (qrow < N) {
    char* orow = reinterpret_cast<char*>(o + head) + (size_t)qrow * kRowBytes;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int i = 4 * g;
      u32x2 w2 = {pack_bf16(ob[i] * inv, ob[i + 1] * inv), pack_bf16(ob[i + 2] * inv, ob[i + 3] * inv)};
      *reinterpret_cast<u32x2*>(orow + (32 * wave + 8 * g + 4 * h) * 2) = w2;
    }
    if (wave == 0 && h == 0) lse[(size_t)bh * N + qrow] = (M + __log2f(L)) * kLn2;
  }
}

// Below these grid sizes (in 256-row blocks) the key-split kernel runs.
// Measured on B1 with N from 1024 to 8192: non-causal, the key split is
// faster up to 64 row blocks (by 1.3-2.5x) and the row kernel from 128 (by
// 1.3x); causal, where the row blocks also differ in length, the key split is
// faster up to 128 row blocks and the row kernel from 256.
constexpr int kSplitBelow = 128;
constexpr int kSplitBelowCausal = 256;

hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const int nqb = (N + SPL_QW - 1) / SPL_QW;
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  dim3 grid((unsigned)(nqb * BH)), block(SPL_WAVES * 64);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  if (causal)
    hipLaunchKernelGGL(fwd_split_kernel<true>, grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  else
    hipLaunchKernelGGL(fwd_split_kernel<false>, grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  return hipGetLastError();
}

hipError_t launch_fwd_rows(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const int nqb = (N + FWD_BR - 1) / FWD_BR;
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  dim3 grid((unsigned)(nqb * BH)), block(FWD_THREADS);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  if (causal)
    hipLaunchKernelGGL(fwd_kernel<true>, grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  else
    hipLaunchKernelGGL(fwd_kernel<false>, grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  return hipGetLastError();
}

template <int SW>
static void launch_rows_sw(dim3 grid, dim3 block, hipStream_t stream, int causal, const uint16_t* qq,
                           const uint16_t* kk, const uint16_t* vv, uint16_t* oo, float* lse, int BH,
                           int N, int nqb, float sl2, signed_scale sc) {
  if (causal)
    hipLaunchKernelGGL((fwd_kernel<true, SW>), grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  else
    hipLaunchKernelGGL((fwd_kernel<false, SW>), grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
}

hipError_t launch_fwd_soft_exp2(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, float scale, int causal, int share,
                                hipStream_t stream) {
  const int BH = B * H;
  const int nqb = (N + FWD_BR - 1) / FWD_BR;
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  dim3 grid((unsigned)(nqb * BH)), block(FWD_THREADS);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  switch (share) {
    case 0: launch_rows_sw<0>(grid, block, stream, causal, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc); break;
    case 8: launch_rows_sw<8>(grid, block, stream, causal, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc); break;
    case 16: launch_rows_sw<16>(grid, block, stream, causal, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc); break;
    case 32: launch_rows_sw<32>(grid, block, stream, causal, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fwd_pingpong(const void* q, const void* k, const void* v, void* o, float* lse,
                              int B, int H, int N, float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const int nqb = (N + FWD_BR - 1) / FWD_BR;
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  dim3 grid((unsigned)(nqb * BH)), block(FWD_THREADS);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint16_t* kk = static_cast<const uint16_t*>(k);
  const uint16_t* vv = static_cast<const uint16_t*>(v);
  uint16_t* oo = static_cast<uint16_t*>(o);
  if (causal)
    hipLaunchKernelGGL(fwd_pp_kernel<true>, grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  else
    hipLaunchKernelGGL(fwd_pp_kernel<false>, grid, block, 0, stream, qq, kk, vv, oo, lse, BH, N, nqb, sl2, sc.keep, sc.flip);
  return hipGetLastError();
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, float scale, int causal, hipStream_t stream) {
  const long rows_grid = (long)B * H * ((N + FWD_BR - 1) / FWD_BR);
  if (rows_grid < (causal ? kSplitBelowCausal : kSplitBelow))
    return launch_fwd_split(q, k, v, o, lse, B, H, N, scale, causal, stream);
  return launch_fwd_rows(q, k, v, o, lse, B, H, N, scale, causal, stream);
}

}  // namespace fa
