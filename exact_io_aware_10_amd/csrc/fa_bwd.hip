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
// Two launches, no atomics (bitwise deterministic):
//   bwd_dq    per query block: Q, dO in registers; -D = -rowsum(dO o O) and
//             L log2(e) of its rows computed from O, dO and LSE and written
//             to the workspace; K, V tiles stream through LDS;
//             dQ^T += K^T dS^T
//   bwd_dkdv  per key block: K in registers, V in LDS; query tiles of Q, dO,
//             L log2(e), -D (from the workspace) stream through LDS;
//             dV^T += dO^T P, dK^T += Q^T dS
// (bwd_pre, exported as a stage of its own, fills the workspace exactly as
// bwd_dq does, for callers that run the dK/dV kernel alone.)
// Both kernels start each dP accumulation chain from -D instead of zero, so
// their MFMAs produce dP - D and dS = P (dP - D) costs one multiply.
// Tiles reach LDS through LDS-direct buffer loads; rows past N read as zero,
// which makes their P finite and their dO, dP, D and dS zero, so they add
// nothing to any gradient.
#include <mutex>

#include "fa.h"
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

// MFMA with the accumulator in VGPRs, as inline assembly.  In kernels that
// run one wave per SIMD the compiler gives every MFMA an AGPR accumulator;
// the score tiles S and dP are read by VALU code right after, so they are
// kept in VGPRs this way.  Hazards the compiler does not see here:
//   * operands written by VALU need 2 wait states before the MFMA reads them
//     (the leading s_nop 1);
//   * VALU access to the result needs the MFMA drained: mfma_v_fence below
//     (16 wait states) sits between the last MFMA and the first such access.
// Back-to-back accumulation into the same registers needs no wait states.
__device__ __forceinline__ void mfma_v_init(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b) : "memory");
}
__device__ __forceinline__ void mfma_v(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b) : "memory");
}
// The first MFMA of a chain started from c0 instead of zero; c0 must stay
// unwritten for a few wait states after it (the matrix core reads it late).
__device__ __forceinline__ void mfma_v_from(f32x16& c, bf16x8 a, bf16x8 b, const f32x16& c0) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(c) : "v"(a), "v"(b), "v"(c0) : "memory");
}
__device__ __forceinline__ void mfma_v_fence(f32x16& c0, f32x16& c1, f32x16& c2, f32x16& c3) {
  asm volatile("s_nop 15" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
}

// ---------------------------------------------------------------------------
// Pre-pass: -D_i = -sum_k dO_ik O_ik and L_i log2(e).  The sum runs in a
// fixed order that the dQ kernel, which computes the same D in the step,
// follows too, so both give the same bits: each 8-dimension chunk j is an fp32
// chain of fused multiply-adds from zero (dimensions 8 j .. 8 j + 7 in order);
// the chunks of one parity (j = 2 kc + h) are added in the tree
// ((c0 + c1) + (c2 + c3)) + ((c4 + c5) + (c6 + c7)) over kc; the two parities
// are added last.  Sixteen lanes per row, one 16-byte load of O and of dO
// each; the tree is the xor-shuffles 2, 4, 8 (kc), then 1 (h).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float dot_bf16x8(u32x4 a, u32x4 b) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    s = __builtin_fmaf(__uint_as_float(a[j] << 16), __uint_as_float(b[j] << 16), s);
    s = __builtin_fmaf(__uint_as_float(a[j] & 0xffff0000u), __uint_as_float(b[j] & 0xffff0000u), s);
  }
  return s;
}

__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ ws, int rows) {
  const int t = threadIdx.x & 15;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  float c = 0.f;
  if (row < rows) {
    const size_t off = (size_t)row * kD + t * 8;
    c = dot_bf16x8(*reinterpret_cast<const u32x4*>(o + off), *reinterpret_cast<const u32x4*>(dO + off));
  }
  c += __shfl_xor(c, 2);
  c += __shfl_xor(c, 4);
  c += __shfl_xor(c, 8);
  c += __shfl_xor(c, 1);
  if (row < rows && t == 0) {
    ws[row] = -c;
    ws[(size_t)rows + row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK / dV
//
// One wave per SIMD, four waves per workgroup: wave w owns keys
// k0 + 64 w .. + 63 as two groups of 32.  Its K fragments stay in registers
// for the whole kernel and the workgroup's V block sits in LDS; 32-query
// tiles of Q, dO, L log2(e) and -D stream through a four-slot LDS ring.
// Owning 64 keys lets each Q / dO fragment read from LDS feed two MFMAs.
// The accumulators dK^T, dV^T (256 registers) live in AGPRs; S and dP are
// computed by VGPR-accumulator MFMAs (mfma_v) so that the softmax can read
// them directly.
// ---------------------------------------------------------------------------
constexpr int KV_BK = 256;                   // keys per workgroup
constexpr int KV_WAVES = 4;                  // 64 keys per wave
constexpr int KV_BQ = 32;                    // queries per streamed tile
constexpr int KV_TILE = KV_BQ * kRowBytes;   // 8 KiB (Q or dO)
constexpr int KV_VBLK = KV_BK * kRowBytes;   // 64 KiB
constexpr int KV_THREADS = KV_WAVES * 64;
constexpr int KV_TLOADS = KV_TILE / 1024 / KV_WAVES;  // LDS-direct loads per wave per tensor
constexpr int KV_VLOADS = KV_VBLK / 1024 / KV_WAVES;
// LDS layout: the ring's Q / dO tiles first, so that every constant offset
// into them fits the 16-bit offset field of LDS instructions (no address
// adds); then per slot four 64-entry float arrays (L log2(e), -D, and two
// sinks: the 4-byte LDS-direct load writes one entry per lane, and every wave
// issues one so that all waves issue the same number of loads); then the V
// block, addressed from a base register.
constexpr int KV_NSLOT = 4;
constexpr int KV_SLOT = 2 * KV_TILE;                       // Q tile, dO tile
constexpr int KV_LD_OFF = KV_NSLOT * KV_SLOT;              // 64 KiB
constexpr int KV_LD_SLOT = 4 * 256;
constexpr int KV_V_OFF = KV_LD_OFF + KV_NSLOT * KV_LD_SLOT;
constexpr int KV_LOADS_PER_TILE = 2 * KV_TLOADS + 1;
static_assert(KV_LOADS_PER_TILE == 5, "the ring wait below counts 5 loads per tile");
static_assert((KV_NSLOT - 1) * KV_SLOT + KV_TILE + KV_TILE / 2 < 65536,
              "ring offsets must fit the LDS offset field");
static_assert(KV_V_OFF % 256 == 0, "the V base must leave the chunk-swizzle bits free");
constexpr int KV_SMEM = KV_V_OFF + KV_VBLK;

template <int V>
struct kv_ic {
  static constexpr int value = V;
};

// Hides x from loop-invariant code motion: an LDS address built from it
// stays "register + constant offset" instead of one hoisted register each.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <bool CAUSAL>
__global__ __launch_bounds__(KV_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                     const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
                     const float* __restrict__ ws, uint16_t* __restrict__ dk,
                     uint16_t* __restrict__ dv, int BH, int N, float sl2, float scale,
                     uint32_t kkeep, uint32_t kflip) {
  __shared__ __attribute__((aligned(16))) char smem[KV_SMEM];
  const uint32_t smem_lds = lds_addr(smem);  // LDS byte address of smem (wave-uniform)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  // Causal: the first key blocks see the most queries; issue them first.
  int kb, bh;
  block_head(blockIdx.x, (N + KV_BK - 1) / KV_BK, BH, false, CAUSAL, &kb, &bh);
  const int k0 = kb * KV_BK;
  const int kw = k0 + 64 * wave;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const size_t rows = (size_t)BH * N;
  const rsrc_t rD = make_rsrc(ws + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rL = make_rsrc(ws + rows + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rLD = (wave & 1) ? rD : rL;

  // V block: instruction n of wave w fills rows 16 n + 4 w .. + 3.
  const int ld_sub = lane >> 4;
  const int ld_pc = lane & 15;
#pragma unroll
  for (int n = 0; n < KV_VLOADS; ++n) {
    const int row0 = 16 * n + 4 * wave;
    const int row = row0 + ld_sub;
    dma16(rv, smem_lds + KV_V_OFF + row0 * kRowBytes,
          (uint32_t)(k0 + row) * kRowBytes + ((ld_pc ^ swz(row)) << 4));
  }
  // K as the B operand of S = Q K^T: lane holds K[kw + 32 g + col][16 kc + 8 h .. + 7],
  // negated for a negative scale and cleared for scale 0 (sl2 is |scale| log2 e;
  // dK = scale dS^T Q takes the signed scale at the store).
  bf16x8 kf[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc)
      kf[g][kc] = __builtin_bit_cast(
          bf16x8, signed_operand(buf_load16(rk, (uint32_t)(kw + 32 * g + col) * kRowBytes + (2 * kc + h) * 16),
                                 kkeep, kflip));
  // Touch kf once here: the compiler waits for the loads at this point, and
  // knows from then on that they have arrived.
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) asm volatile("" : : "v"(kf[g][kc]));

  uint32_t ld_voff[KV_TLOADS];
#pragma unroll
  for (int n = 0; n < KV_TLOADS; ++n) {
    const int row = 16 * n + 4 * wave + ld_sub;
    ld_voff[n] = (uint32_t)row * kRowBytes + ((ld_pc ^ swz(row)) << 4);
  }
  // Loads of tile t into ring slot `sl`.  Issued even past the last tile
  // (those read zeros), so every wave always has exactly 5 per tile in flight.
  auto issue_tile = [&](int t, int sl) {
    const uint32_t base = smem_lds + sl * KV_SLOT;
    const uint32_t toff = (uint32_t)t * KV_TILE;
#pragma unroll
    for (int n = 0; n < KV_TLOADS; ++n) {
      const int row0 = 16 * n + 4 * wave;
      dma16(rq, base + row0 * kRowBytes, ld_voff[n] + toff);
      dma16(rdo, base + KV_TILE + row0 * kRowBytes, ld_voff[n] + toff);
    }
    dma4(rLD, smem_lds + KV_LD_OFF + sl * KV_LD_SLOT + 256 * wave, (uint32_t)(t * KV_BQ + lane) * 4);
  };

  // Per-lane LDS offsets, tile-relative:
  //   row operands: row col, logical chunk 2 kc + h (V rows add 64 w + 32 g);
  //   transpose reads: row 4 h + (lane % 16) / 4 (+ 8 e, + 16 u),
  //   dims 32 mb + 16 ((lane / 16) % 2) + 4 (lane % 4).
  int roff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) roff[kc] = tile_off(col, 2 * kc + h);
  int troff[4][2];
  {
    const int tr_s = lane & 15;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
    const int tr_row = 4 * h + (tr_s >> 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int dim = 32 * mb + tr_dim;
#pragma unroll
      for (int e = 0; e < 2; ++e) troff[mb][e] = tile_off8(tr_row + 8 * e, dim >> 3, (dim >> 2) & 1);
    }
  }
  // This wave's rows of the V block (a multiple of 256: the chunk XOR below
  // only touches bits 5..7).
  const int vrow = KV_V_OFF + 64 * wave * kRowBytes;

  f32x16 dka[2][4], dva[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dka[g][mb][i] = 0.f;
        dva[g][mb][i] = 0.f;
      }

  const int t0 = CAUSAL ? (k0 / KV_BQ) : 0;
  const int ntiles = (N + KV_BQ - 1) / KV_BQ;

  // P and dS of the previous tile, packed for the dV / dK products.  They
  // start at zero: the first step multiplies them into a slot that holds
  // zeros (cleared below) or an earlier tile, which adds nothing.
  bf16x8 pb[2][2], sb[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pb[g][u] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      sb[g][u] = pb[g][u];
    }

  // dV^T += dO^T P and dK^T += Q^T dS for the tile in ring slot `psl`
  // (transposed operands from transpose reads, one (mb, u) step ahead).
  // tro: transpose-read lane offsets (troff, passed through opaque() by the
  // caller outside the region the products are scheduled in).
  auto dvdk = [&](int psl, const int (&tro)[4][2]) {
    const int qsl = psl * KV_SLOT, osl = qsl + KV_TILE;
    bf16x8 a_do[2], a_q[2];
    auto rdt = [&](int n, int b) {
      const int mb = n >> 1, ro2 = 16 * (n & 1) * kRowBytes;
      a_do[b] = join(lds_read_tr(smem + osl + ro2 + tro[mb][0]), lds_read_tr(smem + osl + ro2 + tro[mb][1]));
      a_q[b] = join(lds_read_tr(smem + qsl + ro2 + tro[mb][0]), lds_read_tr(smem + qsl + ro2 + tro[mb][1]));
    };
    rdt(0, 0);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int b = n & 1, mb = n >> 1, u = n & 1;
      if (n < 7) rdt(n + 1, b ^ 1);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        dva[g][mb] = mfma32(a_do[b], pb[g][u], dva[g][mb]);
        dka[g][mb] = mfma32(a_q[b], sb[g][u], dka[g][mb]);
      }
    }
  };

  auto step = [&](int t, auto bc) {
    constexpr int sl = decltype(bc)::value;
    constexpr int psl = (sl + KV_NSLOT - 1) % KV_NSLOT;  // slot of tile t - 1
    constexpr int qsl = sl * KV_SLOT;                    // smem offsets of this slot's parts
    constexpr int osl = qsl + KV_TILE;
    constexpr int lsl = KV_LD_OFF + sl * KV_LD_SLOT;
    constexpr int dsl = lsl + 256;
    // Tile t has landed once only tile t + 1's loads may be in flight; the
    // barrier then publishes every wave's part of it and frees the slot that
    // tile t - 2 used, which tile t + 2 takes (tile t - 1 is still read here).
    ring_wait_barrier<KV_LOADS_PER_TILE>();
    issue_tile(t + 2, (sl + 2) % KV_NSLOT);
    const int qs = t * KV_BQ;
    if (CAUSAL && qs < kw) return;  // every query of the tile precedes every key of the wave

    // Lane offsets from three base registers: logical chunk bits only flip
    // physical chunk bits under the XOR swizzle, so a row operand's chunk
    // 2 kc + h sits at roff[0] ^ (32 kc) and a transpose read's dims 32 mb +
    // ... at troff[0][e] ^ (64 mb).
    const int ro0 = opaque(roff[0]);
    const int rv0 = opaque(roff[0] + vrow);
    const int tr0 = opaque(troff[0][0]), tr1 = opaque(troff[0][1]);
    int ro[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) ro[kc] = ro0 ^ (32 * kc);
    int tro[4][2];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      tro[mb][0] = tr0 ^ (64 * mb);
      tro[mb][1] = tr1 ^ (64 * mb);
    }

    // S = Q K^T and dP - D = dO V^T - D, operands one k-step ahead.  The dP
    // chains start from -D of each element's query (the tile's -D array holds
    // it at the same positions the accumulator tuple does: 4 (i / 4) entries
    // apart, 4 h + i % 4 in), the same for both key groups.
    const float* db = reinterpret_cast<const float*>(smem + dsl);
    f32x16 nd;
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(db + 8 * gg + 4 * h);
#pragma unroll
      for (int j = 0; j < 4; ++j) nd[4 * gg + j] = d4[j];
    }
    f32x16 s[2], dp[2];
    bf16x8 qa[2], da[2], va[2][2];
    auto rd = [&](int kc, int b) {
      qa[b] = __builtin_bit_cast(bf16x8, lds_read16(smem + qsl, ro[kc]));
      da[b] = __builtin_bit_cast(bf16x8, lds_read16(smem + osl, ro[kc]));
      // V rows: the chunk swizzle depends on the row only through col.
      const int vo = rv0 ^ (32 * kc);
      va[b][0] = __builtin_bit_cast(bf16x8, lds_read16(smem, vo));
      va[b][1] = __builtin_bit_cast(bf16x8, lds_read16(smem + 32 * kRowBytes, vo));
    };
    rd(0, 0);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int b = kc & 1;
      if (kc < 7) rd(kc + 1, b ^ 1);
      if (kc == 0) {
        mfma_v_init(s[0], qa[b], kf[0][kc]);
        mfma_v_from(dp[0], da[b], va[b][0], nd);
        mfma_v_init(s[1], qa[b], kf[1][kc]);
        mfma_v_from(dp[1], da[b], va[b][1], nd);
      } else {
        mfma_v(s[0], qa[b], kf[0][kc]);
        mfma_v(dp[0], da[b], va[b][0]);
        mfma_v(s[1], qa[b], kf[1][kc]);
        mfma_v(dp[1], da[b], va[b][1]);
      }
      // The matrix core reads nd for a while after the MFMAs issue: keep its
      // registers from reuse until the next k-step's MFMAs have issued.
      if (kc == 1) asm volatile("" : : "v"(nd));
    }
    mfma_v_fence(s[0], s[1], dp[0], dp[1]);

    // Causal mask, only on the (at most two) tiles that cross the diagonal:
    // S = -inf where the key follows the query, so P and dS come out zero.
    // Element i of a lane is query qs + 8 (i / 4) + 4 h + i % 4 against key
    // kw + 32 g + col.
    if (CAUSAL && qs < kw + 64) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int key = kw + 32 * g + col;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (key > qs + 8 * (i >> 2) + 4 * h + (i & 3)) s[g][i] = -INFINITY;
      }
    }

    // P = exp2(S scale log2(e) - L log2(e)), dS = P (dP - D), interleaved
    // by hand with the dV / dK products of the previous tile: product step
    // n (4 MFMAs) carries the softmax of row group n / 2, key group n % 2,
    // one element per MFMA; sched_barrier keeps the compiler to that order.
    const float* lb = reinterpret_cast<const float*>(smem + lsl);
    const int pq = psl * KV_SLOT, po = pq + KV_TILE;
    bf16x8 a_do[2], a_q[2];
    f32x4 l4[2];
    // Product step n covers query half u = n / 4 of the previous tile and
    // output block mb = n % 4, so that the packed P and dS of half u are last
    // read at step 4 u + 3 and this tile's can take their registers there.
    auto rdt = [&](int n, int b) {
      const int mb = n & 3, ro2 = 16 * (n >> 2) * kRowBytes;
      a_do[b] = join(lds_read_tr(smem + po + ro2 + tro[mb][0]), lds_read_tr(smem + po + ro2 + tro[mb][1]));
      a_q[b] = join(lds_read_tr(smem + pq + ro2 + tro[mb][0]), lds_read_tr(smem + pq + ro2 + tro[mb][1]));
    };
    auto rdl = [&](int gg) {
      const int r = 8 * gg + 4 * h;
      l4[gg & 1] = *reinterpret_cast<const f32x4*>(lb + r);
    };
    rdt(0, 0);
    rdl(0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int b = n & 1, mb = n & 3, u = n >> 2;
      const int gg = n >> 1, g = n & 1;
      if (n < 7) rdt(n + 1, b ^ 1);
      if (g == 1 && gg < 3) rdl(gg + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int gk = k >> 1;
        if ((k & 1) == 0)
          dva[gk][mb] = mfma32(a_do[b], pb[gk][u], dva[gk][mb]);
        else
          dka[gk][mb] = mfma32(a_q[b], sb[gk][u], dka[gk][mb]);
        const int i = 4 * gg + k;
        const float p = fast_exp2(__builtin_fmaf(s[g][i], sl2, -l4[gg & 1][k]));
        s[g][i] = p;
        dp[g][i] = p * dp[g][i];  // dp holds dP - D
        __builtin_amdgcn_sched_barrier(0);
      }
      // Rows 8 v .. 8 v + 7 (row groups 2 v, 2 v + 1) of both key groups are
      // done after step 4 v + 3, the last that reads the previous tile's half
      // v: pack this tile's into those registers.
      if ((n & 3) == 3) {
        const int v = n >> 2, e = 8 * v;
#pragma unroll
        for (int gk = 0; gk < 2; ++gk) {
          pb[gk][v] = pack8(s[gk][e], s[gk][e + 1], s[gk][e + 2], s[gk][e + 3], s[gk][e + 4],
                            s[gk][e + 5], s[gk][e + 6], s[gk][e + 7]);
          sb[gk][v] = pack8(dp[gk][e], dp[gk][e + 1], dp[gk][e + 2], dp[gk][e + 3], dp[gk][e + 4],
                            dp[gk][e + 5], dp[gk][e + 6], dp[gk][e + 7]);
        }
      }
    }
  };

  // Slot 3 feeds the first step's dV / dK products: clear it.
  {
    char* z = smem + 3 * KV_SLOT;
    for (int o = tid * 16; o < KV_SLOT; o += KV_THREADS * 16) lds_write16(z, o, u32x4{0u, 0u, 0u, 0u});
  }
  issue_tile(t0, 0);
  issue_tile(t0 + 1, 1);
  for (int t = t0; t < ntiles; t += 4) {
    step(t, kv_ic<0>{});
    if (t + 1 < ntiles) step(t + 1, kv_ic<1>{});
    if (t + 2 < ntiles) step(t + 2, kv_ic<2>{});
    if (t + 3 < ntiles) step(t + 3, kv_ic<3>{});
  }
  // The last tile's dV / dK products.
  if (ntiles > t0) {
    const int lsl_ = (ntiles - 1 - t0) & 3;
    __syncthreads();
    dvdk(lsl_, troff);
  }
  dma_drain();  // no LDS-direct load may outlive the workgroup

#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int krow = kw + 32 * g + col;
    if (krow < N) {
      char* dkrow = reinterpret_cast<char*>(dk + head) + (size_t)krow * kRowBytes;
      char* dvrow = reinterpret_cast<char*>(dv + head) + (size_t)krow * kRowBytes;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int i = 4 * gg;
          const int off = (32 * mb + 8 * gg + 4 * h) * 2;
          u32x2 wk = {pack_bf16(dka[g][mb][i] * scale, dka[g][mb][i + 1] * scale),
                      pack_bf16(dka[g][mb][i + 2] * scale, dka[g][mb][i + 3] * scale)};
          u32x2 wv = {pack_bf16(dva[g][mb][i], dva[g][mb][i + 1]),
                      pack_bf16(dva[g][mb][i + 2], dva[g][mb][i + 3])};
          *reinterpret_cast<u32x2*>(dkrow + off) = wk;
          *reinterpret_cast<u32x2*>(dvrow + off) = wv;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ
//
// One wave per SIMD, four waves per workgroup: wave w owns queries
// q0 + 64 w .. + 63 as two groups of 32, with their Q and dO fragments (the B
// operands of S^T = K Q^T and dP^T = V dO^T) loaded once, Q into AGPRs, and
// the dQ^T accumulators (128 registers) in AGPRs as well.  32-key tiles of K and V
// stream through a five-slot LDS ring.  Owning 64 queries lets every K or V
// fragment read from LDS feed two MFMAs.  Before the loop the kernel also
// loads O beside dO and forms -D = -rowsum(dO o O) and L log2(e) of its
// queries, which its dP chains start from and which it writes to the
// workspace for the dK/dV kernel (no pre-pass launch).  Per tile t and wave:
//   A  S^T  = K_t Q^T      16 MFMAs (VGPR accumulators, inline assembly)
//   B  dP^T - D = V_t dO^T - D   16 MFMAs (the chain starts from -D of the
//                          lane's query), interleaved with P = exp2(S scale
//                          log2 e - L log2 e) of tile t
//   the ring barrier for tile t + 1, and that tile's first K reads
//   C  dQ^T += K_{t-1}^T dS_{t-1}^T   16 MFMAs, interleaved with
//                          dS = P (dP - D) of tile t (one multiply), packed to bf16
// ---------------------------------------------------------------------------
constexpr int DQ_QW = 64;                    // queries per wave
constexpr int DQ_WAVES = 4;
constexpr int DQ_BQ = DQ_QW * DQ_WAVES;      // queries per workgroup
constexpr int DQ_BK = 32;                    // keys per streamed tile
constexpr int DQ_TILE = DQ_BK * kRowBytes;   // 8 KiB (K or V)
constexpr int DQ_THREADS = DQ_WAVES * 64;
constexpr int DQ_TLOADS = DQ_TILE / 1024 / DQ_WAVES;  // LDS-direct loads per wave per tensor
constexpr int DQ_SLOT = 2 * DQ_TILE;                  // K tile, then V tile
constexpr int DQ_NSLOT = 5;
constexpr int DQ_SMEM = DQ_NSLOT * DQ_SLOT;           // 80 KiB
constexpr int DQ_LOADS_PER_TILE = 2 * DQ_TLOADS;
constexpr int DQ_AHEAD = 3;                           // LDS read-ahead of phases A and B, in k-steps
constexpr int DQ_CA = 3;                              // LDS read-ahead of phase C, in product steps
constexpr int DQ_CPRE = 4;                            // phase B k-step after which phase C's first reads issue

// S^T / dP^T MFMA with the B operand (Q^T or dO^T) in AGPRs and the result in
// VGPRs; hazards as for mfma_v (s_fence2 after the last one).
__device__ __forceinline__ void mfma_va0(f32x16& c, bf16x8 a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b) : "memory");
}
__device__ __forceinline__ void mfma_va(f32x16& c, bf16x8 a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b) : "memory");
}
// dQ^T += A B with the accumulator in AGPRs (fenced by acc_fence8).
__device__ __forceinline__ void mfma_aa(f32x16& c, bf16x8 a, bf16x8 b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void acc_fence8(f32x16 (&c)[2][4]) {
  asm volatile("s_nop 15"
               : "+a"(c[0][0]), "+a"(c[0][1]), "+a"(c[0][2]), "+a"(c[0][3]), "+a"(c[1][0]),
                 "+a"(c[1][1]), "+a"(c[1][2]), "+a"(c[1][3]));
}
__device__ __forceinline__ void s_fence2(f32x16& c0, f32x16& c1) {
  asm volatile("s_nop 15" : "+v"(c0), "+v"(c1));
}

template <bool CAUSAL>
__global__ __launch_bounds__(DQ_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                   const uint16_t* __restrict__ v, const uint16_t* __restrict__ o,
                   const uint16_t* __restrict__ dO, const float* __restrict__ lse,
                   float* __restrict__ ws, uint16_t* __restrict__ dq, int BH, int N, int nqb,
                   float sl2, float scale, uint32_t qkeep, uint32_t qflip) {
  __shared__ __attribute__((aligned(16))) char smem[DQ_SMEM];
  const uint32_t smem_lds = lds_addr(smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  // Causal: issue the longest query blocks first.
  int qblk, bh;
  block_head(blockIdx.x, nqb, BH, CAUSAL, CAUSAL, &qblk, &bh);
  const int q0 = qblk * DQ_BQ;
  const int q0w = q0 + DQ_QW * wave;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const size_t rows = (size_t)BH * N;
  const rsrc_t ro = make_rsrc(o + head, head_bytes);
  const rsrc_t rL = make_rsrc(lse + (size_t)bh * N, (uint32_t)N * 4);

  // Q^T and dO^T as B operands (zero past N): lane holds
  // Q[q0w + 32 g + col][16 kc + 8 h .. + 7].  Q is negated for a negative
  // scale and cleared for scale 0 (sl2 is |scale| log2 e; dQ = scale dS K
  // takes the signed scale at the store), then moved to AGPRs.  Both are
  // ordinary (compiler-tracked) loads, so that no copy of a fragment the
  // register allocator makes can run ahead of the data.
  // O's fragments are loaded beside them (for D below), so that the three
  // loads' latencies overlap.
  bf16x8 qf[2][8], df[2][8];
  u32x4 qraw[2][8], oraw[2][8];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const uint32_t off = (uint32_t)(q0w + 32 * g + col) * kRowBytes + (2 * kc + h) * 16;
      qraw[g][kc] = buf_load16(rq, off);
      df[g][kc] = __builtin_bit_cast(bf16x8, buf_load16(rdo, off));
      oraw[g][kc] = buf_load16(ro, off);
    }
  float lraw[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) lraw[g] = buf_load_f32(rL, (uint32_t)(q0w + 32 * g + col) * 4);
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8 qv = __builtin_bit_cast(bf16x8, signed_operand(qraw[g][kc], qkeep, qflip));
      asm volatile("" : "=a"(qf[g][kc]) : "0"(qv));
    }
  // -D = -rowsum(dO o O) and L log2(e) of the lane's queries ("Interrogating
  // the GPU, part 5", section "What does the backward pass do without P?":
  // delta), summed in the pre-pass's order (one chain per 8-dimension chunk,
  // this lane's chunks kc = 0..7 added as a tree, then the other half of the
  // dimensions from lane ^ 32), and written to the workspace for the dK/dV
  // kernel; rows past N read as zero.
  float l2[2], nd[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int qr = q0w + 32 * g + col;
    float c[8];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) c[kc] = dot_bf16x8(oraw[g][kc], __builtin_bit_cast(u32x4, df[g][kc]));
    float sd = ((c[0] + c[1]) + (c[2] + c[3])) + ((c[4] + c[5]) + (c[6] + c[7]));
    sd += __shfl_xor(sd, 32);
    nd[g] = -sd;
    l2[g] = lraw[g] * kLog2e;
    if (h == 0 && qr < N) {
      ws[(size_t)bh * N + qr] = nd[g];
      ws[rows + (size_t)bh * N + qr] = l2[g];
    }
  }
  // Wait for L here, in the compiler's view as well, before any LDS-direct
  // load (invisible to it) is in flight.
  asm volatile("" : : "v"(l2[0]), "v"(l2[1]), "v"(nd[0]), "v"(nd[1]));
  // -D of the lane's query in every element: the dP^T chain starts from it,
  // so that its MFMAs produce dP - D and dS = P (dP - D) is one multiply.
  f32x16 ndd[2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int i = 0; i < 16; ++i) ndd[g][i] = nd[g];

  // Tiles the workgroup streams, and tiles this wave computes on.
  const int kend = CAUSAL ? min(N, q0 + DQ_BQ) : N;
  const int nt = (kend + DQ_BK - 1) / DQ_BK;
  const int wend = CAUSAL ? min(N, q0w + DQ_QW) : N;
  const int tw = (q0w < N) ? (wend + DQ_BK - 1) / DQ_BK : 0;
  // First tile that needs an element-wise mask (causal diagonal or keys >= N).
  const int tmask = CAUSAL ? min(q0w / DQ_BK, N / DQ_BK) : N / DQ_BK;

  // Tile loader: instruction n of wave w fills rows 16 n + 4 w .. + 3 of the
  // K and V tiles of a slot (rows past N read as zero).
  const int ld_sub = lane >> 4;
  const int ld_pc = lane & 15;
  uint32_t ld_voff[DQ_TLOADS];
#pragma unroll
  for (int n = 0; n < DQ_TLOADS; ++n) {
    const int row = 16 * n + 4 * wave + ld_sub;
    ld_voff[n] = (uint32_t)row * kRowBytes + ((ld_pc ^ swz(row)) << 4);
  }
  auto issue_tile = [&](int t, int sl) {
    const uint32_t base = smem_lds + sl * DQ_SLOT;
    const uint32_t toff = (uint32_t)t * DQ_TILE;
#pragma unroll
    for (int n = 0; n < DQ_TLOADS; ++n) {
      const int row0 = 16 * n + 4 * wave;
      dma16(rk, base + row0 * kRowBytes, ld_voff[n] + toff);
      dma16(rv, base + DQ_TILE + row0 * kRowBytes, ld_voff[n] + toff);
    }
  };

  // Per-lane LDS offsets, tile-relative:
  //   row operands (K, V): row col, logical chunk 2 kc + h;
  //   K^T transpose reads: row 4 h + (lane % 16) / 4 (+ 8 e, + 16 u),
  //   dims 32 mb + 16 ((lane / 16) % 2) + 4 (lane % 4).
  int roff[8];
#pragma unroll
  for (int kc = 0; kc < 8; ++kc) roff[kc] = tile_off(col, 2 * kc + h);
  int troff[4][2];
  {
    const int tr_s = lane & 15;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (tr_s & 3);
    const int tr_row = 4 * h + (tr_s >> 2);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int dim = 32 * mb + tr_dim;
#pragma unroll
      for (int e = 0; e < 2; ++e) troff[mb][e] = tile_off8(tr_row + 8 * e, dim >> 3, (dim >> 2) & 1);
    }
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][mb][i] = 0.f;

  // dS^T of the previous tile as B operands [group][key half]; zero before the
  // first tile, whose products read the K part of the last slot, cleared below.
  bf16x8 sb[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int u = 0; u < 2; ++u) sb[g][u] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

  // Causal / tail mask of tile t on s: element i of a lane is key
  // 32 t + 4 h + c_i, c_i = 8 (i / 4) + i % 4, masked when c_i >= lim.
  auto mask_tile = [&](int t, f32x16 (&s)[2]) {
    const int base = t * DQ_BK + 4 * h;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      int lim = N - base;
      if (CAUSAL) lim = min(lim, q0w + 32 * g + col - base + 1);
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= lim) s[g][i] = -INFINITY;
    }
  };

  // dQ^T += K^T dS^T for the tile in slot psl (phase C), with sb.  Its K^T
  // fragments are read DQ_CA product steps (2 DQ_CA MFMAs) ahead, the first
  // DQ_CA of them by dq_prefetch, which the step issues during phase B.
  bf16x8 ca[DQ_CA + 1];
  auto rdt = [&](int psl, int n) {
    const char* rb = smem + psl * DQ_SLOT + 16 * (n >> 2) * kRowBytes;
    const int mb = n & 3;
    ca[n % (DQ_CA + 1)] = join(lds_read_tr(rb + troff[mb][0]), lds_read_tr(rb + troff[mb][1]));
  };
  auto dq_prefetch = [&](int psl) {
#pragma unroll
    for (int n = 0; n < DQ_CA; ++n) rdt(psl, n);
  };
  auto dq_products = [&](int psl, auto&& between) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int b = n % (DQ_CA + 1), mb = n & 3, u = n >> 2;
      if (n + DQ_CA < 8) rdt(psl, n + DQ_CA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        mfma_aa(acc[g][mb], ca[b], sb[g][u]);
        between(2 * n + g);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // In the same basic block as the MFMAs: later accesses to the
    // accumulators, the register allocator's copies included, come after it.
    acc_fence8(acc);
  };

  // The ring: tile j is in slot j % 5.  The barrier W(j) (ring_wait_barrier)
  // waits until this wave's loads of tile j have landed (only tile j + 1's
  // may still be in flight), publishes every wave's part of it, and is
  // followed by the loads of tile j + 2.  Every wave passes W(0) .. W(nt).
  // K fragments of phase A, read DQ_AHEAD k-steps before their MFMAs (two
  // MFMAs per step are too short to cover the LDS latency); the first
  // DQ_AHEAD of a tile are read before the previous step's phase C, so that
  // its MFMAs cover their latency.
  bf16x8 ka[DQ_AHEAD + 1];
  auto ka_prefetch = [&](int sl) {
#pragma unroll
    for (int j = 0; j < DQ_AHEAD; ++j) ka[j] = __builtin_bit_cast(bf16x8, lds_read16(smem + sl * DQ_SLOT, roff[j]));
  };

  // Step t (slot SL = t % 5, a compile-time constant so that every LDS
  // offset into the slot folds into the instructions): phases A and B of
  // tile t; then W(t + 1), whose barrier also frees the slot of tile t - 2
  // (last read in the previous step's phase C) for tile t + 3; then phase C,
  // the dQ products of tile t - 1 (zero dS before the first tile), whose
  // slot the new loads do not touch.
  auto step = [&](int t, auto slc) {
    constexpr int SL = decltype(slc)::value;
    constexpr int PSL = (SL + DQ_NSLOT - 1) % DQ_NSLOT;
    constexpr int NSL = (SL + 1) % DQ_NSLOT;
    const char* kb = smem + SL * DQ_SLOT;
    const char* vb = kb + DQ_TILE;

    // Phase A: S^T for both query groups; V's first fragments are read
    // during the last K steps.
    f32x16 s[2], dp[2];
    bf16x8 va[DQ_AHEAD + 1];
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int b = kc % (DQ_AHEAD + 1);
      if (kc + DQ_AHEAD < 8)
        ka[(kc + DQ_AHEAD) % (DQ_AHEAD + 1)] = __builtin_bit_cast(bf16x8, lds_read16(kb, roff[kc + DQ_AHEAD]));
      else
        va[kc + DQ_AHEAD - 8] = __builtin_bit_cast(bf16x8, lds_read16(vb, roff[kc + DQ_AHEAD - 8]));
      if (kc == 0) {
        mfma_va0(s[0], ka[b], qf[0][kc]);
        mfma_va0(s[1], ka[b], qf[1][kc]);
      } else {
        mfma_va(s[0], ka[b], qf[0][kc]);
        mfma_va(s[1], ka[b], qf[1][kc]);
      }
    }
    s_fence2(s[0], s[1]);
    if (t >= tmask) mask_tile(t, s);

    // Phase B: dP^T, with P = exp2(S scale log2 e - L log2 e) in between
    // (two scores per MFMA, written over S).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const int b = kc % (DQ_AHEAD + 1);
      if (kc + DQ_AHEAD < 8)
        va[(kc + DQ_AHEAD) % (DQ_AHEAD + 1)] = __builtin_bit_cast(bf16x8, lds_read16(vb, roff[kc + DQ_AHEAD]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        if (kc == 0)
          mfma_v_from(dp[g], va[b], df[g][kc], ndd[g]);
        else
          mfma_v(dp[g], va[b], df[g][kc]);
        const int idx = 2 * (2 * kc + g);  // scores idx, idx + 1 of the 32
        const int sg = idx >> 4, si = idx & 15;
        s[sg][si] = fast_exp2(__builtin_fmaf(s[sg][si], sl2, -l2[sg]));
        s[sg][si + 1] = fast_exp2(__builtin_fmaf(s[sg][si + 1], sl2, -l2[sg]));
        // Here, between this MFMA and the next, not bunched after the last
        // one (where the compiler otherwise puts them).
        asm volatile("" : "+v"(s[sg][si]), "+v"(s[sg][si + 1]));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kc == DQ_CPRE) dq_prefetch(PSL);
      __builtin_amdgcn_sched_barrier(0);
    }
    s_fence2(dp[0], dp[1]);

    ring_wait_barrier<DQ_LOADS_PER_TILE>();  // W(t + 1)
    issue_tile(t + 3, (SL + 3) % DQ_NSLOT);
    if (t + 1 < tw) ka_prefetch(NSL);

    // Phase C: dQ products of tile t - 1, with dS = P (dP - D) of tile t in
    // between, packed into the next step's B operands.
    uint32_t w[2][8];
    dq_products(PSL, [&](int m) {
      const int idx = 2 * m;
      const int sg = idx >> 4, si = idx & 15;
      const float d0 = s[sg][si] * dp[sg][si];  // dp holds dP - D
      const float d1 = s[sg][si + 1] * dp[sg][si + 1];
      w[sg][si >> 1] = pack_bf16(d0, d1);
      asm volatile("" : "+v"(w[sg][si >> 1]));  // convert here, not after the loop
    });
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        sb[g][u] = __builtin_bit_cast(bf16x8, u32x4{w[g][4 * u], w[g][4 * u + 1], w[g][4 * u + 2], w[g][4 * u + 3]});
  };

  // The last slot (that of tile -1) feeds the first step's dQ products:
  // clear its K tile (published by W(0)).
  {
    char* z = smem + (DQ_NSLOT - 1) * DQ_SLOT;
    for (int o = tid * 16; o < DQ_TILE; o += DQ_THREADS * 16) lds_write16(z, o, u32x4{0u, 0u, 0u, 0u});
  }
  issue_tile(0, 0);
  issue_tile(1, 1);
  ring_wait_barrier<DQ_LOADS_PER_TILE>();  // W(0)
  issue_tile(2, 2);
  if (tw > 0) ka_prefetch(0);
  static_assert(DQ_NSLOT == 5, "the step loop is unrolled over the five slots");
  for (int t = 0; t < tw; t += 5) {
    step(t, kv_ic<0>{});
    if (t + 1 < tw) step(t + 1, kv_ic<1>{});
    if (t + 2 < tw) step(t + 2, kv_ic<2>{});
    if (t + 3 < tw) step(t + 3, kv_ic<3>{});
    if (t + 4 < tw) step(t + 4, kv_ic<4>{});
  }
  // The last tile's dQ products (its slot is refilled only at W(tw + 2));
  // then the wave only keeps the ring going up to the workgroup's W(nt).
  if (tw > 0) {
    dq_prefetch((tw - 1) % DQ_NSLOT);
    dq_products((tw - 1) % DQ_NSLOT, [](int) {});
  }
  for (int tt = tw + 1; tt <= nt; ++tt) {
    ring_wait_barrier<DQ_LOADS_PER_TILE>();
    issue_tile(tt + 2, (tt + 2) % DQ_NSLOT);
  }
  dma_drain();  // no LDS-direct load may outlive the workgroup

  if (tw > 0) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int qrow = q0w + 32 * g + col;
      if (qrow < N) {
        char* row = reinterpret_cast<char*>(dq + head) + (size_t)qrow * kRowBytes;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int gg = 0; gg < 4; ++gg) {
            const int i = 4 * gg;
            u32x2 wv = {pack_bf16(acc[g][mb][i] * scale, acc[g][mb][i + 1] * scale),
                        pack_bf16(acc[g][mb][i + 2] * scale, acc[g][mb][i + 3] * scale)};
            *reinterpret_cast<u32x2*>(row + (32 * mb + 8 * gg + 4 * h) * 2) = wv;
          }
      }
    }
  }
}

hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ws, int B, int H,
                          int N, hipStream_t stream) {
  const int rows = B * H * N;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0,
                     stream, static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), lse,
                     ws, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* ws, void* dk, void* dv, int B, int H, int N, float scale,
                           int causal, hipStream_t stream) {
  const int BH = B * H;
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  const int nkb = (N + KV_BK - 1) / KV_BK;
  dim3 grid((unsigned)(nkb * BH)), block(KV_THREADS);
  auto kern = causal ? bwd_dkdv_kernel<true> : bwd_dkdv_kernel<false>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dO), ws, static_cast<uint16_t*>(dk),
                     static_cast<uint16_t*>(dv), BH, N, sl2, scale, sc.keep, sc.flip);
  return hipGetLastError();
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, float* ws, void* dq, int B, int H, int N,
                         float scale, int causal, hipStream_t stream) {
  const int BH = B * H;
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  const int nqb = (N + DQ_BQ - 1) / DQ_BQ;
  dim3 grid((unsigned)(nqb * BH)), block(DQ_THREADS);
  auto kern = causal ? bwd_dq_kernel<true> : bwd_dq_kernel<false>;
  hipLaunchKernelGGL(kern, grid, block, 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(dO), lse, ws,
                     static_cast<uint16_t*>(dq), BH, N, nqb, sl2, scale, sc.keep, sc.flip);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Allocation-free backward (fa_bwd_noalloc): the [-D | L log2(e)] workspace
// lives in this fixed device array, one copy per GPU, held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in): the device address of each GPU's copy is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept here.  Nothing in it needs clearing: the dQ kernel writes every entry
// the dK/dV kernel then reads.  Calls that overlap on one GPU share
// the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t launch_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, float scale, int causal, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      g_scratch_addr[dev] = p;
    }
    ws = static_cast<float*>(g_scratch_addr[dev]);
  }
  e = launch_bwd_dq(q, k, v, o, dO, lse, ws, dq, B, H, N, scale, causal, stream);
  if (e == hipSuccess) e = launch_bwd_dkdv(q, k, v, dO, ws, dk, dv, B, H, N, scale, causal, stream);
  return e;
}

}  // namespace fa
