// Fused backward with atomic dQ: the variant that trades the dQ kernel's two
// recomputed products (S and dP) for atomic traffic ("LLM flash attention",
// section "End-to-end flow": dQ accumulated across key blocks; "Interrogating
// the GPU, part 5: FlashAttention", section "What does the backward pass do
// without P?" for the gradients).
//
// A workgroup owns 128 keys of one (batch, head), 32 per wave, and walks the
// 32-query tiles at or after its keys.  Per tile and wave, as in the dK/dV
// kernel: S = Q K^T and dP = dO V^T (keys in lanes), P = exp2(S scale log2 e -
// L log2 e), dS = P (dP - D), dV^T += dO^T P and dK^T += Q^T dS.  In
// addition: dQ^T += K^T dS^T for the wave's 32 keys (dS staged through LDS in
// query-major order, K^T read transposed from the LDS K block), the four
// waves' partials stored to LDS and summed, and the sum added to an fp32 dQ
// buffer with one global atomic per element and tile.  A second kernel turns
// that buffer into bf16 dQ (times the signed scale).  The backward pre-pass
// (bwd_pre_kernel) supplies -D and L log2 e.
//
// The dQ summation order across key blocks is whatever order the atomics land
// in, so dQ is not bitwise reproducible run to run (dK and dV are).
#include "fa_device.hpp"
#include "fa_internal.h"

namespace fa {

constexpr int AT_WAVES = 4;
constexpr int AT_KW = 32;                 // keys per wave
constexpr int AT_BK = AT_WAVES * AT_KW;   // keys per workgroup
constexpr int AT_BQ = 32;                 // queries per tile
constexpr int AT_THREADS = AT_WAVES * 64;
constexpr int AT_KBLK = AT_BK * kRowBytes;  // 32 KiB (K or V block)
constexpr int AT_TILE = AT_BQ * kRowBytes;  // 8 KiB (Q or dO tile)
// LDS: K block, V block, Q tile, dO tile (swizzled rows), L log2 e and -D of
// the tile, each wave's dS (query-major, 32 x 32 bf16 in 72-byte rows), and
// each wave's dQ partial of the tile (fp32, dim-major in rows of 33: the
// stores of one instruction (32 queries, one dim) and the read-out (one
// query, 64 dims) both fall in distinct banks).  The four partials are
// summed at the read-out: LDS atomics from four waves onto the same
// addresses serialise (about 40 ms for this kernel at B1 H64 N8192).
constexpr int AT_K_OFF = 0;
constexpr int AT_V_OFF = AT_K_OFF + AT_KBLK;
constexpr int AT_Q_OFF = AT_V_OFF + AT_KBLK;
constexpr int AT_DO_OFF = AT_Q_OFF + AT_TILE;
constexpr int AT_L_OFF = AT_DO_OFF + AT_TILE;
constexpr int AT_D_OFF = AT_L_OFF + AT_BQ * 4;
constexpr int AT_DS_OFF = AT_D_OFF + AT_BQ * 4;
constexpr int AT_DS_ROW = AT_KW * 2 + 8;  // 72 bytes: the 8-byte reads of 32 rows hit distinct banks
constexpr int AT_DS_WAVE = AT_BQ * AT_DS_ROW;
constexpr int AT_DQ_LD = AT_BQ + 1;       // dQ partial row stride (floats)
constexpr int AT_DQ_OFF = AT_DS_OFF + AT_WAVES * AT_DS_WAVE;
constexpr int AT_DQ_WAVE = kD * AT_DQ_LD * 4;
constexpr int AT_SMEM = AT_DQ_OFF + AT_WAVES * AT_DQ_WAVE;
static_assert(AT_SMEM <= 160 * 1024, "fits one CU's LDS");

template <bool CAUSAL>
__global__ __launch_bounds__(AT_THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_atomic_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                       const uint16_t* __restrict__ v, const uint16_t* __restrict__ dO,
                       const float* __restrict__ ws, float* __restrict__ dqacc,
                       uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int BH, int N,
                       float sl2, float scale, uint32_t kkeep, uint32_t kflip) {
  __shared__ __attribute__((aligned(16))) char smem[AT_SMEM];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int col = lane & 31;

  const int nkb = (N + AT_BK - 1) / AT_BK;
  int kb, bh;
  block_head(blockIdx.x, nkb, BH, false, CAUSAL, &kb, &bh);
  const int k0 = kb * AT_BK;
  const int kw = k0 + AT_KW * wave;

  const size_t head = (size_t)bh * (size_t)N * kD;
  const uint32_t head_bytes = (uint32_t)N * kRowBytes;
  const rsrc_t rq = make_rsrc(q + head, head_bytes);
  const rsrc_t rk = make_rsrc(k + head, head_bytes);
  const rsrc_t rv = make_rsrc(v + head, head_bytes);
  const rsrc_t rdo = make_rsrc(dO + head, head_bytes);
  const size_t rows = (size_t)BH * N;
  const rsrc_t rD = make_rsrc(ws + (size_t)bh * N, (uint32_t)N * 4);
  const rsrc_t rL = make_rsrc(ws + rows + (size_t)bh * N, (uint32_t)N * 4);

  // The workgroup's K and V rows into LDS (rows past N read as zero).
  for (int j = tid; j < AT_BK * 16; j += AT_THREADS) {
    const int r = j >> 4, c = j & 15;
    const uint32_t goff = (uint32_t)(k0 + r) * kRowBytes + c * 16;
    lds_write16(smem + AT_K_OFF, tile_off(r, c), buf_load16(rk, goff));
    lds_write16(smem + AT_V_OFF, tile_off(r, c), buf_load16(rv, goff));
  }
  const float* dqr = reinterpret_cast<const float*>(smem + AT_DQ_OFF);
  float* dqw = reinterpret_cast<float*>(smem + AT_DQ_OFF + wave * AT_DQ_WAVE);

  // Transpose-read lane offsets, as in the dK/dV kernel: row 4 h + (lane % 16)
  // / 4 (+ 8 e), dims 32 mb + 16 ((lane / 16) % 2) + 4 (lane % 4).
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

  f32x16 dva[4], dka[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dva[mb][i] = 0.f;
      dka[mb][i] = 0.f;
    }

  const float* lt = reinterpret_cast<const float*>(smem + AT_L_OFF);
  const float* dt = reinterpret_cast<const float*>(smem + AT_D_OFF);
  char* dss = smem + AT_DS_OFF + wave * AT_DS_WAVE;
  const int krow = AT_KW * wave + col;  // this lane's key, as a row of the K / V block
  const int key = kw + col;
  const int t0 = CAUSAL ? (k0 / AT_BQ) : 0;
  const int ntiles = (N + AT_BQ - 1) / AT_BQ;

  for (int t = t0; t < ntiles; ++t) {
    const int qs = t * AT_BQ;
    __syncthreads();  // the previous tile's LDS reads are done
    for (int j = tid; j < AT_BQ * 16; j += AT_THREADS) {
      const int r = j >> 4, c = j & 15;
      const uint32_t goff = (uint32_t)(qs + r) * kRowBytes + c * 16;
      lds_write16(smem + AT_Q_OFF, tile_off(r, c), buf_load16(rq, goff));
      lds_write16(smem + AT_DO_OFF, tile_off(r, c), buf_load16(rdo, goff));
    }
    if (tid < AT_BQ) {
      reinterpret_cast<float*>(smem + AT_L_OFF)[tid] = buf_load_f32(rL, (uint32_t)(qs + tid) * 4);
      reinterpret_cast<float*>(smem + AT_D_OFF)[tid] = buf_load_f32(rD, (uint32_t)(qs + tid) * 4);
    }
    __syncthreads();

    // S = Q K^T and dP = dO V^T for the wave's 32 keys: lane = key, element i
    // = query 8 (i / 4) + 4 h + i % 4 of the tile.
    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = 0.f;
      dp[i] = 0.f;
    }
#pragma unroll
    for (int kc = 0; kc < 8; ++kc) {
      const bf16x8 kf = __builtin_bit_cast(
          bf16x8, signed_operand(lds_read16(smem + AT_K_OFF, tile_off(krow, 2 * kc + h)), kkeep, kflip));
      const bf16x8 vf = __builtin_bit_cast(bf16x8, lds_read16(smem + AT_V_OFF, tile_off(krow, 2 * kc + h)));
      const bf16x8 qa = __builtin_bit_cast(bf16x8, lds_read16(smem + AT_Q_OFF, tile_off(col, 2 * kc + h)));
      const bf16x8 da = __builtin_bit_cast(bf16x8, lds_read16(smem + AT_DO_OFF, tile_off(col, 2 * kc + h)));
      s = mfma32(qa, kf, s);
      dp = mfma32(da, vf, dp);
    }
    // P and dS = P (dP - D); masked (future, or past N) pairs give zero.
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lt + 8 * gg + 4 * h);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(dt + 8 * gg + 4 * h);  // -D
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * gg + r;
        const int qrow = qs + 8 * gg + 4 * h + r;
        const bool dead = key >= N || qrow >= N || (CAUSAL && key > qrow);
        const float p = dead ? 0.f : fast_exp2(__builtin_fmaf(s[i], sl2, -l4[r]));
        s[i] = p;
        dp[i] = p * (dp[i] + d4[r]);
      }
    }
    // Packed for the products: half u holds queries 16 u + {4 h, 8 + 4 h} + 0..3.
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = 8 * u;
      pb[u] = pack8(s[e], s[e + 1], s[e + 2], s[e + 3], s[e + 4], s[e + 5], s[e + 6], s[e + 7]);
      sb[u] = pack8(dp[e], dp[e + 1], dp[e + 2], dp[e + 3], dp[e + 4], dp[e + 5], dp[e + 6], dp[e + 7]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS (transposed tile reads).
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int u = n >> 2, mb = n & 3;
      const int ro2 = 16 * u * kRowBytes;
      const bf16x8 ado = join(lds_read_tr(smem + AT_DO_OFF + ro2 + troff[mb][0]),
                              lds_read_tr(smem + AT_DO_OFF + ro2 + troff[mb][1]));
      const bf16x8 aq = join(lds_read_tr(smem + AT_Q_OFF + ro2 + troff[mb][0]),
                             lds_read_tr(smem + AT_Q_OFF + ro2 + troff[mb][1]));
      dva[mb] = mfma32(ado, pb[u], dva[mb]);
      dka[mb] = mfma32(aq, sb[u], dka[mb]);
    }
    // dS of the wave, query-major: dss[query][key] (64-byte rows).
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const u32x4 w = __builtin_bit_cast(u32x4, sb[u]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i0 = 8 * u + 2 * j;  // elements i0, i0 + 1: queries of consecutive i
        const int q0 = 8 * (i0 >> 2) + 4 * h + (i0 & 3);
        *reinterpret_cast<uint16_t*>(dss + q0 * AT_DS_ROW + col * 2) = (uint16_t)(w[j] & 0xffffu);
        *reinterpret_cast<uint16_t*>(dss + (q0 + 1) * AT_DS_ROW + col * 2) = (uint16_t)(w[j] >> 16);
      }
    }
    asm volatile("" : : : "memory");  // the reads below come after these writes
    // dQ^T += K^T dS^T over the wave's keys: lane = query (B operand: the
    // lane's row of dss, keys in the order the transpose reads give K^T).
    f32x16 dqa[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqa[mb][i] = 0.f;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* rowp = dss + col * AT_DS_ROW;
      const i16x4 lo = *reinterpret_cast<const i16x4*>(rowp + (16 * u + 4 * h) * 2);
      const i16x4 hi = *reinterpret_cast<const i16x4*>(rowp + (16 * u + 8 + 4 * h) * 2);
      const bf16x8 bds = join(lo, hi);
      const char* kt = smem + AT_K_OFF + (AT_KW * wave + 16 * u) * kRowBytes;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const bf16x8 ak = join(lds_read_tr(kt + troff[mb][0]), lds_read_tr(kt + troff[mb][1]));
        dqa[mb] = mfma32(ak, bds, dqa[mb]);
      }
    }
    // The wave's partial of the tile: element i of block mb is dim
    // 32 mb + 8 (i / 4) + 4 h + i % 4 of query col.
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int i = 0; i < 16; ++i) dqw[(32 * mb + 8 * (i >> 2) + 4 * h + (i & 3)) * AT_DQ_LD + col] = dqa[mb][i];
    __syncthreads();
    // The four partials summed (in wave order), then one global atomic per
    // element of the tile.
    for (int j = tid; j < AT_BQ * kD; j += AT_THREADS) {
      const int qq = j >> 7, dim = j & (kD - 1);
      const int cell = dim * AT_DQ_LD + qq;
      float val = dqr[cell];
#pragma unroll
      for (int w = 1; w < AT_WAVES; ++w) val += dqr[w * (AT_DQ_WAVE / 4) + cell];
      if (qs + qq < N)
        __hip_atomic_fetch_add(dqacc + ((size_t)bh * N + qs + qq) * kD + dim, val, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  if (key < N) {
    char* dkrow = reinterpret_cast<char*>(dk + head) + (size_t)key * kRowBytes;
    char* dvrow = reinterpret_cast<char*>(dv + head) + (size_t)key * kRowBytes;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int i = 4 * gg;
        const int off = (32 * mb + 8 * gg + 4 * h) * 2;
        u32x2 wk = {pack_bf16(dka[mb][i] * scale, dka[mb][i + 1] * scale),
                    pack_bf16(dka[mb][i + 2] * scale, dka[mb][i + 3] * scale)};
        u32x2 wv = {pack_bf16(dva[mb][i], dva[mb][i + 1]), pack_bf16(dva[mb][i + 2], dva[mb][i + 3])};
        *reinterpret_cast<u32x2*>(dkrow + off) = wk;
        *reinterpret_cast<u32x2*>(dvrow + off) = wv;
      }
  }
}

// dQ buffer: cleared before the fused kernel, converted after it.
__global__ __launch_bounds__(256) void dq_clear_kernel(f32x4* __restrict__ acc, size_t n4) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n4; j += (size_t)gridDim.x * 256) acc[j] = z;
}
__global__ __launch_bounds__(256) void dq_convert_kernel(const f32x4* __restrict__ acc,
                                                        u32x4* __restrict__ dq, size_t n8, float scale) {
  for (size_t j = (size_t)blockIdx.x * 256 + threadIdx.x; j < n8; j += (size_t)gridDim.x * 256) {
    const f32x4 a = acc[2 * j], b = acc[2 * j + 1];
    dq[j] = u32x4{pack_bf16(a[0] * scale, a[1] * scale), pack_bf16(a[2] * scale, a[3] * scale),
                  pack_bf16(b[0] * scale, b[1] * scale), pack_bf16(b[2] * scale, b[3] * scale)};
  }
}

size_t bwd_atomic_dq_offset(int B, int H, int N) {
  const size_t head = 2 * (size_t)B * H * N * sizeof(float);
  return (head + 255) & ~(size_t)255;
}

hipError_t launch_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                             const void* dO, const float* lse, void* ws, void* dq, void* dk,
                             void* dv, int B, int H, int N, float scale, int causal,
                             hipStream_t stream) {
  const int BH = B * H;
  float* wsf = static_cast<float*>(ws);
  float* acc = reinterpret_cast<float*>(static_cast<char*>(ws) + bwd_atomic_dq_offset(B, H, N));
  hipError_t e = launch_bwd_pre(o, dO, lse, wsf, B, H, N, stream);
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)BH * N * kD / 4;
  const size_t cblocks = (n4 + 255) / 256;
  const unsigned cgrid = (unsigned)(cblocks < 8192 ? cblocks : 8192);
  hipLaunchKernelGGL(dq_clear_kernel, dim3(cgrid), dim3(256), 0, stream, reinterpret_cast<f32x4*>(acc), n4);
  const signed_scale sc = split_scale(scale, kSignBitsBf16);
  const float sl2 = sc.mag * kLog2e;
  const int nkb = (N + AT_BK - 1) / AT_BK;
  auto kern = causal ? bwd_atomic_kernel<true> : bwd_atomic_kernel<false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)(nkb * BH)), dim3(AT_THREADS), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), wsf, acc,
                     static_cast<uint16_t*>(dk), static_cast<uint16_t*>(dv), BH, N, sl2, scale,
                     sc.keep, sc.flip);
  const size_t n8 = n4 / 2;
  hipLaunchKernelGGL(dq_convert_kernel, dim3(cgrid), dim3(256), 0, stream,
                     reinterpret_cast<const f32x4*>(acc), static_cast<u32x4*>(dq), n8, scale);
  return hipGetLastError();
}

}  // namespace fa
