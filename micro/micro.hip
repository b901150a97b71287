// Microbenchmarks of the gfx950 rates the attention kernels' design rests on.
//
//   mfma     bf16 32x32x16 MFMA throughput, four independent accumulators
//            per wave, two waves per SIMD, with operands of random bits
//            (a different fragment for every MFMA of the loop) or constant
//            (every fragment 1.0): the chip runs at its power cap, and the
//            switching activity of the operands sets the clock it can hold.
//   valu     cycles per wave64 instruction of v_fma_f32 and v_exp_f32 (16
//            independent chains per wave; core cycles from s_memtime).
//   coexec   an MFMA stream and a VALU stream (exp + fma, as in a softmax):
//            each alone, one of each on every SIMD (two waves), and both in
//            one wave, interleaved.
//   atomic   fp32 global atomic add bandwidth: every lane adds one float,
//            rows of 256 bytes per wave, all to distinct addresses.
//   mix1     one wave per SIMD issuing both streams: per MFMA, 0 to 4
//            fma -> exp2 pairs interleaved (as a backward kernel's
//            softmax rides on its MFMAs), accumulators in AGPRs (the
//            compiler's choice) or in VGPRs (inline assembly, as the
//            kernels keep S and dP); core cycles per MFMA.
//   lds      LDS read bandwidth per CU for ds_read_b128, ds_read_b64 and
//            ds_read_b64_tr_b16 (eight waves per CU, consecutive lanes on
//            consecutive addresses: no bank conflicts); core cycles from
//            s_memtime.
//   copy     HBM bandwidth of a plain 1 GiB device copy (16-byte loads and
//            stores, grid-stride).
//   atomicdq the atomic traffic a dK/dV kernel with fused fp32 dQ would issue
//            at B1 H64 N8192 causal: per head and 256-key block, one
//            32 x 128 fp32 add per 32-query tile at or after the block;
//            the result (a count per dQ element) is checked on the host.
//   order    the same MFMA loop (random operands) for about a second per
//            variant, with the order of the MFMAs changed so that
//            consecutive MFMAs share none, one or both of their operand
//            registers; the board's power (hwmon power1_input) and the
//            graphics clock (pp_dpm_sclk) are sampled every 10 ms meanwhile.
//
// Every kernel writes only through vector stores, every access is to a
// buffer sized on the host for exactly the grid launched, and every loop
// has a fixed trip count.  Prints one JSON line per measurement.
#include <hip/hip_runtime.h>

#include <glob.h>

#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#define CHECK(x)                                                                      \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                                        \
    }                                                                                 \
  } while (0)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kCUs = 256;

// ---------------------------------------------------------------------------
// MFMA throughput.  src holds 8 fragments (16 bytes per lane) per lane of a
// 256-thread block: fragments 0-3 are A operands, 4-7 B operands.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mfma_rate(const u32x4* __restrict__ src, float* __restrict__ out,
                                                 int iters) {
  const int tid = threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[i * 256 + tid]);
    b[i] = __builtin_bit_cast(bf16x8, src[(4 + i) * 256 + tid]);
  }
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[i ^ 1], c[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i ^ 2], b[i ^ 3], c[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  out[blockIdx.x * 256 + tid] = s;
}

// One wave per SIMD (one 256-thread block per CU), four accumulators (in
// VGPRs when VACC); per MFMA, NPAIR fma -> exp2 pairs on independent values
// in between.
template <int NPAIR, int VACC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mix1(const u32x4* __restrict__ src, float* __restrict__ out, long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[i * 256 + tid]);
    b[i] = __builtin_bit_cast(bf16x8, src[(4 + i) * 256 + tid]);
  }
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  float f[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) f[j] = 0.001f * tid + 0.01f * j - 0.5f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (VACC)
        asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+v"(c[i & 3])
                     : "v"(a[i & 3]), "v"(b[(i + 1) & 3]));
      else
        c[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[(i + 1) & 3], c[i & 3], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NPAIR; ++j) {
        const int k = (4 * i + j) & 31;
        f[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[k], 0.5f, -0.25f));
        asm volatile("" : "+v"(f[k]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // the VGPR results are read by VALU only after the last MFMA has drained
  if (VACC) asm volatile("s_nop 15\n\ts_nop 15" : "+v"(c[0]), "+v"(c[1]), "+v"(c[2]), "+v"(c[3]));
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
#pragma unroll
  for (int j = 0; j < 32; ++j) s += f[j];
  out[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) cyc[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

// The same loop with the MFMAs in a fixed order (sched_barrier between them):
//   0  consecutive MFMAs share no operand register
//   1  the A operand is held for two MFMAs, B changes every MFMA
//   2  A held for four MFMAs
//   3  B held for four MFMAs, A changes every MFMA
//   4  A and B both held for four MFMAs (four accumulators)
//   5  as 0, but each accumulator takes two consecutive MFMAs
//   6  as 0, but each accumulator takes four consecutive MFMAs (two in use)
template <int ORDER>
__device__ __forceinline__ void order_ops(int n, int i, int& ai, int& bi) {
  // n: half of the iteration (0, 1); i: MFMA within the half (0..3)
  if (ORDER == 0 || ORDER >= 5) {
    ai = n ? (i ^ 2) : i;
    bi = n ? (i ^ 3) : (i ^ 1);
  } else if (ORDER == 1) {
    ai = 2 * n + (i >> 1);
    bi = i;
  } else if (ORDER == 2) {
    ai = n;
    bi = i;
  } else if (ORDER == 3) {
    ai = i;
    bi = n;
  } else {
    ai = n;
    bi = n;
  }
}
template <int ORDER>
__global__ __launch_bounds__(256) void mfma_order(const u32x4* __restrict__ src, float* __restrict__ out,
                                                  int iters) {
  const int tid = threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[i * 256 + tid]);
    b[i] = __builtin_bit_cast(bf16x8, src[(4 + i) * 256 + tid]);
  }
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int ai, bi;
        order_ops<ORDER>(n, i, ai, bi);
        const int ci = ORDER == 5 ? 2 * n + (i >> 1) : ORDER == 6 ? n : i;
        c[ci] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ai], b[bi], c[ci], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
  out[blockIdx.x * 256 + tid] = s;
}

// ---------------------------------------------------------------------------
// VALU: 16 independent chains of one instruction kind per wave; out gets the
// core cycles the loop took (s_memtime) and a checksum.
// ---------------------------------------------------------------------------
template <int KIND>  // 0: v_fma_f32, 1: v_exp_f32
__global__ __launch_bounds__(256) void valu_rate(float* __restrict__ out, long long* __restrict__ cyc,
                                                 int iters) {
  const int tid = threadIdx.x;
  float f[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) f[j] = 0.001f * tid + 0.01f * j - 0.5f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      if (KIND == 0)
        f[j] = __builtin_fmaf(f[j], 0.999f, 0.0001f);
      else
        f[j] = __builtin_amdgcn_exp2f(f[j]) - 1.0f;  // stays in (-1, 1): exp2 then one add
      asm volatile("" : "+v"(f[j]));
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += f[j];
  out[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) cyc[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

// ---------------------------------------------------------------------------
// One wave per SIMD: the same 16 exp2(fma(x)) pairs per iteration, issued
// either back to back (each exp right after the fma it reads: ORDER 0) or
// software-pipelined (the fma of the next pair between an fma and its exp:
// ORDER 1).  A wave alone on its SIMD has no other wave to fill the cycles a
// dependent instruction waits for its input.
// ---------------------------------------------------------------------------
template <int ORDER>
__global__ __launch_bounds__(256) void valu_dep(float* __restrict__ out, long long* __restrict__ cyc,
                                                int iters) {
  const int tid = threadIdx.x;
  float f[16], x[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) f[j] = 0.001f * tid + 0.01f * j - 0.5f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    if (ORDER == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        x[j] = __builtin_fmaf(f[j], 0.5f, -0.25f);
        asm volatile("" : "+v"(x[j]));
        f[j] = __builtin_amdgcn_exp2f(x[j]);
        asm volatile("" : "+v"(f[j]));
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      x[0] = __builtin_fmaf(f[0], 0.5f, -0.25f);
      asm volatile("" : "+v"(x[0]));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (j + 1 < 16) {
          x[j + 1] = __builtin_fmaf(f[j + 1], 0.5f, -0.25f);
          asm volatile("" : "+v"(x[j + 1]));
        }
        f[j] = __builtin_amdgcn_exp2f(x[j]);
        asm volatile("" : "+v"(f[j]));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += f[j];
  out[blockIdx.x * 256 + tid] = s;
  if ((tid & 63) == 0) cyc[blockIdx.x * 4 + (tid >> 6)] = t1 - t0;
}

// ---------------------------------------------------------------------------
// Co-execution, 512 threads (8 waves) per block, one block per CU: waves w
// and w + 4 share a SIMD.  MODE 0: waves 0-3 run the MFMA stream (4 x 8
// MFMAs per iteration), 4-7 idle; 1: waves 4-7 run the VALU stream (per
// iteration 32 exp2 + 32 fma, a softmax's share per 64-key tile), 0-3 idle;
// 2: both (one of each per SIMD); 3: waves 0-3 run both streams interleaved
// in one instruction stream, 4-7 idle.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(512) void coexec(const u32x4* __restrict__ src, float* __restrict__ out,
                                              long long* __restrict__ cyc, int iters) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const bool mwave = wave < 4;
  const bool do_mfma = mwave && (MODE == 0 || MODE == 2 || MODE == 3);
  const bool do_valu = (MODE == 3) ? mwave : (!mwave && (MODE == 1 || MODE == 2));
  const int t = tid & 255;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, src[i * 256 + t]);
    b[i] = __builtin_bit_cast(bf16x8, src[(4 + i) * 256 + t]);
  }
  f32x16 c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
  float f[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) f[j] = 0.001f * t + 0.01f * j - 0.5f;
  const long long t0 = __builtin_amdgcn_s_memtime();
  if (do_mfma && do_valu) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        c[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[(i + 1) & 3], c[i & 3], 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = 4 * i + j;
          f[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[k], 0.5f, -0.25f));
          asm volatile("" : "+v"(f[k]));
        }
      }
    }
  } else if (do_mfma) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        c[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i & 3], b[(i + 1) & 3], c[i & 3], 0, 0, 0);
    }
  } else if (do_valu) {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        f[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[k], 0.5f, -0.25f));
        asm volatile("" : "+v"(f[k]));
      }
    }
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += c[i][j];
#pragma unroll
  for (int j = 0; j < 32; ++j) s += f[j];
  out[blockIdx.x * 512 + tid] = s;
  if ((tid & 63) == 0) cyc[blockIdx.x * 8 + wave] = (do_mfma || do_valu) ? (t1 - t0) : 0;
}

// ---------------------------------------------------------------------------
// fp32 atomic add bandwidth: thread g adds 1.0 to dst[(g + it * threads) %
// n] for it < iters (n a multiple of the thread count, so every index is in
// bounds and a wave's 64 adds cover one 256-byte row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void atomic_rate(float* __restrict__ dst, int n, int iters) {
  const int threads = gridDim.x * 256;
  const int g = blockIdx.x * 256 + threadIdx.x;
  for (int it = 0; it < iters; ++it) {
    const int idx = (int)(((long long)g + (long long)it * threads) % n);
    __hip_atomic_fetch_add(dst + idx, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
// LDS read bandwidth: 512 threads (eight waves) per block, one block per CU
// (96 KiB of LDS per block: a second block does not fit beside it), a 64 KiB
// LDS array read in a loop, eight reads per iteration, each a wave-wide
// contiguous span; the base offset moves every iteration through a register
// the compiler cannot follow, so no read can be hoisted out of the loop.
// KIND 0: ds_read_b128, 1: ds_read_b64, 2: ds_read_b64_tr_b16, 3: ds_read_b128
// with every lane of a wave at the same address (a broadcast).  cyc gets
// each wave's s_memtime cycles.
constexpr int kLdsWords = 16384;  // 64 KiB of u32
template <int KIND>
__global__ __launch_bounds__(512) void lds_rate(unsigned* __restrict__ out, long long* __restrict__ cyc,
                                                int iters) {
  __shared__ __attribute__((aligned(16))) unsigned buf[kLdsWords];
  __shared__ unsigned pad[kLdsWords / 2];  // only occupies LDS
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsWords; i += 512) buf[i] = (unsigned)i * 2654435761u;
  __syncthreads();
  const char* base = reinterpret_cast<const char*>(buf);
  constexpr int kBytes = (KIND == 0 || KIND == 3) ? 16 : 8;  // per lane and read
  constexpr int kSpan = 64 * kBytes;          // per wave and read
  constexpr int kMask = kLdsWords * 4 - 1;
  unsigned x = 0;
  int b = wave * kSpan + (KIND == 3 ? 0 : lane * kBytes);
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      // wave-wide span u of this iteration, wrapped inside the 64 KiB array
      const int off = (b + u * 8 * kSpan) & kMask;
      if (KIND == 0 || KIND == 3) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(base + off);
        x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      } else if (KIND == 1) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(base + off);
        x ^= v[0] ^ v[1];
      } else {
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + off));
        x ^= (unsigned)(unsigned short)v[0] ^ (unsigned)(unsigned short)v[3];
      }
    }
    b = (b + 3 * kSpan) & kMask;
    asm volatile("" : "+v"(b));
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  pad[tid] = x;
  out[blockIdx.x * 512 + tid] = x ^ pad[tid ^ 1];
  if (lane == 0) cyc[blockIdx.x * 8 + wave] = t1 - t0;
}

// Plain copy, 16 bytes per lane per iteration, grid-stride.
__global__ __launch_bounds__(256) void copy16(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                              long long n) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

// The fused-dQ atomic traffic: block (head, key block kb of 256 keys) adds
// 1.0 to every element of the 32 x 128 dQ rows of each 32-query tile
// qt = 8 kb .. N / 32 - 1 (the tiles at or after the block, causal).
// dq holds heads x n rows x 128 floats.
__global__ __launch_bounds__(256) void atomic_dq(float* __restrict__ dq, int n) {
  const int nkb = n / 256;
  const int head = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  float* hq = dq + (size_t)head * n * 128;
  for (int qt = 8 * kb; qt < n / 32; ++qt) {
    float* tile = hq + (size_t)qt * 32 * 128;
#pragma unroll
    for (int j = 0; j < 16; ++j)
      __hip_atomic_fetch_add(tile + j * 256 + threadIdx.x, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ---------------------------------------------------------------------------
static unsigned lcg(unsigned& s) {
  s = s * 1664525u + 1013904223u;
  return s;
}

// Board power (W) and graphics clock (MHz) of the first AMD GPU, from sysfs;
// negative when not readable.
struct telemetry {
  std::string power_path, sclk_path;
  telemetry() {
    glob_t g;
    if (glob("/sys/class/drm/card*/device/hwmon/hwmon*/power1_input", 0, nullptr, &g) == 0 && g.gl_pathc)
      power_path = g.gl_pathv[0];
    globfree(&g);
    if (glob("/sys/class/drm/card*/device/pp_dpm_sclk", 0, nullptr, &g) == 0 && g.gl_pathc)
      sclk_path = g.gl_pathv[0];
    globfree(&g);
  }
  double power_w() const {
    FILE* f = fopen(power_path.c_str(), "r");
    if (!f) return -1;
    double uw = -1;
    if (fscanf(f, "%lf", &uw) != 1) uw = -1;
    fclose(f);
    return uw < 0 ? -1 : uw / 1e6;
  }
  double sclk_mhz() const {  // the DPM level marked '*'
    FILE* f = fopen(sclk_path.c_str(), "r");
    if (!f) return -1;
    char line[128];
    double mhz = -1;
    while (fgets(line, sizeof line, f)) {
      if (!strchr(line, '*')) continue;
      const char* c = strchr(line, ':');
      if (c) mhz = atof(c + 1);
    }
    fclose(f);
    return mhz;
  }
};

static float time_ms(hipEvent_t e0, hipEvent_t e1) {
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  return ms;
}

int main(int argc, char** argv) {
  const char* only = argc > 1 ? argv[1] : "";
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));

  // Operand fragments: 8 per lane x 256 lanes, 16 bytes each.
  const int nfrag = 8 * 256;
  std::vector<unsigned> rnd(nfrag * 4), one(nfrag * 4, 0x3f803f80u);
  unsigned seed = 12345u;
  for (auto& x : rnd) {
    // random bf16 pairs with exponents in [-8, 7] (finite, no overflow in the sums)
    unsigned lo = (lcg(seed) & 0x807fu) | ((120u + (lcg(seed) % 16u)) << 7);
    unsigned hi = (lcg(seed) & 0x807fu) | ((120u + (lcg(seed) % 16u)) << 7);
    x = lo | (hi << 16);
  }
  u32x4* src;
  CHECK(hipMalloc(&src, nfrag * 16));
  const int blocks = 2 * kCUs * 4;  // 4 blocks of 4 waves per CU, 4 waves per SIMD over the run
  float* out;
  CHECK(hipMalloc(&out, (size_t)blocks * 512 * sizeof(float)));
  long long* cyc;
  CHECK(hipMalloc(&cyc, (size_t)blocks * 8 * sizeof(long long)));
  std::vector<long long> hc((size_t)blocks * 8);

  if (!*only || !strcmp(only, "mfma")) {
    for (int pass = 0; pass < 2; ++pass) {
      for (int rnd_ops = 1; rnd_ops >= 0; --rnd_ops) {
        CHECK(hipMemcpy(src, rnd_ops ? rnd.data() : one.data(), nfrag * 16, hipMemcpyHostToDevice));
        const int iters = 20000;
        const int grid = 2 * kCUs;  // two blocks of four waves per CU: two waves per SIMD
        hipLaunchKernelGGL(mfma_rate, dim3(grid), dim3(256), 0, 0, src, out, 100);
        CHECK(hipDeviceSynchronize());
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(mfma_rate, dim3(grid), dim3(256), 0, 0, src, out, iters);
        CHECK(hipEventRecord(e1));
        CHECK(hipDeviceSynchronize());
        const double ms = time_ms(e0, e1);
        const double flop = (double)grid * 4 * iters * 8 * 32.0 * 32 * 16 * 2;
        if (pass)
          printf("{\"probe\": \"mfma_bf16_32x32x16\", \"operands\": \"%s\", \"ms\": %.3f, \"tflops\": %.1f}\n",
                 rnd_ops ? "random" : "constant", ms, flop / ms / 1e9);
      }
    }
  }
  if (!*only || !strcmp(only, "mix1")) {
    CHECK(hipMemcpy(src, rnd.data(), nfrag * 16, hipMemcpyHostToDevice));
    const int iters = 2000, grid = kCUs;  // one block of four waves per CU: one wave per SIMD
    for (int v = 0; v < 2; ++v)
    for (int np = 0; np <= 4; ++np) {
      for (int w = 0; w < 2; ++w) {
        switch (np + 5 * v) {
          case 0: hipLaunchKernelGGL((mix1<0, 0>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 1: hipLaunchKernelGGL((mix1<1, 0>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 2: hipLaunchKernelGGL((mix1<2, 0>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 3: hipLaunchKernelGGL((mix1<3, 0>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 4: hipLaunchKernelGGL((mix1<4, 0>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 5: hipLaunchKernelGGL((mix1<0, 1>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 6: hipLaunchKernelGGL((mix1<1, 1>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 7: hipLaunchKernelGGL((mix1<2, 1>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          case 8: hipLaunchKernelGGL((mix1<3, 1>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
          default: hipLaunchKernelGGL((mix1<4, 1>), dim3(grid), dim3(256), 0, 0, src, out, cyc, iters); break;
        }
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(hc.data(), cyc, (size_t)grid * 4 * sizeof(long long), hipMemcpyDeviceToHost));
      double avg = 0;
      for (int i = 0; i < grid * 4; ++i) avg += (double)hc[i];
      avg /= grid * 4;
      printf("{\"probe\": \"mix1\", \"accumulators\": \"%s\", \"fma_exp_pairs_per_mfma\": %d, "
             "\"core_cycles_per_mfma\": %.1f}\n", v ? "VGPR" : "AGPR", np, avg / (iters * 8.0));
    }
  }
  if (!*only || !strcmp(only, "order")) {
    CHECK(hipMemcpy(src, rnd.data(), nfrag * 16, hipMemcpyHostToDevice));
    const telemetry tel;
    const char* names[7] = {"no operand shared", "A held for 2", "A held for 4", "B held for 4",
                            "A and B held for 4", "accumulator held for 2", "accumulator held for 4"};
    const int grid = 2 * kCUs, iters = 20000, launches = 160;  // about a second per variant
    for (int order = 0; order < 7; ++order) {
      auto launch = [&](int it) {
        switch (order) {
          case 0: hipLaunchKernelGGL(mfma_order<0>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
          case 1: hipLaunchKernelGGL(mfma_order<1>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
          case 2: hipLaunchKernelGGL(mfma_order<2>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
          case 3: hipLaunchKernelGGL(mfma_order<3>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
          case 4: hipLaunchKernelGGL(mfma_order<4>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
          case 5: hipLaunchKernelGGL(mfma_order<5>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
          default: hipLaunchKernelGGL(mfma_order<6>, dim3(grid), dim3(256), 0, 0, src, out, it); break;
        }
      };
      launch(100);
      CHECK(hipDeviceSynchronize());
      std::this_thread::sleep_for(std::chrono::milliseconds(500));
      std::atomic<bool> stop{false};
      std::vector<double> pw, sc;
      std::thread sampler([&] {
        while (!stop.load()) {
          pw.push_back(tel.power_w());
          sc.push_back(tel.sclk_mhz());
          std::this_thread::sleep_for(std::chrono::milliseconds(10));
        }
      });
      CHECK(hipEventRecord(e0));
      for (int l = 0; l < launches; ++l) launch(iters);
      CHECK(hipEventRecord(e1));
      CHECK(hipDeviceSynchronize());
      stop = true;
      sampler.join();
      const double ms = time_ms(e0, e1);
      const double flop = (double)launches * grid * 4 * iters * 8 * 32.0 * 32 * 16 * 2;
      // mean over the second half of the samples (past the clock's settling)
      double p = 0, c = 0;
      size_t n0 = pw.size() / 2, n = 0;
      for (size_t i = n0; i < pw.size(); ++i, ++n) {
        p += pw[i];
        c += sc[i];
      }
      printf("{\"probe\": \"mfma_order\", \"order\": \"%s\", \"ms\": %.1f, \"tflops\": %.1f, "
             "\"power_w\": %.1f, \"sclk_mhz\": %.0f, \"samples\": %zu}\n",
             names[order], ms, flop / ms / 1e9, n ? p / n : -1.0, n ? c / n : -1.0, n);
      fflush(stdout);
    }
  }
  if (!*only || !strcmp(only, "valu")) {
    for (int kind = 0; kind < 2; ++kind) {
      const int iters = 4000;
      const int grid = 2 * kCUs;
      for (int w = 0; w < 2; ++w) {
        if (kind == 0)
          hipLaunchKernelGGL(valu_rate<0>, dim3(grid), dim3(256), 0, 0, out, cyc, iters);
        else
          hipLaunchKernelGGL(valu_rate<1>, dim3(grid), dim3(256), 0, 0, out, cyc, iters);
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(hc.data(), cyc, (size_t)grid * 4 * sizeof(long long), hipMemcpyDeviceToHost));
      double avg = 0;
      for (int i = 0; i < grid * 4; ++i) avg += (double)hc[i];
      avg /= grid * 4;
      // two waves per SIMD share its issue: cycles per instruction of one wave / 2 = SIMD cost
      printf("{\"probe\": \"valu\", \"instruction\": \"%s\", \"waves_per_simd\": 2, "
             "\"core_cycles_per_wave_instruction\": %.2f, \"simd_cycles_per_instruction\": %.2f}\n",
             kind == 0 ? "v_fma_f32" : "v_exp_f32 + v_add_f32", avg / (iters * 16.0), avg / (iters * 16.0) / 2);
    }
  }
  if (!*only || !strcmp(only, "valu1")) {
    for (int order = 0; order < 2; ++order) {
      const int iters = 4000;
      const int grid = kCUs;  // one block of four waves per CU: one wave per SIMD
      for (int w = 0; w < 2; ++w) {
        if (order == 0)
          hipLaunchKernelGGL(valu_dep<0>, dim3(grid), dim3(256), 0, 0, out, cyc, iters);
        else
          hipLaunchKernelGGL(valu_dep<1>, dim3(grid), dim3(256), 0, 0, out, cyc, iters);
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(hc.data(), cyc, (size_t)grid * 4 * sizeof(long long), hipMemcpyDeviceToHost));
      double avg = 0;
      for (int i = 0; i < grid * 4; ++i) avg += (double)hc[i];
      avg /= grid * 4;
      printf("{\"probe\": \"valu_one_wave_per_simd\", \"order\": \"%s\", \"core_cycles_per_fma_exp_pair\": %.2f}\n",
             order == 0 ? "exp right after its fma" : "next fma between fma and exp", avg / (iters * 16.0));
    }
  }
  if (!*only || !strcmp(only, "coexec")) {
    CHECK(hipMemcpy(src, rnd.data(), nfrag * 16, hipMemcpyHostToDevice));
    const char* names[4] = {"mfma stream alone", "valu stream alone", "one mfma wave + one valu wave per simd",
                            "both streams in one wave"};
    const int iters = 2000;
    const int grid = kCUs;
    for (int mode = 0; mode < 4; ++mode) {
      for (int w = 0; w < 2; ++w) {
        switch (mode) {
          case 0: hipLaunchKernelGGL(coexec<0>, dim3(grid), dim3(512), 0, 0, src, out, cyc, iters); break;
          case 1: hipLaunchKernelGGL(coexec<1>, dim3(grid), dim3(512), 0, 0, src, out, cyc, iters); break;
          case 2: hipLaunchKernelGGL(coexec<2>, dim3(grid), dim3(512), 0, 0, src, out, cyc, iters); break;
          default: hipLaunchKernelGGL(coexec<3>, dim3(grid), dim3(512), 0, 0, src, out, cyc, iters); break;
        }
        CHECK(hipDeviceSynchronize());  // the first launch warms up; the second's cycles are kept
      }
      CHECK(hipMemcpy(hc.data(), cyc, (size_t)grid * 8 * sizeof(long long), hipMemcpyDeviceToHost));
      // waves 0-3 of each block vs waves 4-7 (the MFMA and VALU waves in mode 2)
      double sum[2] = {0, 0};
      int cnt[2] = {0, 0};
      for (int i = 0; i < grid * 8; ++i)
        if (hc[i] > 0) {
          const int grp = (i % 8) >= 4;
          sum[grp] += (double)hc[i];
          ++cnt[grp];
        }
      printf("{\"probe\": \"coexec\", \"mode\": \"%s\", \"core_cycles_per_iteration_waves_0_3\": %.1f, "
             "\"core_cycles_per_iteration_waves_4_7\": %.1f, \"mfma_cycles_per_iteration\": %d, "
             "\"valu_per_iteration\": \"32 exp2 + 32 fma\"}\n",
             names[mode], cnt[0] ? sum[0] / cnt[0] / iters : 0.0, cnt[1] ? sum[1] / cnt[1] / iters : 0.0, 8 * 32);
    }
  }
  if (!*only || !strcmp(only, "atomic")) {
    const int grid = 4 * kCUs;
    const int threads = grid * 256;
    const int n = threads * 16;  // 16 MiB of floats, a multiple of the thread count
    const int iters = 64;
    float* dst;
    CHECK(hipMalloc(&dst, (size_t)n * sizeof(float)));
    CHECK(hipMemset(dst, 0, (size_t)n * sizeof(float)));
    hipLaunchKernelGGL(atomic_rate, dim3(grid), dim3(256), 0, 0, dst, n, 4);
    CHECK(hipDeviceSynchronize());
    CHECK(hipEventRecord(e0));
    hipLaunchKernelGGL(atomic_rate, dim3(grid), dim3(256), 0, 0, dst, n, iters);
    CHECK(hipEventRecord(e1));
    CHECK(hipDeviceSynchronize());
    const double ms = time_ms(e0, e1);
    const double bytes = (double)threads * iters * 4;
    printf("{\"probe\": \"atomic_add_f32\", \"ms\": %.3f, \"gbps\": %.1f}\n", ms, bytes / ms / 1e6);
    CHECK(hipFree(dst));
  }
  if (!*only || !strcmp(only, "lds")) {
    const int grid = kCUs, iters = 4096;
    unsigned* lout;
    long long* lcyc;
    CHECK(hipMalloc(&lout, (size_t)grid * 512 * sizeof(unsigned)));
    CHECK(hipMalloc(&lcyc, (size_t)grid * 8 * sizeof(long long)));
    std::vector<long long> hl((size_t)grid * 8);
    const char* names[3] = {"ds_read_b128", "ds_read_b64", "ds_read_b64_tr_b16"};
    const int bytes[3] = {16, 8, 8};
    for (int kind = 0; kind < 3; ++kind) {
      for (int w = 0; w < 2; ++w) {
        if (kind == 0)
          hipLaunchKernelGGL(lds_rate<0>, dim3(grid), dim3(512), 0, 0, lout, lcyc, iters);
        else if (kind == 1)
          hipLaunchKernelGGL(lds_rate<1>, dim3(grid), dim3(512), 0, 0, lout, lcyc, iters);
        else
          hipLaunchKernelGGL(lds_rate<2>, dim3(grid), dim3(512), 0, 0, lout, lcyc, iters);
        CHECK(hipDeviceSynchronize());
      }
      CHECK(hipMemcpy(hl.data(), lcyc, hl.size() * sizeof(long long), hipMemcpyDeviceToHost));
      double avg = 0;
      for (long long c : hl) avg += (double)c;
      avg /= (double)hl.size();
      const double per_cu = 8.0 * iters * 8 * 64 * bytes[kind];  // eight waves per CU
      printf("{\"probe\": \"lds_read\", \"instruction\": \"%s\", \"bytes_per_core_cycle_per_cu\": %.1f}\n",
             names[kind], per_cu / avg);
    }
    CHECK(hipFree(lout));
    CHECK(hipFree(lcyc));
  }
  if (!*only || !strcmp(only, "copy")) {
    const long long n = (1LL << 30) / 16;  // 1 GiB
    u32x4 *a, *b;
    CHECK(hipMalloc(&a, n * 16));
    CHECK(hipMalloc(&b, n * 16));
    CHECK(hipMemset(a, 1, n * 16));
    const int grid = 8 * kCUs;
    hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, 0, a, b, n);
    CHECK(hipDeviceSynchronize());
    const int reps = 10;
    CHECK(hipEventRecord(e0));
    for (int r = 0; r < reps; ++r) hipLaunchKernelGGL(copy16, dim3(grid), dim3(256), 0, 0, a, b, n);
    CHECK(hipEventRecord(e1));
    CHECK(hipDeviceSynchronize());
    const double ms = time_ms(e0, e1) / reps;
    printf("{\"probe\": \"hbm_copy\", \"bytes_copied\": %lld, \"ms\": %.3f, \"gbps_read_plus_write\": %.0f}\n",
           n * 16, ms, 2.0 * n * 16 / ms / 1e6);
    CHECK(hipFree(a));
    CHECK(hipFree(b));
  }
  if (!*only || !strcmp(only, "atomicdq")) {
    const int heads = 64, n = 8192;
    const size_t elems = (size_t)heads * n * 128;  // 256 MiB of fp32
    float* dq;
    CHECK(hipMalloc(&dq, elems * sizeof(float)));
    const int grid = heads * (n / 256);
    double ms = 0;
    for (int r = 0; r < 2; ++r) {  // the second, timed launch starts from zero too
      CHECK(hipMemset(dq, 0, elems * sizeof(float)));
      CHECK(hipDeviceSynchronize());
      CHECK(hipEventRecord(e0));
      hipLaunchKernelGGL(atomic_dq, dim3(grid), dim3(256), 0, 0, dq, n);
      CHECK(hipEventRecord(e1));
      CHECK(hipDeviceSynchronize());
      ms = time_ms(e0, e1);
    }
    // Every element of query row q was added once per key block kb <= q / 256.
    std::vector<float> row(128);
    bool ok = true;
    for (int q : {0, 255, 256, 4095, 8191}) {
      for (int hh : {0, 63}) {
        CHECK(hipMemcpy(row.data(), dq + ((size_t)hh * n + q) * 128, 128 * sizeof(float), hipMemcpyDeviceToHost));
        for (float v : row) ok = ok && v == (float)(q / 256 + 1);
      }
    }
    double adds = 0;
    for (int kb = 0; kb < n / 256; ++kb) adds += (double)(n / 32 - 8 * kb) * 32 * 128;
    adds *= heads;
    printf("{\"probe\": \"atomic_dq_b1_h64_n8192_causal\", \"atomic_bytes\": %.0f, \"ms\": %.3f, "
           "\"gbps\": %.0f, \"result_checked\": %s}\n", adds * 4, ms, adds * 4 / ms / 1e6, ok ? "true" : "false");
    CHECK(hipFree(dq));
  }
  if (!*only || !strcmp(only, "power")) {
    // Board power and clock while one instruction kind runs alone on every
    // CU for about a second: wave instructions per second, and the power
    // above the idle reading divided by that rate (energy per wave
    // instruction at the clock the board settles at).
    CHECK(hipMemcpy(src, rnd.data(), nfrag * 16, hipMemcpyHostToDevice));
    const telemetry tel;
    unsigned* lout;
    long long* lcyc;
    CHECK(hipMalloc(&lout, (size_t)kCUs * 512 * sizeof(unsigned)));
    CHECK(hipMalloc(&lcyc, (size_t)kCUs * 8 * sizeof(long long)));
    CHECK(hipDeviceSynchronize());
    std::this_thread::sleep_for(std::chrono::milliseconds(1000));
    double idle = 0;
    for (int i = 0; i < 20; ++i) {
      idle += tel.power_w();
      std::this_thread::sleep_for(std::chrono::milliseconds(10));
    }
    idle /= 20;
    const char* names[8] = {"v_fma_f32", "v_exp_f32 + v_add_f32", "ds_read_b128 (+4 v_xor_b32 per read)",
                            "v_mfma_f32_32x32x16_bf16 random operands", "v_mfma_f32_32x32x16_bf16 constant operands",
                            "ds_read_b64 (+2 v_xor_b32 per read)", "ds_read_b64_tr_b16 (+1 v_xor_b32 per read)",
                            "ds_read_b128 broadcast, one address per wave (+4 v_xor_b32 per read)"};
    for (int kind = 0; kind < 8; ++kind) {
      const int vgrid = 2 * kCUs, viters = 20000, liters = 4096, miters = 20000;
      double per_launch = 0;  // wave instructions of the measured kind per launch
      auto launch = [&]() {
        switch (kind) {
          case 0: hipLaunchKernelGGL(valu_rate<0>, dim3(vgrid), dim3(256), 0, 0, out, cyc, viters);
                  per_launch = (double)vgrid * 4 * viters * 16; break;
          case 1: hipLaunchKernelGGL(valu_rate<1>, dim3(vgrid), dim3(256), 0, 0, out, cyc, viters);
                  per_launch = (double)vgrid * 4 * viters * 16; break;
          case 2: hipLaunchKernelGGL(lds_rate<0>, dim3(kCUs), dim3(512), 0, 0, lout, lcyc, liters);
                  per_launch = (double)kCUs * 8 * liters * 8; break;
          case 5: hipLaunchKernelGGL(lds_rate<1>, dim3(kCUs), dim3(512), 0, 0, lout, lcyc, liters);
                  per_launch = (double)kCUs * 8 * liters * 8; break;
          case 6: hipLaunchKernelGGL(lds_rate<2>, dim3(kCUs), dim3(512), 0, 0, lout, lcyc, liters);
                  per_launch = (double)kCUs * 8 * liters * 8; break;
          case 7: hipLaunchKernelGGL(lds_rate<3>, dim3(kCUs), dim3(512), 0, 0, lout, lcyc, liters);
                  per_launch = (double)kCUs * 8 * liters * 8; break;
          default: hipLaunchKernelGGL(mfma_order<0>, dim3(vgrid), dim3(256), 0, 0, src, out, miters);
                  per_launch = (double)vgrid * 4 * miters * 8; break;
        }
      };
      if (kind == 3) CHECK(hipMemcpy(src, rnd.data(), nfrag * 16, hipMemcpyHostToDevice));
      if (kind == 4) CHECK(hipMemcpy(src, one.data(), nfrag * 16, hipMemcpyHostToDevice));
      CHECK(hipEventRecord(e0));
      launch();
      CHECK(hipEventRecord(e1));
      CHECK(hipDeviceSynchronize());
      const int launches = std::max(1, (int)(1000.0 / std::max(time_ms(e0, e1), 0.01f)));
      std::this_thread::sleep_for(std::chrono::milliseconds(500));
      std::atomic<bool> stop{false};
      std::vector<double> pw, sc;
      std::thread sampler([&] {
        while (!stop.load()) {
          pw.push_back(tel.power_w());
          sc.push_back(tel.sclk_mhz());
          std::this_thread::sleep_for(std::chrono::milliseconds(10));
        }
      });
      CHECK(hipEventRecord(e0));
      for (int l = 0; l < launches; ++l) launch();
      CHECK(hipEventRecord(e1));
      CHECK(hipDeviceSynchronize());
      stop = true;
      sampler.join();
      const double ms = time_ms(e0, e1);
      double p = 0, c = 0;
      size_t n0 = pw.size() / 2, n = 0;
      for (size_t i = n0; i < pw.size(); ++i, ++n) {
        p += pw[i];
        c += sc[i];
      }
      p = n ? p / n : -1;
      c = n ? c / n : -1;
      const double rate = per_launch * launches / (ms * 1e-3);  // wave instructions per second
      printf("{\"probe\": \"power\", \"instruction\": \"%s\", \"ms\": %.1f, \"giga_wave_instructions_per_s\": %.2f, "
             "\"power_w\": %.1f, \"idle_w\": %.1f, \"sclk_mhz\": %.0f, \"nj_per_wave_instruction_above_idle\": %.3f, "
             "\"samples\": %zu}\n",
             names[kind], ms, rate / 1e9, p, idle, c, (p - idle) / rate * 1e9, n);
      fflush(stdout);
    }
    CHECK(hipFree(lout));
    CHECK(hipFree(lcyc));
  }
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  return 0;
}
