// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, bf16 MFMA wrappers, LDS tile addressing with an XOR swizzle,
// the LDS transpose read, and cross-half-wave reductions.
//
// MFMA operand layouts (v_mfma_f32_32x32x16_bf16, wave64; lane l, h = l / 32):
//   A (32 x 16, row m, col k): lane l holds A[l % 32][8h .. 8h + 7]
//   B (16 x 32, row k, col n): lane l holds B[8h .. 8h + 7][l % 32]
//   C (32 x 32): lane l holds element i (0..15) at
//                row 8 (i / 4) + 4h + (i % 4), column l % 32
// so a C tile read per lane is "column l % 32, a fixed set of 16 rows".  The
// kernels compute transposed products (S^T = K Q^T, O^T = V^T P^T, ...) so
// that each lane owns one query (or key) column and the softmax statistics of
// a row stay inside one lane pair (l, l ^ 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kD = 128;            // head dimension handled by every kernel
constexpr int kRowBytes = kD * 2;  // one bf16 row of Q/K/V in bytes (256)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Physical 16-byte chunk of logical chunk c (0..15) in tile row r.  The map
// is c ^ f(r) with f swapping the two 2-bit halves of r & 15, so
//   * 16 consecutive rows reading one logical chunk hit 16 distinct chunks
//     (row-wise MFMA operand reads, ds_read_b128), and
//   * 4 consecutive rows (aligned to 4) reading 4 adjacent logical chunks
//     (aligned to 4) hit 16 distinct chunks: the 32 lanes of a transpose read
//     (ds_read_b64_tr_b16) cover all 64 banks.
__device__ __forceinline__ int swz(int r) {
  return ((r & 3) << 2) | ((r >> 2) & 3);
}
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz(row)) << 4);
}
// Byte offset of the 8-byte half `half` (0/1) of logical chunk `chunk`.
__device__ __forceinline__ int tile_off8(int row, int chunk, int half) {
  return tile_off(row, chunk) + (half << 3);
}

__device__ __forceinline__ u32x4 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const u32x4*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, source lane s supplies the address of 4 consecutive bf16; output
// lane i receives element (i % 4) of the rows supplied by source lanes
// (i / 4) + 4 j for j = 0..3.  With source lane s pointing at
// T[r0 + s / 4][c0 + 4 (s % 4)], output lane i gets T[r0 + j][c0 + i], j=0..3.
__device__ __forceinline__ i16x4 lds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join(i16x4 lo, i16x4 hi) {
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Value of x held by lane l ^ 32 combined with this lane's: max / sum over
// the two half-waves (v_permlane32_swap).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float pair -> packed bf16 pair (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// A register-held operand under a signed softmax scale: every element's bits
// ANDed with `keep` and XORed with `flip` (negated for a negative scale,
// cleared for scale 0; the host side derives the two words).
__device__ __forceinline__ u32x4 signed_operand(u32x4 u, uint32_t keep, uint32_t flip) {
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = (u[i] & keep) ^ flip;
  return u;
}

// acc + the two bf16 values packed in `pair`, in fp32 (one v_dot2c_f32_bf16
// against (1, 1): the products are exact).
__device__ __forceinline__ float add_bf16_pair(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}

__device__ __forceinline__ bf16x8 pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                        float a6, float a7) {
  u32x4 u = {pack_bf16(a0, a1), pack_bf16(a2, a3), pack_bf16(a4, a5), pack_bf16(a6, a7)};
  return __builtin_bit_cast(bf16x8, u);
}

// Buffer resource over [base, base + bytes): loads past the end return zero
// (and, for the LDS-direct form, write zero), so tails need no branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw 32-bit dwords, gfx9 family
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds_base + 16 i (lds_base must be wave-uniform).  The global byte offset
// voff is per lane and is the part the hardware range-checks.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, char* lds_base, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, 0, 0, 0);
}

// LDS-direct loads written as inline assembly, invisible to the compiler's
// LDS dependency tracking: kernels that use them order the ring themselves
// (ring_wait_barrier).  M0 carries the wave-uniform LDS base; nothing else in
// these kernels uses M0.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
// lds_base: wave-uniform LDS byte address (lds_addr of the destination);
// 16 (dma16) or 4 (dma4) bytes per lane, lane i writing lds_base + size i.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void dma4(rsrc_t r, uint32_t lds_base, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(r)
               : "memory");
}
// Wait until at most PENDING of this wave's LDS-direct loads are in flight
// and its LDS reads are done, then barrier.  The "memory" clobber keeps the
// compiler from moving LDS accesses across it.
template <int PENDING>
__device__ __forceinline__ void ring_wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(PENDING) : "memory");
}
__device__ __forceinline__ void dma_drain() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

// Workgroup -> (block, head) map.  Workgroups are dealt round-robin to the 8
// XCDs (each with its own L2); when the head count is a multiple of 8, every
// head's blocks go to one XCD, so the head's K/V (or Q/dO) stream is shared
// through that XCD's L2.  Within an XCD the order is either head by head
// (`lpt` false: a head's blocks run together, the best L2 reuse when all
// blocks cost the same) or block rank by block rank across the XCD's heads
// (`lpt` true: causal blocks differ in cost up to the sequence length over the
// block size, and issuing every head's longest block before any shorter one
// keeps the last workgroups short; head by head, a head issued late puts its
// longest block at the end, which idled about a third of the machine with two
// workgroups per CU).  The rank-by-rank order runs over groups of kLptGroup
// heads, group after group: a group is long enough that its last (short)
// blocks still balance the tail, and few enough heads are in flight on an
// XCD at once that blocks of one head start close together and share its
// tiles in L2 (with all eight heads of an XCD in flight at N = 8192 the L2
// misses were 1.3-1.8x higher and the kernels 1-2 % slower).  `rev` reverses the
// block index (the longest causal block is the last query block, but the
// first key block).
constexpr int kXcds = 8;
constexpr int kLptGroup = 4;
__device__ __forceinline__ void block_head(int id, int nblk, int BH, bool rev, bool lpt, int* blk,
                                           int* bh) {
  int b, hd;
  if ((BH % kXcds) == 0) {
    const int xcd = id % kXcds;
    const int local = id / kXcds;
    const int hpx = BH / kXcds;  // heads per XCD
    if (lpt) {
      const int g0 = (local / (kLptGroup * nblk)) * kLptGroup;  // first head of the group
      const int gs = min(kLptGroup, hpx - g0);                  // heads in the group
      const int w = local - g0 * nblk;
      hd = xcd + kXcds * (g0 + w % gs);
      b = w / gs;
    } else {
      hd = xcd + kXcds * (local / nblk);
      b = local % nblk;
    }
  } else {
    hd = id % BH;
    b = id / BH;
  }
  *blk = rev ? (nblk - 1 - b) : b;
  *bh = hd;
}

__device__ __forceinline__ u32x4 load16_or_zero(const char* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  if (ok) z = *reinterpret_cast<const u32x4*>(p);
  return z;
}

}  // namespace fa
