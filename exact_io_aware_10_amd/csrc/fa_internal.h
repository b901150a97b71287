// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments are validated by the caller; these only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// A signed softmax scale, as the kernels take it.  The scores are
// scale * q . k; the kernels work with the magnitude `mag` (> 0) and fold the
// sign into the operand they hold in registers (Q, or K in the dK/dV kernel):
// its bit patterns are ANDed with `keep` and XORed with `flip`.  Negating
// every element is exact, and so the scores come out exactly negated; for
// scale = 0 the operand is cleared, every visible score is exactly 0 and the
// weights are uniform over the visible keys (mag is then an arbitrary
// positive value that multiplies zeros).  `sign_bits` holds the sign bit of
// every element packed in a 32-bit word (0x80008000 for bf16 pairs,
// 0x80808080 for four FP8 codes).
struct signed_scale {
  float mag;
  uint32_t keep, flip;
};
inline signed_scale split_scale(float scale, uint32_t sign_bits) {
  if (scale > 0.f) return {scale, 0xffffffffu, 0u};
  if (scale < 0.f) return {-scale, 0xffffffffu, sign_bits};
  return {1.f, 0u, 0u};
}
constexpr uint32_t kSignBitsBf16 = 0x80008000u;
constexpr uint32_t kSignBitsFp8 = 0x80808080u;

// launch_fwd picks the row-block kernel (launch_fwd_rows) or, for grids too
// small to fill the chip, the key-split kernel (launch_fwd_split).
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, float scale, int causal, hipStream_t stream);
hipError_t launch_fwd_rows(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, float scale, int causal, hipStream_t stream);
hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, float scale, int causal, hipStream_t stream);
// The ping-pong forward (fwd_pp_kernel): the row-block tiling with waves
// w and w + 4 of a SIMD one phase apart.
hipError_t launch_fwd_pingpong(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, float scale, int causal, hipStream_t stream);
// The row-block kernel with `share` (0, 8, 16 or 32) of each lane's 32
// exponentials per tile computed on the FMA path (soft_exp2).
hipError_t launch_fwd_soft_exp2(const void* q, const void* k, const void* v, void* o, float* lse,
                                int B, int H, int N, float scale, int causal, int share,
                                hipStream_t stream);

// Fused backward with atomic dQ: workspace [-D | L log2(e)] (padded to 256
// bytes, bwd_atomic_dq_offset) followed by an fp32 dQ buffer of B*H*N*128.
size_t bwd_atomic_dq_offset(int B, int H, int N);
hipError_t launch_bwd_atomic(const void* q, const void* k, const void* v, const void* o,
                             const void* dO, const float* lse, void* ws, void* dq, void* dk,
                             void* dv, int B, int H, int N, float scale, int causal,
                             hipStream_t stream);

// Backward workspace layout (2 B*H*N floats): [-D = -rowsum(dO * O) | L * log2(e)].
hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ws, int B, int H,
                          int N, hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* ws, void* dk, void* dv, int B, int H, int N, float scale,
                           int causal, hipStream_t stream);

// dQ, and [-D | L log2(e)] of every row written into ws for the dK/dV kernel.
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                         const void* dO, const float* lse, float* ws, void* dq, int B, int H, int N,
                         float scale, int causal, hipStream_t stream);

// The backward with its workspace in the library's fixed per-GPU scratch
// array (fa_bwd.hip); the caller has checked the size against it.
hipError_t launch_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const void* dO, const float* lse, void* dq, void* dk, void* dv,
                              int B, int H, int N, float scale, int causal, hipStream_t stream);

// FP8 path (fa_fp8.hip).
hipError_t launch_fp8_quant(const void* x, const float* signs, void* codes, int* exps, int B, int H,
                            int N, int layout, hipStream_t stream);
hipError_t launch_fwd_fp8(const void* q8, const int* qexp, const void* k8, const int* kexp,
                          const void* v8, const int* vexp, const float* signs, void* o, float* lse,
                          int B, int H, int N, float scale, int causal, hipStream_t stream);

}  // namespace fa
