// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments are validated by the caller; these only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// launch_fwd picks the row-block kernel (launch_fwd_rows) or, for grids too
// small to fill the chip, the key-split kernel (launch_fwd_split).
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, float scale, int causal, hipStream_t stream);
hipError_t launch_fwd_rows(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, float scale, int causal, hipStream_t stream);
hipError_t launch_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int N, float scale, int causal, hipStream_t stream);

// Backward workspace layout (2 B*H*N floats): [D = rowsum(dO * O) | L * log2(e)].
hipError_t launch_bwd_pre(const void* o, const void* dO, const float* lse, float* ws, int B, int H,
                          int N, hipStream_t stream);

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                           const float* ws, void* dk, void* dv, int B, int H, int N, float scale,
                           int causal, hipStream_t stream);

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                         const float* ws, void* dq, int B, int H, int N, float scale, int causal,
                         hipStream_t stream);

// FP8 path (fa_fp8.hip).
hipError_t launch_fp8_quant(const void* x, const float* signs, void* codes, int* exps, int B, int H,
                            int N, int layout, hipStream_t stream);
hipError_t launch_fwd_fp8(const void* q8, const int* qexp, const void* k8, const int* kexp,
                          const void* v8, const int* vexp, const float* signs, void* o, float* lse,
                          int B, int H, int N, float scale, int causal, hipStream_t stream);

}  // namespace fa
