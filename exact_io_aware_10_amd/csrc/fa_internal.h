// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
// Arguments are validated by the caller; these only launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int N, float scale, int causal, hipStream_t stream);

// D = rowsum(dO * O) into `delta` (B*H*N floats), then the dK/dV and dQ kernels.
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
                      const float* lse, void* dq, void* dk, void* dv, int B, int H, int N,
                      float scale, int causal, float* delta, hipStream_t stream);

}  // namespace fa
