// C ABI of libfa.so: argument validation and dispatch to the HIP kernels.
// Declared in include/fa.h; every check runs before anything is launched.
#include "fa.h"

#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace {

constexpr int kHeadDim = 128;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared shape/scalar checks.  Returns FA_OK, or the status to report.
// *empty is set when there is nothing to compute (some of B, H, N is 0).
int check_common(int B, int H, int N, int d, float scale, int causal, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (d != kHeadDim) return FA_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  const int64_t elems = (int64_t)B * H * N * d;
  if (elems >= ((int64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  // Per-head byte offsets (plus one tile of padding) must fit the 32-bit
  // buffer offsets the kernels use.
  if ((int64_t)N * d * 2 + 65536 >= ((int64_t)1 << 32)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Argument checks shared by the forward entry points, then the launch.
typedef hipError_t (*fwd_launcher)(const void*, const void*, const void*, void*, float*, int, int,
                                   int, float, int, hipStream_t);
int checked_fwd(fwd_launcher launch, const void* q, const void* k, const void* v, void* o,
                float* lse, int B, int H, int N, int d, float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_UNSUPPORTED;
  hipError_t e = launch(q, k, v, o, lse, B, H, N, scale, causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, void* stream) {
  return checked_fwd(fa::launch_fwd, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, void* stream) {
  return checked_fwd(fa::launch_fwd_split, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_pingpong(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int d, float scale, int causal, void* stream) {
  return checked_fwd(fa::launch_fwd_pingpong, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_soft_exp2(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int N, int d, float scale, int causal, int software_share,
                     void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK) return st;
  if (software_share != 0 && software_share != 8 && software_share != 16 && software_share != 32)
    return FA_ERR_INVALID_ARG;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_fwd_soft_exp2(q, k, v, o, lse, B, H, N, scale, causal, software_share,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, int causal) {
  bool empty = false;
  if (check_common(B, H, N, d, 1.f, causal, &empty) != FA_OK) return 0;
  if (empty) return 0;
  const size_t bytes = 2 * (size_t)B * H * N * sizeof(float);  // D and L log2(e)
  return (bytes + 255) & ~(size_t)255;
}

int fa_bwd_preprocess(const void* o, const void* dO, const float* lse, void* workspace,
                      size_t workspace_bytes, int B, int H, int N, int d, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, 1.f, 0, &empty);
  if (st != FA_OK || empty) return st;
  if (!o || !dO || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(dO) || !aligned16(lse)) return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, H, N, d, 0) || !aligned16(workspace))
    return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_bwd_pre(o, dO, lse, static_cast<float*>(workspace), B, H, N,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const void* workspace,
                size_t workspace_bytes, void* dk, void* dv, int B, int H, int N, int d, float scale,
                int causal, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !dO || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dk) ||
      !aligned16(dv))
    return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, H, N, d, causal) ||
      !aligned16(workspace))
    return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_bwd_dkdv(q, k, v, dO, static_cast<const float*>(workspace), dk, dv, B,
                                     H, N, scale, causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
              const float* lse, void* workspace, size_t workspace_bytes, void* dq, int B, int H,
              int N, int d, float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq))
    return FA_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < fa_bwd_workspace_size(B, H, N, d, causal) ||
      !aligned16(workspace))
    return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_bwd_dq(q, k, v, o, dO, lse, static_cast<float*>(workspace), dq, B, H,
                                   N, scale, causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale,
           int causal, void* workspace, size_t workspace_bytes, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_UNSUPPORTED;
  const size_t need = fa_bwd_workspace_size(B, H, N, d, causal);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  float* ws = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = fa::launch_bwd_dq(q, k, v, o, dO, lse, ws, dq, B, H, N, scale, causal, s);
  if (e == hipSuccess) e = fa::launch_bwd_dkdv(q, k, v, dO, ws, dk, dv, B, H, N, scale, causal, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                   float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_UNSUPPORTED;
  if (fa_bwd_workspace_size(B, H, N, d, causal) > (size_t)FA_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_TOO_LARGE;
  hipError_t e = fa::launch_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, scale, causal,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_atomic_workspace_size(int B, int H, int N, int d, int causal) {
  bool empty = false;
  if (check_common(B, H, N, d, 1.f, causal, &empty) != FA_OK) return 0;
  if (empty) return 0;
  return fa::bwd_atomic_dq_offset(B, H, N) + (size_t)B * H * N * d * sizeof(float);
}

int fa_bwd_atomic_dq(const void* q, const void* k, const void* v, const void* o, const void* dO,
                     const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                     float scale, int causal, void* workspace, size_t workspace_bytes,
                     void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_UNSUPPORTED;
  const size_t need = fa_bwd_atomic_workspace_size(B, H, N, d, causal);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return FA_ERR_WORKSPACE;
  hipError_t e = fa::launch_bwd_atomic(q, k, v, o, dO, lse, workspace, dq, dk, dv, B, H, N, scale,
                                       causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fp8_codes_size(int B, int H, int N, int d, int layout) {
  bool empty = false;
  if (check_common(B, H, N, d, 1.f, 0, &empty) != FA_OK || empty) return 0;
  if (layout == FA_FP8_ROWS) return (size_t)B * H * N * d;
  if (layout == FA_FP8_VT) return (size_t)B * H * ((N + 63) / 64) * 64 * d;
  return 0;
}

size_t fa_fp8_exps_size(int B, int H, int N, int d) {
  bool empty = false;
  if (check_common(B, H, N, d, 1.f, 0, &empty) != FA_OK || empty) return 0;
  return (size_t)B * H * ((N + 63) / 64) * sizeof(int);
}

int fa_fp8_quantize(const void* x, const float* signs, void* codes, int* exps, int B, int H, int N,
                    int d, int layout, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, 1.f, 0, &empty);
  if (st != FA_OK || empty) return st;
  if (layout != FA_FP8_ROWS && layout != FA_FP8_VT) return FA_ERR_INVALID_ARG;
  if (!x || !signs || !codes || !exps) return FA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(signs) || !aligned16(codes) || !aligned16(exps))
    return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_fp8_quant(x, signs, codes, exps, B, H, N, layout,
                                      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q8, const int* qexp, const void* k8, const int* kexp, const void* v8,
               const int* vexp, const float* signs, void* o, float* lse, int B, int H, int N, int d,
               float scale, int causal, void* stream) {
  bool empty = false;
  int st = check_common(B, H, N, d, scale, causal, &empty);
  if (st != FA_OK || empty) return st;
  if (!q8 || !qexp || !k8 || !kexp || !v8 || !vexp || !signs || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned16(q8) || !aligned16(qexp) || !aligned16(k8) || !aligned16(kexp) || !aligned16(v8) ||
      !aligned16(vexp) || !aligned16(signs) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_UNSUPPORTED;
  hipError_t e = fa::launch_fwd_fp8(q8, qexp, k8, kexp, v8, vexp, signs, o, lse, B, H, N, scale,
                                    causal, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size, non-finite scale or bad causal flag)";
    case FA_ERR_UNSUPPORTED: return "unsupported (head dim other than 128, misaligned pointer, or size overflow)";
    case FA_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than fa_bwd_workspace_size()";
    case FA_ERR_HIP: return "HIP runtime rejected the launch";
    case FA_ERR_TOO_LARGE:
      return "problem too large for fa_bwd_noalloc's fixed scratch (B*H*N above FA_NOALLOC_MAX_ROWS)";
    default: return "unknown status";
  }
}

}  // extern "C"
