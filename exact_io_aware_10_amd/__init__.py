"""Python binding of libfa.so, the gfx950 exact-attention library.

Argument marshalling only: every step of the attention path runs in the HIP
kernels behind the C ABI declared in include/fa.h.  PyTorch supplies device
memory and the current stream.  There is no fallback: if the library is not
built, or the tensors are not on a ROCm device, the calls raise.

Functions mirror the C entry points:
  fa_fwd(q, k, v, o, lse, scale, causal)                       -> None
  fa_fwd_split(q, k, v, o, lse, scale, causal)                 -> None
  fa_fwd_soft_exp2(q, k, v, o, lse, scale, causal, share)      -> None
  fa_fwd_pingpong(q, k, v, o, lse, scale, causal)              -> None
  fa_bwd(q, k, v, o, dO, lse, dq, dk, dv, scale, causal, ws)   -> None
  fa_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, scale, causal) -> None
  fa_bwd_atomic_dq(q, k, v, o, dO, lse, dq, dk, dv, scale, causal, ws) -> None
  fa_bwd_atomic_workspace_size(B, H, N, d, causal)             -> int
  fa_bwd_dq(q, k, v, o, dO, lse, ws, dq, scale, causal)        -> None
  fa_bwd_dkdv(q, k, v, dO, ws, dk, dv, scale, causal)          -> None
  fa_bwd_preprocess(o, dO, lse, ws)                            -> None
  fa_bwd_workspace_size(B, H, N, d, causal)                    -> int
  fa_fp8_codes_size(B, H, N, d, layout), fa_fp8_exps_size(B, H, N, d) -> int
  fa_fp8_quantize(x, signs, codes, exps, layout)               -> None
  fa_fwd_fp8(q8, qe, k8, ke, v8, ve, signs, o, lse, scale, causal) -> None
  fa_strerror(status)                                          -> str
plus allocating conveniences forward(...), backward(...), quantize_fp8(...)
and forward_fp8(...).
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so libfa.so binds to the HIP runtime torch already holds

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")
HEAD_DIM = 128

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4
FA_ERR_TOO_LARGE = 5
NOALLOC_MAX_ROWS = (16 << 20) // 8   # FA_NOALLOC_MAX_ROWS of include/fa.h

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"libfa status {status}: {fa_strerror(status)}")
        self.status = status


def load_library() -> ctypes.CDLL:
    """Load libfa.so (built in-tree by exact_io_aware_10_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m exact_io_aware_10_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd.restype = i
        lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd_split.restype = i
        lib.fa_fwd_pingpong.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd_pingpong.restype = i
        lib.fa_fwd_soft_exp2.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, vp]
        lib.fa_fwd_soft_exp2.restype = i
        lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
        lib.fa_bwd_workspace_size.restype = sz
        lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
        lib.fa_bwd.restype = i
        lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd_noalloc.restype = i
        lib.fa_bwd_atomic_workspace_size.argtypes = [i, i, i, i, i]
        lib.fa_bwd_atomic_workspace_size.restype = sz
        lib.fa_bwd_atomic_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, sz, vp]
        lib.fa_bwd_atomic_dq.restype = i
        lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, vp, sz, i, i, i, i, vp]
        lib.fa_bwd_preprocess.restype = i
        lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, sz, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd_dkdv.restype = i
        lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, sz, vp, i, i, i, i, f, i, vp]
        lib.fa_bwd_dq.restype = i
        lib.fa_fp8_codes_size.argtypes = [i, i, i, i, i]
        lib.fa_fp8_codes_size.restype = sz
        lib.fa_fp8_exps_size.argtypes = [i, i, i, i]
        lib.fa_fp8_exps_size.restype = sz
        lib.fa_fp8_quantize.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
        lib.fa_fp8_quantize.restype = i
        lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.fa_fwd_fp8.restype = i
        lib.fa_strerror.argtypes = [i]
        lib.fa_strerror.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def fa_strerror(status: int) -> str:
    return load_library().fa_strerror(int(status)).decode()


def fa_bwd_workspace_size(B: int, H: int, N: int, d: int = HEAD_DIM, causal: bool = False) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, N, d, int(bool(causal))))


def fa_bwd_atomic_workspace_size(B: int, H: int, N: int, d: int = HEAD_DIM,
                                 causal: bool = False) -> int:
    return int(load_library().fa_bwd_atomic_workspace_size(B, H, N, d, int(bool(causal))))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_tensor(name, t, dtype, shape):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a ROCm device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shape(q):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    return tuple(q.shape)


def _fwd_call(entry, q, k, v, o, lse, scale, causal, stream):
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    st = getattr(load_library(), entry)(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                        float(scale), int(bool(causal)), _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    _fwd_call("fa_fwd", q, k, v, o, lse, scale, causal, stream)


def fa_fwd_split(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    _fwd_call("fa_fwd_split", q, k, v, o, lse, scale, causal, stream)


def fa_fwd_pingpong(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    _fwd_call("fa_fwd_pingpong", q, k, v, o, lse, scale, causal, stream)


def fa_fwd_soft_exp2(q, k, v, o, lse, scale: float, causal: bool, share: int, stream=None) -> None:
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    st = load_library().fa_fwd_soft_exp2(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d,
                                         float(scale), int(bool(causal)), int(share), _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, workspace,
           stream=None) -> None:
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", do), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq),
                               _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                               _ptr(workspace), nbytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_bwd_atomic_dq(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool, workspace,
                     stream=None) -> None:
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", do), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    st = load_library().fa_bwd_atomic_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                         _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                         int(bool(causal)), _ptr(workspace), nbytes, _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_bwd_noalloc(q, k, v, o, do, lse, dq, dk, dv, scale: float, causal: bool,
                   stream=None) -> None:
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", do), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    st = load_library().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse),
                                       _ptr(dq), _ptr(dk), _ptr(dv), B, H, N, d, float(scale),
                                       int(bool(causal)), _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def _ws(workspace):
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def fa_bwd_preprocess(o, do, lse, workspace, stream=None) -> None:
    B, H, N, d = _shape(o)
    _check_tensor("o", o, torch.bfloat16, (B, H, N, d))
    _check_tensor("dO", do, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    wp, wn = _ws(workspace)
    st = load_library().fa_bwd_preprocess(_ptr(o), _ptr(do), _ptr(lse), wp, wn, B, H, N, d,
                                          _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_bwd_dkdv(q, k, v, do, workspace, dk, dv, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("dO", do), ("dk", dk), ("dv", dv)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    wp, wn = _ws(workspace)
    st = load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(do), wp, wn, _ptr(dk), _ptr(dv),
                                     B, H, N, d, float(scale), int(bool(causal)), _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_bwd_dq(q, k, v, o, do, lse, workspace, dq, scale: float, causal: bool, stream=None) -> None:
    B, H, N, d = _shape(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dO", do), ("dq", dq)):
        _check_tensor(name, t, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    wp, wn = _ws(workspace)
    st = load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), wp, wn,
                                   _ptr(dq), B, H, N, d, float(scale), int(bool(causal)),
                                   _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def forward(q, k, v, scale: float, causal: bool, stream=None):
    """Allocate O and LSE with torch and run fa_fwd.  Returns (o, lse)."""
    B, H, N, d = _shape(q)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, scale, causal, stream)
    return o, lse


def workspace_for(B, H, N, causal, device):
    n = max(fa_bwd_workspace_size(B, H, N, HEAD_DIM, causal), 16)
    return torch.empty(n, dtype=torch.uint8, device=device)


def backward(q, k, v, o, do, lse, scale: float, causal: bool, stream=None, workspace=None):
    """Allocate dQ, dK, dV (and the workspace) with torch and run fa_bwd."""
    B, H, N, d = _shape(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        workspace = workspace_for(B, H, N, causal, q.device)
    fa_bwd(q, k, v, o, do, lse, dq, dk, dv, scale, causal, workspace, stream)
    return dq, dk, dv


# ---------------------------------------------------------------------------
# FP8 path
# ---------------------------------------------------------------------------
FA_FP8_ROWS = 0
FA_FP8_VT = 1


def fa_fp8_codes_size(B: int, H: int, N: int, d: int = HEAD_DIM, layout: int = FA_FP8_ROWS) -> int:
    return int(load_library().fa_fp8_codes_size(B, H, N, d, int(layout)))


def fa_fp8_exps_size(B: int, H: int, N: int, d: int = HEAD_DIM) -> int:
    return int(load_library().fa_fp8_exps_size(B, H, N, d))


def _check_buf(name, t, dtype, nbytes):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous ROCm device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name} needs at least {nbytes} bytes")


def fa_fp8_quantize(x, signs, codes, exps, layout: int, stream=None) -> None:
    B, H, N, d = _shape(x)
    _check_tensor("x", x, torch.bfloat16, (B, H, N, d))
    _check_tensor("signs", signs, torch.float32, (d,))
    _check_buf("codes", codes, torch.uint8, fa_fp8_codes_size(B, H, N, d, layout))
    _check_buf("exps", exps, torch.int32, fa_fp8_exps_size(B, H, N, d))
    st = load_library().fa_fp8_quantize(_ptr(x), _ptr(signs), _ptr(codes), _ptr(exps), B, H, N, d,
                                        int(layout), _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def fa_fwd_fp8(q8, qe, k8, ke, v8, ve, signs, o, lse, scale: float, causal: bool,
               stream=None) -> None:
    B, H, N, d = _shape(o)
    _check_tensor("o", o, torch.bfloat16, (B, H, N, d))
    _check_tensor("lse", lse, torch.float32, (B, H, N))
    _check_tensor("signs", signs, torch.float32, (d,))
    rows = fa_fp8_codes_size(B, H, N, d, FA_FP8_ROWS)
    _check_buf("q8", q8, torch.uint8, rows)
    _check_buf("k8", k8, torch.uint8, rows)
    _check_buf("v8", v8, torch.uint8, fa_fp8_codes_size(B, H, N, d, FA_FP8_VT))
    ne = fa_fp8_exps_size(B, H, N, d)
    for name, t in (("qe", qe), ("ke", ke), ("ve", ve)):
        _check_buf(name, t, torch.int32, ne)
    st = load_library().fa_fwd_fp8(_ptr(q8), _ptr(qe), _ptr(k8), _ptr(ke), _ptr(v8), _ptr(ve),
                                   _ptr(signs), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                                   int(bool(causal)), _stream(stream))
    if st != FA_OK:
        raise FAError(st)


def quantize_fp8(x, signs, layout: int, stream=None):
    """Allocate and fill (codes, exps) for one tensor."""
    B, H, N, d = _shape(x)
    codes = torch.empty(max(fa_fp8_codes_size(B, H, N, d, layout), 16), dtype=torch.uint8, device=x.device)
    exps = torch.empty(max(fa_fp8_exps_size(B, H, N, d) // 4, 4), dtype=torch.int32, device=x.device)
    fa_fp8_quantize(x, signs, codes, exps, layout, stream)
    return codes, exps


def forward_fp8(q, k, v, signs, scale: float, causal: bool, stream=None):
    """Quantise Q, K, V and run the FP8 forward.  Returns (o, lse)."""
    B, H, N, d = _shape(q)
    q8, qe = quantize_fp8(q, signs, FA_FP8_ROWS, stream)
    k8, ke = quantize_fp8(k, signs, FA_FP8_ROWS, stream)
    v8, ve = quantize_fp8(v, signs, FA_FP8_VT, stream)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd_fp8(q8, qe, k8, ke, v8, ve, signs, o, lse, scale, causal, stream)
    return o, lse
