"""Thin ctypes binding of libfa.so (argument marshalling only).

Every step of the attention computation runs in the library's HIP kernels;
PyTorch only supplies device memory and the current stream.  If the library is
not built the first call raises -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

PKG = os.path.dirname(os.path.abspath(__file__))

FA_DTYPE_FP16 = 0
FA_DTYPE_BF16 = 1
FA_OK = 0
FA_ERR_HIP = -9

_DTYPES = {torch.float16: FA_DTYPE_FP16, torch.bfloat16: FA_DTYPE_BF16}

_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return os.environ.get("FA_LIBRARY", os.path.join(PKG, "libfa.so"))


def load_library() -> ctypes.CDLL:
    """Load libfa.so once; raise if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"{path} is not built; run `python -m exact_attention_16_amd.build` "
                    "(or __graft_entry__.build()) first")
            lib = ctypes.CDLL(path)
            vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
            lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
            lib.fa_fwd.restype = i
            lib.fa_status_string.argtypes = [i]
            lib.fa_status_string.restype = ctypes.c_char_p
            lib.fa_last_hip_error.argtypes = []
            lib.fa_last_hip_error.restype = ctypes.c_char_p
            lib.fa_version.argtypes = []
            lib.fa_version.restype = i
            _lib = lib
    return _lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_last_hip_error() -> str:
    return load_library().fa_last_hip_error().decode()


def fa_version() -> int:
    return int(load_library().fa_version())


def fa_fwd(q, k, v, o, lse, B, H, S, d, causal, scale, dtype, stream) -> int:
    """The C entry point with plain integers as pointers; returns the status."""
    return int(load_library().fa_fwd(q, k, v, o, lse, int(B), int(H), int(S), int(d), int(causal),
                                      float(scale), int(dtype), stream))


class FaError(RuntimeError):
    def __init__(self, status: int):
        msg = fa_status_string(status)
        if status == FA_ERR_HIP:
            msg += f" ({fa_last_hip_error()})"
        super().__init__(f"fa_fwd failed with status {status}: {msg}")
        self.status = status


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Exact attention forward on [B, H, S, d] fp16/bf16 device tensors.

    Returns (o [B, H, S, d] in the input dtype, lse [B, H, S] float32).  The
    launch is asynchronous on ``stream`` (default: the current stream).
    """
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError(f"q, k, v must share one [B, H, S, d] shape, got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise TypeError("q, k, v must all be float16 or all bfloat16")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be device tensors")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, S, d = q.shape
    if scale is None:
        scale = float(torch.tensor(d, dtype=torch.float32).rsqrt())
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, S, d, 1 if causal else 0, scale, _DTYPES[q.dtype], s.cuda_stream)
    if st != FA_OK:
        raise FaError(st)
    return out, lse
