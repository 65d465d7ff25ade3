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
FA_ERR_WORKSPACE = -10
FA_ERR_STRIDE = -11
FA_ERR_SCRATCH = -12
FA_DECODE_NOALLOC_MAX_BYTES = 16 << 20

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
            lib.fa_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
            lib.fa_fwd_kv.restype = i
            lib.fa_fwd_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, ctypes.c_size_t, vp]
            lib.fa_fwd_decode.restype = i
            lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, f, i, vp]
            lib.fa_fwd_strided.restype = i
            lib.fa_fwd_decode_strided.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, f, i, vp,
                                                  ctypes.c_size_t, vp]
            lib.fa_fwd_decode_strided.restype = i
            lib.fa_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
            lib.fa_fwd_decode_noalloc.restype = i
            lib.fa_fwd_decode_workspace_size.argtypes = [i, i, i, i, i]
            lib.fa_fwd_decode_workspace_size.restype = ctypes.c_size_t
            lib.fa_bwd.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, vp]
            lib.fa_bwd.restype = i
            lib.fa_bwd_kv.argtypes = [vp] * 10 + [i, i, i, i, i, i, f, i, vp]
            lib.fa_bwd_kv.restype = i
            lib.fa_bwd_strided.argtypes = [vp] * 10 + [i, i, i, i, i, vp, i, f, i, vp]
            lib.fa_bwd_strided.restype = i
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


def fa_fwd_kv(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, stream) -> int:
    """The C entry point with plain integers as pointers; returns the status."""
    return int(load_library().fa_fwd_kv(q, k, v, o, lse, int(B), int(H), int(Sq), int(Sk), int(d), int(causal),
                                         float(scale), int(dtype), stream))


def fa_fwd_decode(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, workspace, workspace_bytes,
                  stream) -> int:
    """The C entry point with plain integers as pointers; returns the status."""
    return int(load_library().fa_fwd_decode(q, k, v, o, lse, int(B), int(H), int(Sq), int(Sk), int(d), int(causal),
                                             float(scale), int(dtype), workspace, int(workspace_bytes), stream))


def fa_fwd_decode_noalloc(q, k, v, o, lse, B, H, Sq, Sk, d, causal, scale, dtype, stream) -> int:
    """The C entry point with plain integers as pointers; returns the status."""
    return int(load_library().fa_fwd_decode_noalloc(q, k, v, o, lse, int(B), int(H), int(Sq), int(Sk), int(d),
                                                     int(causal), float(scale), int(dtype), stream))


def _strides_arg(strides):
    """Element strides as a host int64 array (None stays NULL)."""
    if strides is None:
        return None
    arr = (ctypes.c_longlong * len(strides))(*[int(x) for x in strides])
    return ctypes.cast(arr, ctypes.c_void_p), arr  # keep arr alive with the pointer


def fa_fwd_strided(q, k, v, o, lse, B, H, Sq, Sk, d, strides, causal, scale, dtype, stream) -> int:
    """The C entry point; ``strides`` is a sequence of 12 element strides (q, k,
    v, o: batch, head, row) or None; returns the status."""
    arg = _strides_arg(strides)
    return int(load_library().fa_fwd_strided(q, k, v, o, lse, int(B), int(H), int(Sq), int(Sk), int(d),
                                              arg[0] if arg else None, int(causal), float(scale), int(dtype),
                                              stream))


def fa_fwd_decode_strided(q, k, v, o, lse, B, H, Sq, Sk, d, strides, causal, scale, dtype, workspace,
                          workspace_bytes, stream) -> int:
    arg = _strides_arg(strides)
    return int(load_library().fa_fwd_decode_strided(q, k, v, o, lse, int(B), int(H), int(Sq), int(Sk), int(d),
                                                     arg[0] if arg else None, int(causal), float(scale),
                                                     int(dtype), workspace, int(workspace_bytes), stream))


def fa_fwd_decode_workspace_size(B, H, Sq, Sk, d) -> int:
    return int(load_library().fa_fwd_decode_workspace_size(int(B), int(H), int(Sq), int(Sk), int(d)))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, S, d, causal, scale, dtype, stream) -> int:
    """The C entry point with plain integers as pointers; returns the status."""
    return int(load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, int(B), int(H), int(S), int(d),
                                      int(causal), float(scale), int(dtype), stream))


def fa_bwd_kv(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Sq, Sk, d, causal, scale, dtype, stream) -> int:
    """The C entry point with plain integers as pointers; returns the status."""
    return int(load_library().fa_bwd_kv(q, k, v, o, lse, dout, dq, dk, dv, delta, int(B), int(H), int(Sq), int(Sk),
                                         int(d), int(causal), float(scale), int(dtype), stream))


def fa_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, Sq, Sk, d, strides, causal, scale, dtype,
                   stream) -> int:
    """The C entry point; ``strides`` is a sequence of 24 element strides (q, k,
    v, o, dout, dq, dk, dv: batch, head, row) or None; returns the status."""
    arg = _strides_arg(strides)
    return int(load_library().fa_bwd_strided(q, k, v, o, lse, dout, dq, dk, dv, delta, int(B), int(H), int(Sq),
                                              int(Sk), int(d), arg[0] if arg else None, int(causal), float(scale),
                                              int(dtype), stream))


class FaError(RuntimeError):
    def __init__(self, status: int, entry: str = "fa_fwd"):
        msg = fa_status_string(status)
        if status == FA_ERR_HIP:
            msg += f" ({fa_last_hip_error()})"
        super().__init__(f"{entry} failed with status {status}: {msg}")
        self.status = status


def _layout(*ts):
    """None when all tensors are contiguous; else their element strides
    (batch, head, row each) for the strided entry points, which need the head
    dimension contiguous."""
    if all(t.is_contiguous() for t in ts):
        return None
    if any(t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1) for t in ts):
        raise ValueError("attention tensors need a contiguous last (head) dimension")
    out = []
    for t in ts:
        # a size-1 dimension's stride is arbitrary in torch: batch / head get
        # 0, a single row gets d (rows past the end must stay out of range)
        out += [t.stride(0) if t.shape[0] > 1 else 0, t.stride(1) if t.shape[1] > 1 else 0,
                t.stride(2) if t.shape[2] > 1 else t.shape[3]]
    return out


def _on_device(device, **named):
    """Every named tensor must live in device memory on ``device`` (the
    kernels read and write them there; a host pointer would fault)."""
    for name, t in named.items():
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{name} must be a device tensor on {device}, got {t.device}")


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            scale: float | None = None, out: torch.Tensor | None = None,
            lse: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Exact attention forward on fp16/bf16 device tensors q [B, H, Sq, d] and
    k, v [B, H, Sk, d].

    Returns (o [B, H, Sq, d] in the input dtype, lse [B, H, Sq] float32).
    With Sq != Sk this is fa_fwd_kv (causal mask aligned to the sequence
    end), else fa_fwd; tensors that are not contiguous (e.g. [B, S, H, d]
    storage viewed as [B, H, S, d], or a slice of a cache) go to
    fa_fwd_strided, and a default ``out`` takes q's layout.  The launch is
    asynchronous on ``stream`` (default: the current stream).
    """
    if (q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[:2] != q.shape[:2]
            or k.shape[3] != q.shape[3]):
        raise ValueError(f"need q [B, H, Sq, d] and k, v [B, H, Sk, d], got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise TypeError("q, k, v must all be float16 or all bfloat16")
    if not q.is_cuda:
        raise ValueError("q, k, v must be device tensors")
    B, H, S, d = q.shape
    Sk = k.shape[2]
    if scale is None:
        scale = float(torch.tensor(d, dtype=torch.float32).rsqrt())
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _on_device(q.device, k=k, v=v, out=out, lse=lse)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be a tensor like q")
    if lse.shape != (B, H, S) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    strides = _layout(q, k, v, out)
    if strides is not None:
        st, entry = fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   B, H, S, Sk, d, strides, 1 if causal else 0, scale, _DTYPES[q.dtype],
                                   s.cuda_stream), "fa_fwd_strided"
    elif Sk == S:
        st, entry = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           B, H, S, d, 1 if causal else 0, scale, _DTYPES[q.dtype], s.cuda_stream), "fa_fwd"
    else:
        st, entry = fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                              B, H, S, Sk, d, 1 if causal else 0, scale, _DTYPES[q.dtype],
                              s.cuda_stream), "fa_fwd_kv"
    if st != FA_OK:
        raise FaError(st, entry)
    return out, lse


def decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
           scale: float | None = None, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
           workspace: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """fa_fwd_decode: q [B, H, Sq, d] (Sq small, e.g. 1) over k, v [B, H, Sk, d],
    split over the keys.  Same results as ``forward`` to rounding.

    ``workspace`` is a uint8 device tensor of at least
    ``fa_fwd_decode_workspace_size(B, H, Sq, Sk, d)`` bytes (allocated here if
    not given).  Non-contiguous tensors (e.g. the first Sk rows of a
    [B, S_max, H, d] cache viewed as [B, H, Sk, d]) go to
    fa_fwd_decode_strided.  Returns (o, lse).  Asynchronous on ``stream``.
    """
    if (q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[:2] != q.shape[:2]
            or k.shape[3] != q.shape[3]):
        raise ValueError(f"need q [B, H, Sq, d] and k, v [B, H, Sk, d], got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise TypeError("q, k, v must all be float16 or all bfloat16")
    if not q.is_cuda:
        raise ValueError("q, k, v must be device tensors")
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    if scale is None:
        scale = float(torch.tensor(d, dtype=torch.float32).rsqrt())
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device) if lse is None else lse
    _on_device(q.device, k=k, v=v, out=out, lse=lse)
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be a tensor like q")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    need = fa_fwd_decode_workspace_size(B, H, Sq, Sk, d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _on_device(q.device, workspace=workspace)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = workspace.numel() * workspace.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    strides = _layout(q, k, v, out)
    if strides is None:
        st, entry = fa_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H,
                                  Sq, Sk, d, 1 if causal else 0, scale, _DTYPES[q.dtype], workspace.data_ptr(),
                                  nbytes, s.cuda_stream), "fa_fwd_decode"
    else:
        st, entry = fa_fwd_decode_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                          lse.data_ptr(), B, H, Sq, Sk, d, strides, 1 if causal else 0, scale,
                                          _DTYPES[q.dtype], workspace.data_ptr(), nbytes,
                                          s.cuda_stream), "fa_fwd_decode_strided"
    if st != FA_OK:
        raise FaError(st, entry)
    return out, lse


def decode_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                   causal: bool = False, scale: float | None = None, stream: torch.cuda.Stream | None = None):
    """fa_fwd_decode_noalloc: ``decode`` with the library's own scratch array
    instead of a workspace, for callers that cannot allocate.  Dense tensors
    only; ``out`` [B, H, Sq, d] and ``lse`` [B, H, Sq] float32 are the
    caller's.  Calls that may overlap on one device race on the shared array.
    Returns (out, lse)."""
    if (q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or k.shape[:2] != q.shape[:2]
            or k.shape[3] != q.shape[3]):
        raise ValueError(f"need q [B, H, Sq, d] and k, v [B, H, Sk, d], got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DTYPES:
        raise TypeError("q, k, v must all be float16 or all bfloat16")
    if not q.is_cuda:
        raise ValueError("q, k, v must be device tensors")
    _on_device(q.device, k=k, v=v, out=out, lse=lse)
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must be a tensor like q")
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, Sq] tensor")
    if not all(t.is_contiguous() for t in (q, k, v, out, lse)):
        raise ValueError("fa_fwd_decode_noalloc takes dense (contiguous) tensors")
    if scale is None:
        scale = float(torch.tensor(d, dtype=torch.float32).rsqrt())
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    st = fa_fwd_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Sq,
                               Sk, d, 1 if causal else 0, scale, _DTYPES[q.dtype], s.cuda_stream)
    if st != FA_OK:
        raise FaError(st, "fa_fwd_decode_noalloc")
    return out, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, lse: torch.Tensor,
             dout: torch.Tensor, causal: bool = False, scale: float | None = None,
             dq: torch.Tensor | None = None, dk: torch.Tensor | None = None, dv: torch.Tensor | None = None,
             delta: torch.Tensor | None = None, stream: torch.cuda.Stream | None = None):
    """Gradients (dq, dk, dv) of exact attention for the upstream gradient dout.

    q, o, dout: [B, H, Sq, d] and k, v: [B, H, Sk, d] fp16/bf16 device tensors
    (o and lse from ``forward`` on the same inputs, causal flag and scale;
    with Sq != Sk the causal mask is aligned to the end, as in ``forward``);
    lse: [B, H, Sq] float32.  ``delta`` is a [B, H, Sq] float32 scratch
    buffer the call fills with D_i = dout_i . o_i (allocated here if not
    given).  Square problems go through fa_bwd, others through fa_bwd_kv;
    tensors with a contiguous last dimension but other strides (a
    [B, S, H, d] storage seen through ``transpose(1, 2)``, slices of a packed
    QKV buffer) through fa_bwd_strided.  Gradients allocated here match the
    layout of q (dq) and k (dk, dv).  Asynchronous on ``stream`` (default:
    the current stream).
    """
    ts = (q, k, v, o, dout)
    if q.dim() != 4 or any(t.dim() != 4 for t in ts):
        raise ValueError("q, k, v, o, dout must be 4-d [B, H, S, d] tensors")
    B, H, Sq, d = q.shape
    Sk = k.shape[2]
    if o.shape != q.shape or dout.shape != q.shape or k.shape != (B, H, Sk, d) or v.shape != k.shape:
        raise ValueError("q, o, dout must be [B, H, Sq, d] and k, v [B, H, Sk, d]")
    if any(t.dtype != q.dtype for t in ts) or q.dtype not in _DTYPES:
        raise TypeError("q, k, v, o, dout must all be float16 or all bfloat16")
    if not q.is_cuda:
        raise ValueError("q, k, v, o, dout must be device tensors")
    _on_device(q.device, k=k, v=v, o=o, dout=dout, lse=lse)
    if lse.shape != (B, H, Sq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, Sq] tensor")
    if scale is None:
        scale = float(torch.tensor(d, dtype=torch.float32).rsqrt())
    # empty_like keeps the source's strides when it is dense in some permutation
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    if delta is None:
        delta = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _on_device(q.device, dq=dq, dk=dk, dv=dv, delta=delta)
    for name, t, like in (("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t.shape != like.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must be a device tensor shaped like {'q' if like is q else 'k'}")
    if delta.shape != (B, H, Sq) or delta.dtype != torch.float32 or not delta.is_contiguous():
        raise ValueError("delta must be a contiguous float32 [B, H, Sq] tensor")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr())
    strides = _layout(q, k, v, o, dout, dq, dk, dv)
    c, dt = 1 if causal else 0, _DTYPES[q.dtype]
    if strides is not None:
        st, entry = fa_bwd_strided(*ptrs, B, H, Sq, Sk, d, strides, c, scale, dt, s.cuda_stream), "fa_bwd_strided"
    elif Sq == Sk:
        st, entry = fa_bwd(*ptrs, B, H, Sq, d, c, scale, dt, s.cuda_stream), "fa_bwd"
    else:
        st, entry = fa_bwd_kv(*ptrs, B, H, Sq, Sk, d, c, scale, dt, s.cuda_stream), "fa_bwd_kv"
    if st != FA_OK:
        raise FaError(st, entry)
    return dq, dk, dv
