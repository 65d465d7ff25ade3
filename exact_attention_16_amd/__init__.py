"""MI355X-native exact attention (FlashAttention-2 style) for gfx950.

``forward(q, k, v, causal, scale) -> (o, lse)`` (k, v may hold a different
number of rows than q), ``decode(q, k, v, causal, scale) -> (o, lse)`` (the
same split over the keys, for a few queries over many keys) and
``backward(q, k, v, o, lse, dout, causal, scale) -> (dq, dk, dv)`` (also with
separate lengths and strided layouts) run the HIP
kernels of ``libfa.so`` through its C ABI (include/fa.h).  The library is
loaded on first use and its absence is an error.
"""

from .binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_FP16,
    FA_DECODE_NOALLOC_MAX_BYTES,
    FA_ERR_SCRATCH,
    FA_ERR_STRIDE,
    FA_ERR_WORKSPACE,
    FaError,
    backward,
    decode,
    decode_noalloc,
    fa_bwd,
    fa_bwd_kv,
    fa_bwd_strided,
    fa_fwd,
    fa_fwd_decode,
    fa_fwd_decode_noalloc,
    fa_fwd_decode_strided,
    fa_fwd_decode_workspace_size,
    fa_fwd_kv,
    fa_fwd_strided,
    fa_last_hip_error,
    fa_status_string,
    fa_version,
    forward,
    library_path,
    load_library,
)
