"""MI355X-native exact attention (FlashAttention-2 style) for gfx950.

``forward(q, k, v, causal, scale) -> (o, lse)`` (k, v may hold a different
number of rows than q) and
``backward(q, k, v, o, lse, dout, causal, scale) -> (dq, dk, dv)`` run the HIP
kernels of ``libfa.so`` through its C ABI (include/fa.h).  The library is
loaded on first use and its absence is an error.
"""

from .binding import (  # noqa: F401
    FA_DTYPE_BF16,
    FA_DTYPE_FP16,
    FaError,
    backward,
    fa_bwd,
    fa_fwd,
    fa_fwd_kv,
    fa_last_hip_error,
    fa_status_string,
    fa_version,
    forward,
    library_path,
    load_library,
)
