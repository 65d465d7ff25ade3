"""Plain fp64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``exact_attention_16_amd/``.

What the pages fix: the method is exact attention used to train GPT-style
models (searcharxiv abstract page, "Abstract"), and its outputs and gradients
differ from the plain calculation only by floating-point rounding, so they are
compared with tolerances (IPLEX blog "FlashAttention-2: making long-context
attention run efficiently on GPUs", section "Tiling preserves the attention
calculation").  The pages do not describe how the gradients are computed, so
the oracle is the gradient of the forward definition (see ``oracle.exact``),
obtained by the chain rule and written out, per (batch b, head h), in float64
on the float64 upcast of the dtype-rounded inputs.  With dO the gradient of a
scalar loss with respect to O:

    P_ij  = exp(s_ij - LSE_i) for j in A(i), 0 otherwise   (forward definition)
    dV    = P^T dO
    dP    = dO V^T
    D_i   = sum_j P_ij dP_ij
    dS_ij = P_ij (dP_ij - D_i)
    dQ    = scale * dS K
    dK    = scale * dS^T Q

(dS is the gradient with respect to the scaled scores s; the softmax Jacobian
of row i is diag(P_i) - P_i P_i^T, which gives the D_i term.)  Because
sum_j P_ij v_j = O_i, D_i also equals dO_i . O_i; ``backward_samples`` uses that
identity so single key columns can be checked without the whole S x S block,
and a pin checks the two forms against each other.

Each step is its own small function so a test can plant a mistake in exactly
one of them and show that a pin catches it.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import exact

__all__ = ["attention_backward", "attention_backward_head", "backward_samples"]


def _probabilities(q, k, causal: bool, scale: float):
    """P [S, S] of one head (forward definition, full rows)."""
    S = q.shape[0]
    s = exact._apply_mask(exact._scores(q, k, scale), exact.allowed_key_mask(np.arange(S), S, causal))
    lse = exact._logsumexp(s, exact._row_max(s))
    return exact._probabilities(s, lse)


def _grad_v(p, do):
    """dV = P^T dO."""
    return p.T @ do


def _grad_p(do, v):
    """dP = dO V^T."""
    return do @ v.T


def _row_delta(p, dp):
    """D_i = sum_j P_ij dP_ij."""
    return np.sum(p * dp, axis=1)


def _grad_s(p, dp, dlt):
    """dS_ij = P_ij (dP_ij - D_i)."""
    return p * (dp - dlt[:, None])


def _grad_q(ds, k, scale: float):
    """dQ = scale * dS K."""
    return scale * (ds @ k)


def _grad_k(ds, q, scale: float):
    """dK = scale * dS^T Q."""
    return scale * (ds.T @ q)


def attention_backward_head(q, k, v, do, causal: bool, scale: float):
    """(dQ, dK, dV) of one head; all arguments [S, d] float64."""
    p = _probabilities(q, k, causal, scale)
    dv = _grad_v(p, do)
    dp = _grad_p(do, v)
    ds = _grad_s(p, dp, _row_delta(p, dp))
    return _grad_q(ds, k, scale), _grad_k(ds, q, scale), dv


def attention_backward(q, k, v, do, causal: bool, scale: float, workers: int = 1):
    """(dQ, dK, dV) of [B, H, S, d] tensors (float64 numpy), head by head."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H = q.shape[:2]
    dq, dk, dv = (np.empty_like(q) for _ in range(3))

    def one(bh):
        b, h = divmod(bh, H)
        dq[b, h], dk[b, h], dv[b, h] = attention_backward_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                               causal, scale)

    if workers <= 1:
        for bh in range(B * H):
            one(bh)
    else:
        try:
            from threadpoolctl import threadpool_limits
            limit = threadpool_limits(1, "blas")
        except ImportError:  # pragma: no cover
            limit = None
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(one, range(B * H)))
        if limit is not None:
            limit.unregister()
    return dq, dk, dv


def backward_samples(q, k, v, do, causal: bool, scale: float, q_rows, kv_rows):
    """Selected gradient rows of whole tensors.

    ``q_rows``: (b, h, i) triples -> dQ rows; ``kv_rows``: (b, h, j) triples ->
    dK and dV rows.  Each head touched is run through the forward definition
    once (LSE and O of every row), then single rows of dQ use P_i. and dP_i.,
    and single key rows use the column P_.j, dP_.j with D_i = dO_i . O_i.
    Returns (dq [n, d], dk [m, d], dv [m, d]).
    """
    q_rows = [tuple(int(x) for x in t) for t in q_rows]
    kv_rows = [tuple(int(x) for x in t) for t in kv_rows]
    d = q.shape[3]
    dq = np.empty((len(q_rows), d))
    dk = np.empty((len(kv_rows), d))
    dv = np.empty((len(kv_rows), d))
    heads = sorted({(b, h) for b, h, _ in q_rows} | {(b, h) for b, h, _ in kv_rows})
    for b, h in heads:
        qh, kh, vh, doh = (np.asarray(x[b, h], dtype=np.float64) for x in (q, k, v, do))
        S = qh.shape[0]
        o, lse = exact.attention_head(qh, kh, vh, causal, scale)
        dlt = np.sum(doh * o, axis=1)
        for t, (bb, hh, i) in enumerate(q_rows):
            if (bb, hh) != (b, h):
                continue
            keys = np.arange(i + 1) if causal else np.arange(S)
            p = np.exp(scale * (kh[keys] @ qh[i]) - lse[i])
            dp = vh[keys] @ doh[i]
            dq[t] = scale * ((p * (dp - dlt[i])) @ kh[keys])
        for t, (bb, hh, j) in enumerate(kv_rows):
            if (bb, hh) != (b, h):
                continue
            rows = np.arange(j, S) if causal else np.arange(S)
            p = np.exp(scale * (qh[rows] @ kh[j]) - lse[rows])
            dp = doh[rows] @ vh[j]
            ds = p * (dp - dlt[rows])
            dv[t] = p @ doh[rows]
            dk[t] = scale * (ds @ qh[rows])
    return dq, dk, dv
