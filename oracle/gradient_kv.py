"""Plain fp64 CPU oracle for the gradients of exact attention with separate
query and key lengths.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``exact_attention_16_amd/``.

What it computes: the gradients of ``oracle.kv``'s forward definition (Sq
query rows over Sk keys, causal mask aligned to the end: key j is kept for
query row i iff j <= i + Sk - Sq) with respect to q, k and v, for an upstream
gradient dO of the output.  The pages fix that the method's gradients equal
those of the plain calculation up to rounding (IPLEX blog "FlashAttention-2:
making long-context attention run efficiently on GPUs", section "Tiling
preserves the attention calculation") and give no formula, so the steps are
the chain rule of the forward definition, exactly as ``oracle.gradient``
writes them for the square case, on P of shape [Sq, Sk]:

    P_ij  = exp(s_ij - LSE_i) for j in A(i), 0 otherwise
    dV = P^T dO,   dP = dO V^T,   D_i = sum_j P_ij dP_ij,
    dS_ij = P_ij (dP_ij - D_i),   dQ = scale dS K,   dK = scale dS^T Q.

Reading for rows with no key (causal with Sq > Sk, rows i < Sq - Sk): the
forward output of such a row is the constant 0 whatever q_i, k and v are, so
its P row is 0, its dQ row is 0 and it adds nothing to dK and dV.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import exact, gradient, kv

__all__ = ["attention_backward_kv", "attention_backward_kv_head", "probabilities_kv"]


def probabilities_kv(q, k, causal: bool, scale: float):
    """P [Sq, Sk] of one head (forward definition of ``oracle.kv``)."""
    Sq, Sk = q.shape[0], k.shape[0]
    allowed = kv.allowed_keys_kv(np.arange(Sq), Sq, Sk, causal)
    p = np.zeros((Sq, Sk))
    live = allowed.any(axis=1)
    if live.any():
        s = exact._apply_mask(exact._scores(q[live], k, float(scale)), allowed[live])
        lse = exact._logsumexp(s, exact._row_max(s))
        p[live] = exact._probabilities(s, lse)
    return p


def attention_backward_kv_head(q, k, v, do, causal: bool, scale: float):
    """(dQ [Sq, d], dK [Sk, d], dV [Sk, d]) of one head, float64."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    p = probabilities_kv(q, k, causal, scale)
    dv = gradient._grad_v(p, do)
    dp = gradient._grad_p(do, v)
    ds = gradient._grad_s(p, dp, gradient._row_delta(p, dp))
    return gradient._grad_q(ds, k, scale), gradient._grad_k(ds, q, scale), dv


def attention_backward_kv(q, k, v, do, causal: bool, scale: float, workers: int = 1):
    """q, do [B, H, Sq, d], k, v [B, H, Sk, d] -> (dq, dk, dv), head by head."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, H = q.shape[:2]
    dq, dk, dv = np.empty_like(q), np.empty_like(k), np.empty_like(v)

    def one(bh):
        b, h = divmod(bh, H)
        dq[b, h], dk[b, h], dv[b, h] = attention_backward_kv_head(q[b, h], k[b, h], v[b, h], do[b, h],
                                                                  causal, scale)

    if workers <= 1:
        for bh in range(B * H):
            one(bh)
    else:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(one, range(B * H)))
    return dq, dk, dv
