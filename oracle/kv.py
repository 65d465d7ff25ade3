"""Plain fp64 CPU oracle for exact attention with separate query and key lengths.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``exact_attention_16_amd/``.

What it computes: the forward definition of ``oracle.exact`` for Sq query
rows over Sk keys.  The pages separate the processing of a long prompt from
token-by-token generation (IPLEX blog "FlashAttention-2: making long-context
attention run efficiently on GPUs", section "Document the implementation
difference"); in generation the new queries are the last Sq positions of a
sequence whose first Sk positions are the keys.  Readings (the pages give no
formula for these shapes):

* causal masking is aligned to the end ("bottom-right"): query row i is at
  sequence position i + (Sk - Sq), so key j is kept iff j <= i + Sk - Sq.
  With Sq = Sk this is the square causal mask of ``oracle.exact``; with
  Sq = 1 the single query sees every key.
* a row with no key left (only when causal and Sq > Sk, for rows
  i < Sq - Sk) has O_i = 0 and LSE_i = -inf: the softmax over an empty set is
  taken as contributing nothing.

Per (b, h), per query row i, in float64 on the dtype-rounded inputs:

    A(i)  = {0 .. Sk-1}                     (no mask)
          = {j : j <= i + Sk - Sq}          (causal)
    s_ij  = scale * q_i . k_j,   LSE_i = ln sum_{j in A(i)} exp(s_ij)
    O_i   = sum_{j in A(i)} exp(s_ij - LSE_i) v_j
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import exact

__all__ = ["allowed_keys_kv", "attention_kv", "attention_kv_rows", "attention_kv_samples"]


def allowed_keys_kv(rows, Sq: int, Sk: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), Sk]: True where key j is in A(i) for query row i."""
    keys = np.arange(Sk)[None, :]
    if causal:
        return keys <= np.asarray(rows)[:, None] + (Sk - Sq)
    return np.ones((len(rows), Sk), dtype=bool)


def attention_kv_rows(q_rows, row_ids, Sq: int, k, v, causal: bool, scale: float):
    """(o [n, d], lse [n]) for query rows ``row_ids`` of one head (k, v: [Sk, d])."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    allowed = allowed_keys_kv(row_ids, Sq, k.shape[0], causal)
    o = np.zeros((q_rows.shape[0], v.shape[1]))
    lse = np.full(q_rows.shape[0], -np.inf)
    live = allowed.any(axis=1)
    if live.any():
        s = exact._apply_mask(exact._scores(q_rows[live], k, float(scale)), allowed[live])
        m = exact._row_max(s)
        lse[live] = exact._logsumexp(s, m)
        o[live] = exact._output(exact._probabilities(s, lse[live]), v)
    return o, lse


def attention_kv(q, k, v, causal: bool, scale: float, workers: int = 1):
    """q [B, H, Sq, d], k, v [B, H, Sk, d] -> (o [B, H, Sq, d], lse [B, H, Sq])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    B, H, Sq, _ = q.shape
    o = np.empty((B, H, Sq, v.shape[3]))
    lse = np.empty((B, H, Sq))
    step = max(1, exact._MAX_BLOCK_ELEMS // max(1, k.shape[2]))

    def one(bh):
        b, h = divmod(bh, H)
        for r0 in range(0, Sq, step):
            rows = np.arange(r0, min(Sq, r0 + step))
            o[b, h, rows], lse[b, h, rows] = attention_kv_rows(q[b, h, rows], rows, Sq, k[b, h], v[b, h], causal,
                                                               scale)

    if workers <= 1:
        for bh in range(B * H):
            one(bh)
    else:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(one, range(B * H)))
    return o, lse


def attention_kv_samples(q, k, v, causal: bool, scale: float, samples):
    """Selected (b, h, i) rows: returns (o [n, d], lse [n])."""
    samples = [tuple(int(x) for x in t) for t in samples]
    Sq = q.shape[2]
    o = np.empty((len(samples), v.shape[3]))
    lse = np.empty(len(samples))
    by_head: dict = {}
    for t, (b, h, i) in enumerate(samples):
        by_head.setdefault((b, h), []).append(t)
    for (b, h), idx in by_head.items():
        rows = np.array([samples[t][2] for t in idx])
        o[idx], lse[idx] = attention_kv_rows(np.asarray(q[b, h][rows], dtype=np.float64), rows, Sq, k[b, h],
                                             v[b, h], causal, scale)
    return o, lse
