"""Plain fp64 CPU oracle for the exact-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, constants or
helpers with the HIP library under ``exact_attention_16_amd/``.

What it computes, and why it is the plain definition rather than a tiling:

* FlashAttention-2 abstract (searcharxiv abstract page, "Abstract"): the method
  computes attention exactly, without approximating it; the standard
  algorithm's runtime and memory grow quadratically in the sequence length.
* IPLEX blog "FlashAttention-2: making long-context attention run efficiently
  on GPUs", section "Tiling preserves the attention calculation": tiling with an
  online softmax is an exact-attention algorithm; it differs from the plain
  calculation only by floating-point rounding, so results are compared with
  tolerances.

Hence the oracle is the definition written out, per (batch b, head h), per
query row i, in float64 on the float64 upcast of the (already dtype-rounded)
inputs:

    A(i)  = {0 .. S-1}             (no mask)
          = {0 .. i}               (causal: key j kept iff j <= i)
    s_ij  = scale * sum_c q_ic k_jc          for j in A(i)
    M_i   = max_{j in A(i)} s_ij
    LSE_i = M_i + ln( sum_{j in A(i)} exp(s_ij - M_i) )        (natural log)
    P_ij  = exp(s_ij - LSE_i)  for j in A(i),  0 otherwise
    O_i   = sum_j P_ij v_j

Readings where the pages are silent (each is listed with its reason in the
design notes): the logsumexp output and its natural-log base, the causal
alignment "key j <= query i" (query and key lengths are equal), and the scale
as an explicit argument that multiplies the scores before the max and the exp.

Rows are independent in the definition, so computing them in groups of rows
(to bound the materialised score block) and computing heads in parallel threads
changes no arithmetic.  Each step below is its own small function so that a
test can replace exactly one step with a planted mistake and show that the
oracle's pins catch it.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

__all__ = [
    "attention",
    "attention_head",
    "attention_rows",
    "attention_samples",
    "allowed_key_mask",
]

# Largest score block materialised at once, in elements (float64): 32 MiB.
_MAX_BLOCK_ELEMS = 1 << 22


def allowed_key_mask(rows: np.ndarray, S: int, causal: bool) -> np.ndarray:
    """Boolean [len(rows), S]: True where key j is in A(i) for query row i.

    Causal reading: query and key sequences have the same length, so the
    lower-triangular mask keeps key j for query i iff j <= i (the diagonal is
    kept).
    """
    keys = np.arange(S)[None, :]
    if causal:
        return keys <= np.asarray(rows)[:, None]
    return np.ones((len(rows), S), dtype=bool)


def _scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """s_ij = scale * <q_i, k_j> for the given query rows and all keys."""
    return scale * (q_rows @ k.T)


def _apply_mask(s: np.ndarray, allowed: np.ndarray) -> np.ndarray:
    """Keys outside A(i) get score -inf, i.e. probability exactly 0."""
    return np.where(allowed, s, -np.inf)


def _row_max(s: np.ndarray) -> np.ndarray:
    """M_i = max over the allowed keys."""
    return s.max(axis=1)


def _logsumexp(s: np.ndarray, m: np.ndarray) -> np.ndarray:
    """LSE_i = M_i + ln sum_j exp(s_ij - M_i)."""
    return m + np.log(np.exp(s - m[:, None]).sum(axis=1))


def _probabilities(s: np.ndarray, lse: np.ndarray) -> np.ndarray:
    """P_ij = exp(s_ij - LSE_i); masked keys have s = -inf, so P = 0."""
    return np.exp(s - lse[:, None])


def _output(p: np.ndarray, v: np.ndarray) -> np.ndarray:
    """O_i = sum_j P_ij v_j."""
    return p @ v


def attention_rows(q_rows, row_ids, k, v, causal: bool, scale: float):
    """Outputs for selected query rows of one head.

    q_rows: [n, d] the query vectors of rows ``row_ids`` (positions in the
    sequence), k, v: [S, d] the whole head.  Returns (o [n, d], lse [n]) in
    float64.
    """
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    row_ids = np.asarray(row_ids, dtype=np.int64)
    S = k.shape[0]
    s = _scores(q_rows, k, float(scale))
    s = _apply_mask(s, allowed_key_mask(row_ids, S, causal))
    m = _row_max(s)
    lse = _logsumexp(s, m)
    p = _probabilities(s, lse)
    return _output(p, v), lse


def attention_head(q, k, v, causal: bool, scale: float):
    """All rows of one head: q, k, v [S, d] -> (o [S, d], lse [S])."""
    q = np.asarray(q, dtype=np.float64)
    S, d = q.shape
    o = np.empty((S, v.shape[1]), dtype=np.float64)
    lse = np.empty(S, dtype=np.float64)
    step = max(1, _MAX_BLOCK_ELEMS // max(1, S))
    for r0 in range(0, S, step):
        rows = np.arange(r0, min(S, r0 + step))
        o[rows], lse[rows] = attention_rows(q[rows], rows, k, v, causal, scale)
    return o, lse


def attention(q, k, v, causal: bool, scale: float, workers: int = 1):
    """Whole tensors: q, k, v [B, H, S, d] -> (o [B, H, S, d], lse [B, H, S]).

    ``workers`` > 1 computes independent heads in a thread pool (numpy releases
    the GIL in matmul and exp); BLAS is then held to one thread per worker so
    the pool does not oversubscribe the cores.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, d = q.shape
    o = np.empty((B, H, S, v.shape[3]), dtype=np.float64)
    lse = np.empty((B, H, S), dtype=np.float64)

    def one(bh):
        b, h = divmod(bh, H)
        o[b, h], lse[b, h] = attention_head(q[b, h], k[b, h], v[b, h], causal, scale)

    if workers <= 1:
        for bh in range(B * H):
            one(bh)
    else:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(one, range(B * H)))
    return o, lse


def attention_samples(q, k, v, causal: bool, scale: float, samples):
    """Selected outputs of whole tensors, one (b, h, i) triple at a time.

    ``samples``: iterable of (b, h, i).  Returns (o [n, d], lse [n]).  Used to
    check outputs of full-size workloads where the whole oracle would be slow.
    """
    samples = [tuple(int(x) for x in t) for t in samples]
    n = len(samples)
    d_v = v.shape[3]
    o = np.empty((n, d_v), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    # group by head so each head's K and V are upcast once
    by_head: dict[tuple[int, int], list[int]] = {}
    for idx, (b, h, i) in enumerate(samples):
        by_head.setdefault((b, h), []).append(idx)
    for (b, h), idxs in by_head.items():
        rows = np.array([samples[t][2] for t in idxs], dtype=np.int64)
        oh, lh = attention_rows(
            np.asarray(q[b, h][rows], dtype=np.float64), rows,
            np.asarray(k[b, h], dtype=np.float64),
            np.asarray(v[b, h], dtype=np.float64), causal, scale)
        o[idxs] = oh
        lse[idxs] = lh
    return o, lse


if __name__ == "__main__":  # tiny self-demo, no I/O beyond stdout
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((1, 1, 4, 2)) for _ in range(3))
    o, lse = attention(q, k, v, causal=True, scale=1 / math.sqrt(2))
    print(o[0, 0], lse[0, 0])
