"""Pins for the fp64 CPU oracle: checks against things other than itself.

Each ``pin_*`` function takes the oracle's ``attention`` entry point and raises
AssertionError when the result disagrees with what mathematics fixes:
arbitrary-precision brute force, closed forms, a library routine for a special
case, hand-derived values, and invariants of exact attention.  The meta-test at
the end plants plausible mistakes into the oracle's individual steps
(monkeypatched, on the CPU) and requires every one of them to fail some pin.

Definition pinned: exact attention, computed without approximation
(FlashAttention-2 abstract, searcharxiv abstract page "Abstract"), with the
logsumexp, causal alignment and scale readings stated in the oracle's header.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle.exact as OA
from tests._bruteforce import attention_bruteforce

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def run(q, k, v, causal, scale):
    """Call the oracle through its module attribute so monkeypatches apply."""
    return OA.attention(q, k, v, causal, scale)


def rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# --------------------------------------------------------------------- pins


def pin_bruteforce(att):
    """50-digit brute force on tiny shapes, both mask modes."""
    cases = [(1, 1), (2, 1), (3, 2), (5, 3), (8, 4), (7, 2)]
    for n, (S, d) in enumerate(cases):
        for causal in (False, True):
            q, k, v = (rand((1, 1, S, d), 100 * n + t) for t in range(3))
            v = v[..., : max(1, d - 1)] if d > 2 else v  # dv != d once
            scale = 0.37 + 0.2 * n
            o, lse = att(q, k, v, causal, scale)
            bo, bl = attention_bruteforce(q[0, 0], k[0, 0], v[0, 0], causal, scale)
            np.testing.assert_allclose(o[0, 0], np.array(bo), rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[0, 0], np.array(bl), rtol=0, atol=1e-12)


def pin_zero_query(att):
    """Q = 0: uniform weights, O_i = mean of allowed v_j, LSE_i = ln |A(i)|."""
    B, H, S, d = 2, 3, 37, 8
    k = rand((B, H, S, d), 1)
    v = rand((B, H, S, d), 2)
    q = np.zeros((B, H, S, d))
    for causal in (False, True):
        o, lse = att(q, k, v, causal, 0.5)
        if causal:
            counts = np.arange(1, S + 1)
            mean = np.cumsum(v, axis=2) / counts[:, None]
        else:
            counts = np.full(S, S)
            mean = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        np.testing.assert_allclose(o, mean, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse, np.broadcast_to(np.log(counts), lse.shape),
                                   rtol=0, atol=1e-13)


def pin_scale_zero(att):
    """scale = 0 with random Q: the same closed form as Q = 0."""
    B, H, S, d = 1, 2, 19, 4
    q, k, v = (rand((B, H, S, d), 10 + t) for t in range(3))
    o, lse = att(q, k, v, False, 0.0)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, math.log(S), rtol=0, atol=1e-13)


def pin_causal_row0(att):
    """Causal row 0 sees only key 0: O_0 = v_0 and LSE_0 = scale q_0.k_0."""
    B, H, S, d = 2, 2, 23, 16
    q, k, v = (rand((B, H, S, d), 20 + t) for t in range(3))
    scale = 0.25
    o, lse = att(q, k, v, True, scale)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], rtol=0, atol=1e-14)
    ref = scale * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], ref, rtol=0, atol=1e-13)


def pin_two_keys(att):
    """d = 1, S = 2, no mask: O_i = sigma(s_i0 - s_i1) v_0 + sigma(s_i1 - s_i0) v_1
    and LSE_i = s_i0 + ln(1 + exp(s_i1 - s_i0))."""
    q = np.array([0.7, -1.3]).reshape(1, 1, 2, 1)
    k = np.array([1.1, 2.5]).reshape(1, 1, 2, 1)
    v = np.array([-2.0, 3.0]).reshape(1, 1, 2, 1)
    scale = 0.9
    o, lse = att(q, k, v, False, scale)
    for i in range(2):
        s0 = scale * q[0, 0, i, 0] * k[0, 0, 0, 0]
        s1 = scale * q[0, 0, i, 0] * k[0, 0, 1, 0]
        sig = 1.0 / (1.0 + math.exp(s1 - s0))
        assert abs(o[0, 0, i, 0] - (sig * -2.0 + (1 - sig) * 3.0)) < 1e-14
        assert abs(lse[0, 0, i] - (s0 + math.log1p(math.exp(s1 - s0)))) < 1e-14


def pin_library(att):
    """torch's CPU flash-attention routine in float64 (O and logsumexp)."""
    for causal, S, d in ((False, 64, 16), (True, 64, 16), (True, 130, 8), (False, 9, 3)):
        q, k, v = (rand((2, 3, S, d), 30 + S + t) for t in range(3))
        scale = 1.0 / math.sqrt(d)
        o, lse = att(q, k, v, causal, scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ro, rl = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
            tq, tk, tv, 0.0, causal, attn_mask=None, scale=scale)[:2]
        np.testing.assert_allclose(o, ro.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, rl.numpy(), rtol=0, atol=1e-12)


def pin_probability_rows(att):
    """With V = identity (S = dv) the output rows are the probability rows:
    nonnegative, summing to 1, zero above the diagonal when causal."""
    S, d = 12, 5
    q, k = rand((1, 1, S, d), 40), rand((1, 1, S, d), 41)
    v = np.eye(S).reshape(1, 1, S, S)
    for causal in (False, True):
        p, _ = att(q, k, v, causal, 0.8)
        p = p[0, 0]
        assert (p >= 0).all()
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        if causal:
            assert np.all(p[np.triu_indices(S, 1)] == 0.0)
        else:
            assert (p > 0).all()


def pin_lse_bounds(att):
    """M_i <= LSE_i <= M_i + ln |A(i)|, with M_i the largest allowed score."""
    S, d = 33, 6
    q, k, v = (rand((1, 1, S, d), 50 + t, 2.0) for t in range(3))
    scale = 0.6
    for causal in (False, True):
        _, lse = att(q, k, v, causal, scale)
        s = scale * q[0, 0] @ k[0, 0].T
        if causal:
            s = np.where(np.tril(np.ones((S, S), bool)), s, -np.inf)
        m = s.max(axis=1)
        n = np.arange(1, S + 1) if causal else np.full(S, S)
        assert np.all(lse[0, 0] >= m - 1e-12)
        assert np.all(lse[0, 0] <= m + np.log(n) + 1e-12)
        # the bound is attained strictly inside for random scores
        assert np.all(lse[0, 0][1:] > m[1:])


def pin_key_shift(att):
    """Adding w to every key shifts LSE_i by scale q_i.w and leaves O unchanged."""
    S, d = 29, 8
    q, k, v = (rand((1, 2, S, d), 60 + t) for t in range(3))
    w = rand((d,), 63)
    scale = 0.45
    for causal in (False, True):
        o1, l1 = att(q, k, v, causal, scale)
        o2, l2 = att(q, k + w, v, causal, scale)
        np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l2 - l1, scale * (q @ w), rtol=0, atol=1e-12)


def pin_permutation(att):
    """Permuting Q rows permutes outputs; without a mask, permuting (K, V) rows
    jointly changes nothing."""
    S, d = 31, 4
    q, k, v = (rand((1, 1, S, d), 70 + t) for t in range(3))
    perm = np.random.default_rng(73).permutation(S)
    o, l = att(q, k, v, False, 0.7)
    o2, l2 = att(q[:, :, perm], k, v, False, 0.7)
    np.testing.assert_allclose(o2, o[:, :, perm], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l[:, :, perm], rtol=0, atol=1e-13)
    o3, l3 = att(q, k[:, :, perm], v[:, :, perm], False, 0.7)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l3, l, rtol=0, atol=1e-13)


def pin_linear_in_v(att):
    """O is linear in V; V = c gives O = c (both mask modes)."""
    S, d = 21, 6
    q, k, v1, v2 = (rand((1, 1, S, d), 80 + t) for t in range(4))
    for causal in (False, True):
        a, b = 1.7, -0.3
        o1, _ = att(q, k, v1, causal, 0.9)
        o2, _ = att(q, k, v2, causal, 0.9)
        o3, _ = att(q, k, a * v1 + b * v2, causal, 0.9)
        np.testing.assert_allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12)
        c = np.broadcast_to(np.arange(d, dtype=float), v1.shape)
        oc, _ = att(q, k, c, causal, 0.9)
        np.testing.assert_allclose(oc, c, rtol=0, atol=1e-12)


def pin_hull(att):
    """Each O_i lies in the coordinatewise range of the allowed v_j."""
    S, d = 40, 3
    q, k, v = (rand((1, 1, S, d), 90 + t, 3.0) for t in range(3))
    for causal in (False, True):
        o, _ = att(q, k, v, causal, 1.0)
        for i in range(S):
            vv = v[0, 0, : i + 1] if causal else v[0, 0]
            assert np.all(o[0, 0, i] >= vv.min(axis=0) - 1e-12)
            assert np.all(o[0, 0, i] <= vv.max(axis=0) + 1e-12)


def pin_golden_uniform(att):
    """Hand-derived fixture: uniform weights (scale = 0) on small integers."""
    with open(os.path.join(GOLDEN, "uniform_weights.json")) as f:
        g = json.load(f)
    q, k, v = (np.array(g[n], dtype=float)[None, None] for n in ("q", "k", "v"))
    for causal, key in ((False, "non_causal"), (True, "causal")):
        o, lse = att(q, k, v, causal, g["scale"])
        np.testing.assert_array_equal(o[0, 0], np.array(g[key]["o"]))
        np.testing.assert_allclose(lse[0, 0], np.log(g[key]["lse_exp"]), rtol=0, atol=1e-15)


PINS = [pin_bruteforce, pin_zero_query, pin_scale_zero, pin_causal_row0, pin_two_keys,
        pin_library, pin_probability_rows, pin_lse_bounds, pin_key_shift,
        pin_permutation, pin_linear_in_v, pin_hull, pin_golden_uniform]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(run)


def test_rows_and_samples_match_whole():
    """The row-subset and sampled entry points agree with the whole-tensor one
    (they run the same per-row definition; chunking rows changes nothing)."""
    B, H, S, d = 2, 2, 300, 8
    q, k, v = (rand((B, H, S, d), 110 + t) for t in range(3))
    for causal in (False, True):
        o, lse = OA.attention(q, k, v, causal, 0.3)
        ow, lw = OA.attention(q, k, v, causal, 0.3, workers=3)
        # BLAS may pick another summation order with one thread per worker
        np.testing.assert_allclose(ow, o, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lw, lse, rtol=0, atol=1e-13)
        samples = [(0, 0, 0), (1, 1, S - 1), (0, 1, 128), (1, 0, 77)]
        so, sl = OA.attention_samples(q, k, v, causal, 0.3, samples)
        for n, (b, h, i) in enumerate(samples):
            np.testing.assert_allclose(so[n], o[b, h, i], rtol=0, atol=1e-13)
            np.testing.assert_allclose(sl[n], lse[b, h, i], rtol=0, atol=1e-13)
    # small row blocks: force several chunks per head
    old = OA._MAX_BLOCK_ELEMS
    try:
        OA._MAX_BLOCK_ELEMS = 7 * S
        o2, l2 = OA.attention(q, k, v, True, 0.3)
    finally:
        OA._MAX_BLOCK_ELEMS = old
    o1, l1 = OA.attention(q, k, v, True, 0.3)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-14)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-14)


# ------------------------------------------------------ planted mistakes


def _sq(f):
    """Apply f only to square blocks (where a transposition type-checks)."""
    def g(a, *rest):
        return f(a, *rest) if a.shape[0] == a.shape[1] else a
    return g


MUTANTS = {
    "scores_without_scale": ("_scores", lambda q, k, scale: q @ k.T),
    "scores_scale_squared": ("_scores", lambda q, k, scale: scale * scale * (q @ k.T)),
    "scores_transposed": ("_scores", lambda q, k, scale: _sq(lambda s: s.T)(scale * (q @ k.T))),
    "mask_excludes_diagonal": ("allowed_key_mask",
                               lambda rows, S, causal: (np.arange(S)[None, :] < np.asarray(rows)[:, None])
                               if causal else np.ones((len(rows), S), bool)),
    "mask_upper_triangle": ("allowed_key_mask",
                            lambda rows, S, causal: (np.arange(S)[None, :] >= np.asarray(rows)[:, None])
                            if causal else np.ones((len(rows), S), bool)),
    "mask_one_ahead": ("allowed_key_mask",
                       lambda rows, S, causal: (np.arange(S)[None, :] <= np.asarray(rows)[:, None] + 1)
                       if causal else np.ones((len(rows), S), bool)),
    "mask_ignored": ("allowed_key_mask", lambda rows, S, causal: np.ones((len(rows), S), bool)),
    "lse_drops_max": ("_logsumexp", lambda s, m: np.log(np.exp(s - m[:, None]).sum(axis=1))),
    "lse_log2": ("_logsumexp", lambda s, m: m + np.log2(np.exp(s - m[:, None]).sum(axis=1))),
    "lse_wrong_axis": ("_logsumexp", lambda s, m: m + np.log(np.exp(s - m[:, None]).sum(axis=0))
                       if s.shape[0] == s.shape[1] else m + np.log(np.exp(s - m[:, None]).sum(axis=1)) + 1),
    "prob_sign_flipped": ("_probabilities", lambda s, lse: np.exp(lse[:, None] - s)),
    "prob_unnormalised": ("_probabilities", lambda s, lse: np.exp(s)),
    "prob_uses_max_only": ("_probabilities", lambda s, lse: np.exp(s - s.max(axis=1)[:, None])),
    "output_transposed_p": ("_output", lambda p, v: _sq(lambda x: x.T)(p) @ v),
    "output_ignores_p": ("_output", lambda p, v: np.broadcast_to(v.mean(axis=0), (p.shape[0], v.shape[1])).copy()),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(run)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
