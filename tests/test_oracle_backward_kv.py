"""Pins of the separate-length gradient oracle (``oracle.gradient_kv``) to things
other than itself.

* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU with the end-aligned mask as an explicit boolean mask, differentiated
  by autograd (shapes where every query row keeps at least one key);
* brute force: central finite differences of L = sum(O * dO) through the
  separate-length forward oracle (``oracle.kv``, pinned on its own), on tiny
  inputs that include rows with no key;
* special case: with Sq = Sk it is the square gradient oracle;
* invariants: the key gradients sum to zero; the value gradients sum to the
  upstream gradients of the rows that keep a key; a row with no key has a
  zero dQ row and adds nothing to dK or dV.

Every planted mistake in the oracle's own step (the P of the end-aligned
mask) must fail at least one pin.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.gradient as OG
import oracle.gradient_kv as OGK

SHAPES = [(4, 9), (9, 4), (1, 7), (7, 7), (12, 5)]
CASES = [(False, 0.41), (True, 0.41), (True, 1.0)]


def _inputs(Sq, Sk, d=6, B=1, H=2, seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Sq, d))
    k = rng.standard_normal((B, H, Sk, d))
    v = rng.standard_normal((B, H, Sk, d))
    do = rng.standard_normal((B, H, Sq, d))
    return q, k, v, do


def pin_torch_autograd():
    for Sq, Sk in [(4, 9), (1, 7), (7, 7), (3, 11)]:  # Sq <= Sk: every row keeps a key
        for causal, scale in CASES:
            q, k, v, do = _inputs(Sq, Sk, seed=Sq * 31 + Sk)
            mask = torch.tensor(oracle.allowed_keys_kv(np.arange(Sq), Sq, Sk, causal))
            tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
            o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
            o.backward(torch.tensor(do))
            dq, dk, dv = OGK.attention_backward_kv(q, k, v, do, causal, scale)
            for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
                np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def pin_finite_differences():
    for Sq, Sk in [(3, 5), (5, 3), (1, 4)]:
        for causal, scale in CASES:
            q, k, v, do = _inputs(Sq, Sk, d=3, H=1, seed=7 * Sq + Sk)
            dq, dk, dv = OGK.attention_backward_kv(q, k, v, do, causal, scale)

            def loss(q_, k_, v_):
                o, _ = oracle.attention_kv(q_, k_, v_, causal, scale)
                return float(np.sum(o * do))

            h = 1e-5
            for idx, grad in ((0, dq), (1, dk), (2, dv)):
                args = [q, k, v]
                num = np.empty_like(grad)
                for pos in np.ndindex(grad.shape):
                    plus = [a.copy() for a in args]
                    minus = [a.copy() for a in args]
                    plus[idx][pos] += h
                    minus[idx][pos] -= h
                    num[pos] = (loss(*plus) - loss(*minus)) / (2 * h)
                np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def pin_square_case_is_the_square_oracle():
    for causal, scale in CASES:
        q, k, v, do = _inputs(13, 13, seed=5)
        got = OGK.attention_backward_kv(q, k, v, do, causal, scale)
        ref = OG.attention_backward(q, k, v, do, causal, scale)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, rtol=1e-12, atol=1e-13)


def pin_invariants():
    for Sq, Sk in SHAPES:
        for causal, scale in CASES:
            q, k, v, do = _inputs(Sq, Sk, seed=3 * Sq + 5 * Sk)
            dq, dk, dv = OGK.attention_backward_kv(q, k, v, do, causal, scale)
            np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
            live = oracle.allowed_keys_kv(np.arange(Sq), Sq, Sk, causal).any(axis=1)
            np.testing.assert_allclose(dv.sum(axis=2), do[:, :, live].sum(axis=2), rtol=1e-12, atol=1e-12)
            assert np.all(dq[:, :, ~live] == 0.0)


def pin_rows_without_keys_add_nothing():
    # causal, Sq > Sk: rows i < Sq - Sk keep no key; changing their q or dO
    # changes no gradient of k or v
    Sq, Sk = 9, 4
    q, k, v, do = _inputs(Sq, Sk, seed=77)
    _, dk, dv = OGK.attention_backward_kv(q, k, v, do, True, 0.5)
    q2, do2 = q.copy(), do.copy()
    q2[:, :, : Sq - Sk] *= -3.0
    do2[:, :, : Sq - Sk] += 5.0
    _, dk2, dv2 = OGK.attention_backward_kv(q2, k, v, do2, True, 0.5)
    np.testing.assert_array_equal(dk, dk2)
    np.testing.assert_array_equal(dv, dv2)


PINS = [pin_torch_autograd, pin_finite_differences, pin_square_case_is_the_square_oracle, pin_invariants,
        pin_rows_without_keys_add_nothing]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


ORIGINAL_P = OGK.probabilities_kv


def _top_left(q, k, causal, scale):
    # the mask aligned to the start instead of the end
    Sq, Sk = q.shape[0], k.shape[0]
    allowed = np.arange(Sk)[None, :] <= np.arange(Sq)[:, None] if causal else np.ones((Sq, Sk), bool)
    s = np.where(allowed, scale * q @ k.T, -np.inf)
    m = s.max(axis=1)
    return np.exp(s - (m + np.log(np.exp(s - m[:, None]).sum(axis=1)))[:, None])


def _uniform_empty_rows(q, k, causal, scale):
    # rows without a key get uniform weights instead of none
    p = ORIGINAL_P(q, k, causal, scale)
    p[p.sum(axis=1) == 0] = 1.0 / k.shape[0]
    return p


def _scale_dropped(q, k, causal, scale):
    return ORIGINAL_P(q, k, causal, 1.0)


MUTANTS = {"top_left_mask": _top_left, "uniform_empty_rows": _uniform_empty_rows, "scale_dropped": _scale_dropped}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    monkeypatch.setattr(OGK, "probabilities_kv", MUTANTS[name])
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
