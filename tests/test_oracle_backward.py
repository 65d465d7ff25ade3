"""Pins of the gradient oracle (``oracle.gradient``) to things other than itself.

* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU, differentiated by autograd (an independent computation of the same
  gradients);
* brute force: central finite differences of L = sum(O * dO) through the
  forward oracle, on tiny inputs;
* closed forms and invariants: adding one vector to every key row changes no
  output, so the key gradients sum to zero; each softmax row sums to one, so
  the value gradients sum to the upstream gradients; with scale = 0 the
  weights are uniform over the allowed keys, dQ = dK = 0 and dV is a plain
  average; the row term D_i equals dO_i . O_i;
* the sampled-row form agrees with the whole-head form.

Every planted mistake in a step of the oracle must fail at least one pin.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.gradient as OG

CASES = [(False, 0.37), (True, 0.37), (True, 1.0)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(B=1, H=2, S=19, d=8, seed=0):
    return tuple(_rand((B, H, S, d), seed + i) for i in range(4))


def pin_torch_autograd():
    for causal, scale in CASES:
        q, k, v, do = _inputs(seed=11)
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
        o.backward(torch.tensor(do))
        dq, dk, dv = OG.attention_backward(q, k, v, do, causal, scale)
        for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def pin_finite_differences():
    for causal, scale in CASES:
        q, k, v, do = _inputs(S=5, d=3, H=1, seed=23)
        dq, dk, dv = OG.attention_backward(q, k, v, do, causal, scale)

        def loss(q_, k_, v_):
            o, _ = oracle.attention(q_, k_, v_, causal, scale)
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


def pin_key_gradients_sum_to_zero():
    for causal, scale in CASES:
        q, k, v, do = _inputs(seed=31)
        _, dk, _ = OG.attention_backward(q, k, v, do, causal, scale)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def pin_value_gradients_sum_to_upstream():
    for causal, scale in CASES:
        q, k, v, do = _inputs(seed=37)
        _, _, dv = OG.attention_backward(q, k, v, do, causal, scale)
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), rtol=1e-12, atol=1e-12)


def pin_scale_zero_closed_form():
    for causal in (False, True):
        q, k, v, do = _inputs(seed=41)
        dq, dk, dv = OG.attention_backward(q, k, v, do, causal, 0.0)
        assert np.all(dq == 0.0) and np.all(dk == 0.0)
        S = q.shape[2]
        ref = np.zeros_like(dv)
        for i in range(S):
            keys = range(i + 1) if causal else range(S)
            for j in keys:
                ref[:, :, j] += do[:, :, i] / len(keys)
        np.testing.assert_allclose(dv, ref, rtol=1e-12, atol=1e-13)


def pin_row_term_is_do_dot_o():
    for causal, scale in CASES:
        q, k, v, do = (x[0, 0] for x in _inputs(seed=43))
        p = OG._probabilities(q, k, causal, scale)
        dlt = OG._row_delta(p, OG._grad_p(do, v))
        o, _ = oracle.attention_head(q, k, v, causal, scale)
        np.testing.assert_allclose(dlt, np.sum(do * o, axis=1), rtol=1e-11, atol=1e-12)


def pin_samples_match_whole_heads():
    for causal, scale in CASES:
        q, k, v, do = _inputs(B=2, H=2, S=23, d=8, seed=47)
        dq, dk, dv = OG.attention_backward(q, k, v, do, causal, scale)
        rows = [(0, 1, 0), (1, 0, 22), (1, 1, 7), (0, 0, 11)]
        sq, sk, sv = OG.backward_samples(q, k, v, do, causal, scale, rows, rows)
        for t, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(sq[t], dq[b, h, i], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(sk[t], dk[b, h, i], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(sv[t], dv[b, h, i], rtol=1e-11, atol=1e-12)


PINS = [pin_torch_autograd, pin_finite_differences, pin_key_gradients_sum_to_zero,
        pin_value_gradients_sum_to_upstream, pin_scale_zero_closed_form, pin_row_term_is_do_dot_o,
        pin_samples_match_whole_heads]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


MUTANTS = {
    "dv_not_transposed": ("_grad_v", lambda p, do: p @ do),
    "dv_from_scores_sum": ("_grad_v", lambda p, do: p.sum(axis=0)[:, None] * do),
    "dp_transposed": ("_grad_p", lambda do, v: (do @ v.T).T),
    "delta_zero": ("_row_delta", lambda p, dp: np.zeros(p.shape[0])),
    "delta_from_dp_only": ("_row_delta", lambda p, dp: dp.sum(axis=1)),
    "ds_sign_of_delta": ("_grad_s", lambda p, dp, dl: p * (dp + dl[:, None])),
    "ds_without_p": ("_grad_s", lambda p, dp, dl: dp - dl[:, None]),
    "dq_without_scale": ("_grad_q", lambda ds, k, scale: ds @ k),
    "dq_transposed_ds": ("_grad_q", lambda ds, k, scale: scale * (ds.T @ k)),
    "dk_not_transposed": ("_grad_k", lambda ds, q, scale: scale * (ds @ q)),
    "dk_without_scale": ("_grad_k", lambda ds, q, scale: ds.T @ q),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OG, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
