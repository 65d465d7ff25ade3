"""Pins of the separate-length oracle (``oracle.kv``) to things other than itself.

* a library routine: torch's scaled_dot_product_attention in float64 with
  torch's own end-aligned ("lower right") causal bias, for O, and torch's
  logsumexp over the scores masked by that same library mask, for the LSE;
* brute force: mpmath at 50 digits on tiny shapes, keys enumerated from the
  sequence positions (query i of Sq sits at position i + Sk - Sq);
* special cases of the pinned square oracle: Sq = Sk gives oracle.exact; the
  last Sq rows of a square causal attention equal Sq queries over the same
  keys; a single query sees every key with or without the causal flag;
* rows with no key (causal, Sq > Sk) give O = 0 and LSE = -inf.

Every planted mistake in a step must fail at least one pin.
"""

import mpmath
import numpy as np
import pytest
import torch
from torch.nn.attention.bias import causal_lower_right

import oracle
import oracle.kv as OK

# torch warns that its lower-right mask gives NaN rows when Sq > Sk; those rows
# are compared against the reading (O = 0, LSE = -inf) separately.
pytestmark = pytest.mark.filterwarnings("ignore:Lower right causal bias")

SHAPES = [(1, 37), (5, 37), (37, 37), (20, 11), (11, 20), (64, 200)]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _qkv(Sq, Sk, d=8, H=2, seed=0):
    return _rand((1, H, Sq, d), seed), _rand((1, H, Sk, d), seed + 1), _rand((1, H, Sk, d), seed + 2)


def pin_torch_lower_right():
    for Sq, Sk in SHAPES:
        for causal in (False, True):
            q, k, v = _qkv(Sq, Sk, seed=Sq * 100 + Sk)
            scale = 0.3
            o, lse = OK.attention_kv(q, k, v, causal, scale)
            tq, tk, tv = (torch.tensor(x) for x in (q, k, v))
            if causal:
                mask = causal_lower_right(Sq, Sk)._materialize(torch.device("cpu"))
            else:
                mask = torch.ones(Sq, Sk, dtype=torch.bool)
            live = mask.any(dim=1).numpy()
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)
            s = scale * (tq @ tk.transpose(-1, -2))
            rl = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=-1)
            np.testing.assert_allclose(o[:, :, live], ref.numpy()[:, :, live], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(lse[:, :, live], rl.numpy()[:, :, live], rtol=1e-12, atol=1e-12)


def _brute(q, k, v, causal, scale):
    Sq, Sk = len(q), len(k)
    o, lse = [], []
    with mpmath.workdps(50):
        for i in range(Sq):
            pos = i + Sk - Sq  # the query's position in the whole sequence
            keys = [j for j in range(Sk) if (not causal) or j <= pos]
            if not keys:
                o.append([0.0] * len(v[0]))
                lse.append(float("-inf"))
                continue
            w = []
            for j in keys:
                dot = mpmath.mpf(0)
                for c in range(len(q[0])):
                    dot += mpmath.mpf(float(q[i][c])) * mpmath.mpf(float(k[j][c]))
                w.append(mpmath.exp(mpmath.mpf(float(scale)) * dot))
            z = mpmath.fsum(w)
            o.append([float(mpmath.fsum(w[t] / z * mpmath.mpf(float(v[j][c])) for t, j in enumerate(keys)))
                      for c in range(len(v[0]))])
            lse.append(float(mpmath.log(z)))
    return np.array(o), np.array(lse)


def pin_bruteforce():
    for Sq, Sk in ((3, 5), (5, 3), (1, 4), (4, 4)):
        for causal in (False, True):
            q, k, v = _qkv(Sq, Sk, d=3, H=1, seed=7 * Sq + Sk)
            o, lse = OK.attention_kv(q, k, v, causal, 0.8)
            bo, bl = _brute(q[0, 0].tolist(), k[0, 0].tolist(), v[0, 0].tolist(), causal, 0.8)
            np.testing.assert_allclose(o[0, 0], bo, rtol=1e-12, atol=1e-13)
            np.testing.assert_array_equal(np.isinf(lse[0, 0]), np.isinf(bl))
            fin = np.isfinite(bl)
            np.testing.assert_allclose(lse[0, 0][fin], bl[fin], rtol=1e-12, atol=1e-13)


def pin_square_is_exact():
    for causal in (False, True):
        q, k, v = _qkv(29, 29, seed=3)
        o, lse = OK.attention_kv(q, k, v, causal, 0.4)
        ro, rl = oracle.attention(q, k, v, causal, 0.4)
        np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-13)


def pin_suffix_of_square_causal():
    S, d = 40, 8
    qf, k, v = _qkv(S, S, d=d, seed=5)
    ro, rl = oracle.attention(qf, k, v, True, 0.5)
    for Sq in (1, 7, 40):
        o, lse = OK.attention_kv(qf[:, :, S - Sq:], k, v, True, 0.5)
        np.testing.assert_allclose(o, ro[:, :, S - Sq:], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse, rl[:, :, S - Sq:], rtol=1e-12, atol=1e-13)


def pin_single_query_sees_all_keys():
    q, k, v = _qkv(1, 53, seed=9)
    a = OK.attention_kv(q, k, v, True, 0.7)
    b = OK.attention_kv(q, k, v, False, 0.7)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def pin_rows_without_keys():
    q, k, v = _qkv(9, 4, seed=11)
    o, lse = OK.attention_kv(q, k, v, True, 0.5)
    assert np.all(o[:, :, :5] == 0.0) and np.all(np.isneginf(lse[:, :, :5]))
    assert np.all(np.isfinite(lse[:, :, 5:]))


def pin_samples_match_whole():
    q, k, v = _qkv(50, 70, H=3, seed=13)
    for causal in (False, True):
        o, lse = OK.attention_kv(q, k, v, causal, 0.6)
        rows = [(0, 0, 0), (0, 2, 49), (0, 1, 17)]
        so, sl = OK.attention_kv_samples(q, k, v, causal, 0.6, rows)
        for t, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(so[t], o[b, h, i], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(sl[t], lse[b, h, i], rtol=1e-13, atol=1e-14)


PINS = [pin_torch_lower_right, pin_bruteforce, pin_square_is_exact, pin_suffix_of_square_causal,
        pin_single_query_sees_all_keys, pin_rows_without_keys, pin_samples_match_whole]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


MUTANTS = {
    "top_left_alignment": ("allowed_keys_kv", lambda rows, Sq, Sk, causal: (
        np.arange(Sk)[None, :] <= np.asarray(rows)[:, None]) if causal else np.ones((len(rows), Sk), bool)),
    "offset_off_by_one": ("allowed_keys_kv", lambda rows, Sq, Sk, causal: (
        np.arange(Sk)[None, :] < np.asarray(rows)[:, None] + (Sk - Sq)) if causal else np.ones((len(rows), Sk), bool)),
    "offset_sign": ("allowed_keys_kv", lambda rows, Sq, Sk, causal: (
        np.arange(Sk)[None, :] <= np.asarray(rows)[:, None] + (Sq - Sk)) if causal else np.ones((len(rows), Sk), bool)),
    "mask_ignored": ("allowed_keys_kv", lambda rows, Sq, Sk, causal: np.ones((len(rows), Sk), bool)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OK, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
