"""CPU checks of what the pages say about tiling, against the oracle.

IPLEX blog "FlashAttention-2: making long-context attention run efficiently on
GPUs", section "Tiling preserves the attention calculation":
  * an online softmax, which carries row statistics from block to block and
    rescales the partial outputs accordingly, reproduces the exact softmax
    over the whole row;
  * a per-block softmax whose block results are simply summed computes
    something else.

Both statements are checked here with small float64 tilings written in this
test (not in the oracle and not in the HIP library): the faithful tiling agrees
with the oracle to rounding, and the counter-example -- plus the other planted
slips a kernel could make (no rescale of the partial output, the diagonal
dropped, the scale dropped) -- all miss the oracle by more than the parity
tolerance (2e-2 on O), so the parity tests would catch each of them.
"""

import math

import numpy as np
import pytest

import oracle
from exact_attention_16_amd.inputs import WORKLOADS_BY_NAME, default_scale, make_inputs

TOL_O = 2e-2


def tiled(q, k, v, causal, scale, bn, mistake=None):
    """Online-softmax tiling over key blocks of bn keys for one head."""
    S, d = q.shape
    o = np.zeros((S, v.shape[1]))
    lse = np.zeros(S)
    sc = 1.0 if mistake == "no_scale" else scale
    for i in range(S):
        m, l, acc = -np.inf, 0.0, np.zeros(v.shape[1])
        parts = []
        for j0 in range(0, S, bn):
            j = np.arange(j0, min(S, j0 + bn))
            s = sc * (k[j] @ q[i])
            if causal:
                keep = j < i if mistake == "drop_diagonal" else j <= i
                if not keep.any():
                    continue
                s, jj = s[keep], j[keep]
            else:
                jj = j
            if mistake == "normalise_blocks":
                p = np.exp(s - s.max())
                parts.append((p / p.sum()) @ v[jj])
                continue
            m_new = max(m, s.max())
            alpha = math.exp(m - m_new) if m > -np.inf else 0.0
            p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            acc = (acc if mistake == "no_rescale" else alpha * acc) + p @ v[jj]
            m = m_new
        if mistake == "normalise_blocks":
            o[i] = np.sum(parts, axis=0)
            continue
        if not np.isfinite(m):  # every key masked (only with drop_diagonal, row 0)
            o[i] = 0.0
            lse[i] = -np.inf
            continue
        o[i] = acc / l
        lse[i] = m + math.log(l)
    return o, lse


@pytest.fixture(scope="module")
def tiny():
    w = WORKLOADS_BY_NAME["tiny"]
    q, k, v = (x.double().numpy() for x in make_inputs(w))
    return q, k, v, default_scale(w.d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bn", [16, 32, 64, 128])
def test_online_softmax_tiling_is_exact(tiny, causal, bn):
    q, k, v, scale = tiny
    o, lse = oracle.attention(q, k, v, causal, scale)
    for h in range(q.shape[1]):
        to, tl = tiled(q[0, h], k[0, h], v[0, h], causal, scale, bn)
        np.testing.assert_allclose(to, o[0, h], rtol=0, atol=1e-12)
        np.testing.assert_allclose(tl, lse[0, h], rtol=0, atol=1e-12)


@pytest.mark.parametrize("mistake,causal", [
    ("normalise_blocks", False), ("normalise_blocks", True),
    ("no_rescale", False), ("no_rescale", True),
    ("drop_diagonal", True), ("no_scale", False),
])
def test_slips_exceed_the_tolerance(tiny, mistake, causal):
    q, k, v, scale = tiny
    o, _ = oracle.attention(q, k, v, causal, scale)
    err = 0.0
    for h in range(q.shape[1]):
        with np.errstate(all="ignore"):
            mo, _ = tiled(q[0, h], k[0, h], v[0, h], causal, scale, 32, mistake=mistake)
        err = max(err, float(np.nanmax(np.abs(mo - o[0, h]))))
    assert err > TOL_O, f"{mistake}: max error {err} would pass parity"
