"""Seeded random configurations through every forward entry point, against the
fp64 oracle.

Each case draws (B, H, Sq, Sk, d, causal, dtype, layout, entry point) from a
fixed seed, so the set is the same on every run: square and separate
lengths, d in {64, 128, 192, 256}, dense or [B, S, H, d] storage, and the
prefill or the split-key decoding pass (the latter for Sq <= 64).  Sizes are
small enough for the oracle to check every element.  Tolerances as for the
other forward tests: max-abs 2e-2 on O and 1e-3 on LSE; rows that see no key
must give O = 0, LSE = -inf exactly.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, say, to64

pytestmark = pytest.mark.gpu


def draw(i):
    rng = np.random.default_rng(1_000_000 + i)
    d = int(rng.choice([64, 128, 192, 256]))
    Sq = int(rng.choice([1, 2, 7, 31, 32, 33, 100, 257, 600]))
    Sk = int(rng.choice([Sq, Sq, 1, 63, 64, 65, 333, 1000]))
    return dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), Sq=Sq, Sk=Sk, d=d,
                causal=bool(rng.integers(0, 2)), dtype=str(rng.choice(["bf16", "fp16"])),
                bshd=bool(rng.integers(0, 2)), decode=bool(Sq <= 64 and rng.integers(0, 2)),
                seed=int(rng.integers(1 << 30)))


def bshd(x):
    return x.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("i", range(60))
def test_random_config(i):
    c = draw(i)
    q, k, v = make_inputs_kv(c["B"], c["H"], c["Sq"], c["Sk"], c["d"], c["dtype"], c["seed"])
    scale = default_scale(c["d"])
    say(f"random {i}: {c}")
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    if c["bshd"]:
        qd, kd, vd = bshd(qd), bshd(kd), bshd(vd)
    f = fa.decode if c["decode"] else fa.forward
    o, lse = f(qd, kd, vd, causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_kv(to64(q), to64(k), to64(v), c["causal"], scale, workers=8)
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    dead = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), dead)
    assert (o[dead] == 0).all()
    eo = float(np.abs(o - o_ref).max())
    el = float(np.abs(lse[~dead] - l_ref[~dead]).max()) if (~dead).any() else 0.0
    print(f"random {i}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE, (c, eo, el)
