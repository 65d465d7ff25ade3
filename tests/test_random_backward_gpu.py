"""Seeded random configurations through every backward entry point, against
the fp64 gradient oracle.

Each case draws (B, H, Sq, Sk, d, causal, dtype, layout) from a fixed seed,
so the set is the same on every run: square and separate lengths (fa_bwd,
fa_bwd_kv), d in {64, 128, 192, 256}, dense or [B, S, H, d] storage
(fa_bwd_strided).  o and lse come from the HIP forward pass on the same
inputs.  Sizes are small enough for the oracle to check every element.
Tolerance as for the other backward tests: per tensor, max |g - g_ref| <=
2e-2 max |g_ref| + 1e-4; rows that keep no key get dq = 0 exactly.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import say, to64

pytestmark = pytest.mark.gpu


def draw(i):
    rng = np.random.default_rng(2_000_000 + i)
    d = int(rng.choice([64, 128, 192, 256]))
    Sq = int(rng.choice([1, 2, 31, 32, 33, 100, 257, 500]))
    Sk = int(rng.choice([Sq, Sq, 1, 63, 64, 65, 333, 700]))
    return dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), Sq=Sq, Sk=Sk, d=d,
                causal=bool(rng.integers(0, 2)), dtype=str(rng.choice(["bf16", "fp16"])),
                bshd=bool(rng.integers(0, 2)), seed=int(rng.integers(1 << 30)))


def bshd(x):
    return x.transpose(1, 2).contiguous().transpose(1, 2)


@pytest.mark.parametrize("i", range(40))
def test_random_backward_config(i):
    c = draw(i)
    q, k, v = make_inputs_kv(c["B"], c["H"], c["Sq"], c["Sk"], c["d"], c["dtype"], c["seed"])
    g = torch.Generator().manual_seed(c["seed"] + 1)
    do = torch.randn(c["B"], c["H"], c["Sq"], c["d"], generator=g).to(q.dtype)
    scale = default_scale(c["d"])
    say(f"random backward {i}: {c}")
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    if c["bshd"]:
        qd, kd, vd, dod = bshd(qd), bshd(kd), bshd(vd), bshd(dod)
    o, lse = fa.forward(qd, kd, vd, causal=c["causal"], scale=scale)
    got = fa.backward(qd, kd, vd, o, lse, dod, causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward_kv(to64(q), to64(k), to64(v), to64(do), c["causal"], scale, workers=8)
    for name, gt, r in zip(("dq", "dk", "dv"), got, ref):
        gt = gt.float().cpu().double().numpy()
        assert np.isfinite(gt).all(), f"random backward {i}: {name} not finite"
        err = float(np.abs(gt - r).max()) if r.size else 0.0
        mag = float(np.abs(r).max()) if r.size else 0.0
        print(f"random backward {i} {name}: max|err|={err:.3e} max|ref|={mag:.3e}")
        assert err <= 2e-2 * mag + 1e-4, (i, name, err, mag)
    if c["causal"] and c["Sq"] > c["Sk"]:
        assert torch.all(got[0][:, :, : c["Sq"] - c["Sk"]] == 0).item()
