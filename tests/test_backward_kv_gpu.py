"""GPU parity of the backward pass with separate query and key lengths
(fa_bwd_kv, and fa_bwd_strided with Sq != Sk) through the C ABI, against the
fp64 separate-length gradient oracle (``oracle.gradient_kv``).

o and lse come from the HIP forward pass (fa_fwd_kv) on the same inputs;
with causal and Sq > Sk the first Sq - Sk rows keep no key (o = 0,
LSE = -inf) and must get dq = 0 and add nothing to dk, dv.  Tolerance as in
the square backward tests: per tensor, max |g - g_ref| <= 2e-2 max |g_ref| +
1e-4.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import say, to64

pytestmark = pytest.mark.gpu

TOL_REL = 2e-2
TOL_ABS = 1e-4


def upstream(B, H, Sq, d, dtype, seed):
    g = torch.Generator().manual_seed(seed + 777_777)
    x = torch.randn(B, H, Sq, d, generator=g, dtype=torch.float32)
    return x.to(torch.float16 if dtype == "fp16" else torch.bfloat16)


def check(got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.float().cpu().double().numpy()
        assert np.isfinite(g).all(), f"{label}: {name} not finite"
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        mag = float(np.max(np.abs(r))) if r.size else 0.0
        print(f"{label} {name}: max|err|={err:.3e} max|ref|={mag:.3e}")
        assert err <= TOL_REL * mag + TOL_ABS, f"{label}: {name} max|err| {err} > {TOL_REL} * {mag} + {TOL_ABS}"


def run(B, H, Sq, Sk, d, dtype, causal, seed):
    q, k, v = make_inputs_kv(B, H, Sq, Sk, d, dtype, seed=seed)
    do = upstream(B, H, Sq, d, dtype, seed)
    scale = default_scale(d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    grads = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, do, scale), (o, lse), grads


SHAPES = [(1, 300), (17, 64), (100, 333), (333, 100), (256, 1000), (1000, 256), (65, 129), (129, 65), (300, 1)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk", SHAPES)
def test_backward_kv_against_oracle(Sq, Sk, d, causal):
    dtype = "fp16" if (Sq + Sk) % 2 else "bf16"
    label = f"bwd_kv Sq={Sq} Sk={Sk} d={d} causal={causal} {dtype}"
    say(label)
    (q, k, v, do, scale), _, grads = run(2, 2, Sq, Sk, d, dtype, causal, seed=97_000 + 3 * Sq + Sk + d)
    ref = oracle.attention_backward_kv(to64(q), to64(k), to64(v), to64(do), causal, scale, workers=8)
    check(grads, ref, label)
    if causal and Sq > Sk:
        assert torch.all(grads[0][:, :, : Sq - Sk] == 0).item()  # rows with no key


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_kv_square_equals_fa_bwd(d, causal):
    """fa_bwd_kv with Sq = Sk is bitwise fa_bwd."""
    S = 300
    say(f"bwd_kv square bitwise d={d} causal={causal}")
    (q, k, v, do, scale), (o, lse), ref = run(1, 3, S, S, d, "bf16", causal, seed=98_000 + d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    delta = torch.empty_like(lse)
    st = fa.fa_bwd_kv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(), lse.data_ptr(), dod.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), 1, 3, S, S, d,
                      1 if causal else 0, scale, fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    for g, r in zip((dq, dk, dv), ref):
        assert torch.equal(g, r)


@pytest.mark.parametrize("Sq,Sk", [(100, 333), (333, 100)])
def test_backward_kv_strided_equals_dense(Sq, Sk):
    """[B, S, H, d] storage with Sq != Sk: bitwise the dense fa_bwd_kv result."""
    say(f"bwd_kv strided Sq={Sq} Sk={Sk}")
    (q, k, v, do, scale), (o, lse), ref = run(2, 3, Sq, Sk, 128, "bf16", True, seed=99_000 + Sq)

    def bshd(x):
        return x.transpose(1, 2).contiguous().transpose(1, 2)

    qd, kd, vd, dod = (bshd(x.cuda()) for x in (q, k, v, do))
    got = fa.backward(qd, kd, vd, bshd(o), lse, dod, causal=True, scale=scale)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)


def test_backward_kv_empty_sides():
    """Sq = 0 writes dk = dv = 0; Sk = 0 writes dq = 0 and delta = 0."""
    say("bwd_kv empty sides")
    d = 64
    k = torch.randn(1, 2, 70, d, device="cuda").to(torch.bfloat16)
    q0 = torch.empty(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    lse0 = torch.empty(1, 2, 0, device="cuda")
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(k, float("nan"))
    fa.backward(q0, k, k, q0, lse0, q0, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0).item() and torch.all(dv == 0).item()

    q = torch.randn(1, 2, 70, d, device="cuda").to(torch.bfloat16)
    k0 = torch.empty(1, 2, 0, d, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.forward(q, k0, k0)
    dq = torch.full_like(q, float("nan"))
    delta = torch.full((1, 2, 70), float("nan"), device="cuda")
    fa.backward(q, k0, k0, o, lse, torch.randn_like(q), dq=dq, delta=delta)
    torch.cuda.synchronize()
    assert torch.all(o == 0).item() and torch.all(torch.isneginf(lse)).item()
    assert torch.all(dq == 0).item() and torch.all(delta == 0).item()
