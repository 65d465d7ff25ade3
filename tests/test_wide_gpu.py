"""GPU parity of wide heads (d = 192 and 256) through the C ABI against the fp64
oracle: the forward pass (square and separate lengths, dense and strided) and
the decoding pass.  Tolerances as for d = 64 / 128: max-abs 2e-2 on O, 1e-3 on
LSE.  The wide kernel runs four wavefronts of 32 query rows per work-group
(128 rows), so the lengths straddle 128-row and 64-key tiles.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, say, to64

pytestmark = pytest.mark.gpu


def compare(o, lse, o_ref, l_ref, label):
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    dead = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), dead), label
    assert (o[dead] == 0).all(), label
    live = ~dead
    eo = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    el = float(np.max(np.abs(lse[live] - l_ref[live]))) if live.any() else 0.0
    print(f"{label}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert np.isfinite(o).all() and eo <= TOL_O and el <= TOL_LSE, (label, eo, el)


def run_case(B, H, Sq, Sk, d, causal, dtype, seed, entry="forward"):
    q, k, v = make_inputs_kv(B, H, Sq, Sk, d, dtype, seed)
    scale = default_scale(d)
    label = f"wide {entry} B={B} H={H} Sq={Sq} Sk={Sk} d={d} causal={causal} {dtype}"
    say(label)
    f = fa.forward if entry == "forward" else fa.decode
    o, lse = f(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_kv(to64(q), to64(k), to64(v), causal, scale, workers=8)
    compare(o, lse, o_ref, l_ref, label)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [192, 256])
@pytest.mark.parametrize("S", [1, 17, 64, 65, 128, 129, 300, 1000])
def test_wide_square(S, d, causal):
    run_case(1, 2, S, S, d, causal, "bf16" if S % 2 == 0 else "fp16", 95_000 + S + d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [192, 256])
@pytest.mark.parametrize("Sq,Sk", [(1, 700), (100, 333), (333, 100), (129, 4000)])
def test_wide_kv(Sq, Sk, d, causal):
    run_case(2, 2, Sq, Sk, d, causal, "bf16", 96_000 + Sq + Sk + d)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [192, 256])
@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 5000), (4, 999), (40, 3000)])
def test_wide_decode(Sq, Sk, d, causal):
    run_case(2, 3, Sq, Sk, d, causal, "bf16", 97_000 + Sq + Sk + d, entry="decode")


@pytest.mark.parametrize("d", [192, 256])
def test_wide_strided_bitwise(d):
    """[B, S, H, d] storage gives bitwise the dense results (forward and decode)."""
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 3, 200, 333, d, "bf16", seed=98_000 + d))
    t = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)  # noqa: E731
    say(f"wide strided d={d}")
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.forward(t(q), t(k), t(v), causal=True)
    o3, l3 = fa.decode(q[:, :, :5], k, v, causal=True)
    o4, l4 = fa.decode(t(q[:, :, :5]), t(k), t(v), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o3, o4) and torch.equal(l3, l4)


@pytest.mark.parametrize("d,causal", [(256, True), (192, False)])
def test_wide_large_sampled(d, causal):
    B, H, S = 2, 8, 4096
    q, k, v = make_inputs_kv(B, H, S, S, d, "bf16", seed=99_000 + d)
    scale = default_scale(d)
    say(f"wide large d={d} causal={causal}")
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(d)
    rows = sorted({0, 1, 127, 128, 2047, 4095} | set(rng.choice(S, 10, replace=False).tolist()))
    samples = [(b, h, i) for b in range(B) for h in (0, H - 1) for i in rows]
    so, sl = oracle.attention_kv_samples(to64(q), to64(k), to64(v), causal, scale, samples)
    got_o = np.stack([o[b, h, i] for (b, h, i) in samples])
    got_l = np.array([lse[b, h, i] for (b, h, i) in samples])
    eo, el = float(np.abs(got_o - so).max()), float(np.abs(got_l - sl).max())
    print(f"wide large d={d}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


# ---------------------------------------------------------------- backward


def _grads_check(got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g = g.float().cpu().double().numpy()
        assert np.isfinite(g).all(), f"{label}: {name} not finite"
        err = float(np.max(np.abs(g - r))) if r.size else 0.0
        mag = float(np.max(np.abs(r))) if r.size else 0.0
        print(f"{label} {name}: max|err|={err:.3e} max|ref|={mag:.3e}")
        assert err <= 2e-2 * mag + 1e-4, f"{label}: {name} max|err| {err} > 2e-2 * {mag} + 1e-4"


def _upstream(shape, dtype, seed):
    g = torch.Generator().manual_seed(seed + 777_777)
    return torch.randn(*shape, generator=g).to(torch.float16 if dtype == "fp16" else torch.bfloat16)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [192, 256])
@pytest.mark.parametrize("Sq,Sk", [(1, 1), (65, 65), (129, 129), (300, 300), (100, 333), (333, 100)])
def test_wide_backward_against_oracle(Sq, Sk, d, causal):
    """Gradients at d = 192 / 256 (fa_bwd / fa_bwd_kv) against the fp64 oracle,
    every element."""
    dtype = "fp16" if Sq % 2 else "bf16"
    label = f"wide bwd Sq={Sq} Sk={Sk} d={d} causal={causal} {dtype}"
    say(label)
    q, k, v = make_inputs_kv(2, 2, Sq, Sk, d, dtype, seed=100_000 + Sq + 3 * Sk + d)
    do = _upstream((2, 2, Sq, d), dtype, Sq + d)
    scale = default_scale(d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    got = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_backward_kv(to64(q), to64(k), to64(v), to64(do), causal, scale, workers=8)
    _grads_check(got, ref, label)


@pytest.mark.parametrize("causal", [False, True])
def test_wide_backward_multi_tile_and_strided(causal):
    """S = 1500 at d = 256 against the oracle; the same gradients through
    [B, S, H, d] views are bitwise equal."""
    S, d = 1500, 256
    say(f"wide bwd S={S} d={d} causal={causal} (+ strided)")
    q, k, v = make_inputs_kv(1, 2, S, S, d, "bf16", seed=101_000 + causal)
    do = _upstream((1, 2, S, d), "bf16", 5)
    scale = default_scale(d)
    qd, kd, vd, dod = (x.cuda() for x in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    got = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)

    def bshd(x):
        return x.transpose(1, 2).contiguous().transpose(1, 2)

    got_s = fa.backward(bshd(qd), bshd(kd), bshd(vd), bshd(o), lse, bshd(dod), causal=causal, scale=scale)
    torch.cuda.synchronize()
    for g, gs in zip(got, got_s):
        assert torch.equal(g, gs)
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), causal, scale, workers=8)
    _grads_check(got, ref, f"wide bwd S={S}")
