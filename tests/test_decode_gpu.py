"""GPU parity of the split-key decoding pass: fa_fwd_decode (through the C ABI)
against the fp64 oracle ``oracle.attention_kv``.

Same operation as fa_fwd_kv (end-aligned causal mask; rows that see no key give
O = 0 and LSE = -inf), computed as per-split partial results merged by their
LSE, so the tolerances are those of the forward pass: max-abs 2e-2 on O and
1e-3 on LSE.  Cases: one to a few dozen queries over key counts around the
split and tile sizes, rows without keys, no keys at all, scale 0, the decoding
workloads at full size (sampled heads against the oracle), and the workspace
contract (size check, contents on entry irrelevant, deterministic, reusable
across shapes, no device allocation).
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import DECODE, DECODE_BY_NAME, default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, say, to64

pytestmark = pytest.mark.gpu


def compare(o, lse, o_ref, lse_ref, label):
    o = o.float().cpu().double().numpy() if torch.is_tensor(o) else o
    lse = lse.cpu().double().numpy() if torch.is_tensor(lse) else lse
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), dead), f"{label}: rows without keys differ"
    assert (o[dead] == 0).all(), f"{label}: a row without keys has O != 0"
    live = ~dead
    eo = float(np.max(np.abs(o[live] - o_ref[live]))) if live.any() else 0.0
    el = float(np.max(np.abs(lse[live] - lse_ref[live]))) if live.any() else 0.0
    print(f"{label}: max|dO|={eo:.3e} max|dLSE|={el:.3e} rows without keys={int(dead.sum())}")
    assert np.isfinite(o).all() and np.isfinite(lse[live]).all()
    assert eo <= TOL_O and el <= TOL_LSE, (label, eo, el)


def run(q, k, v, causal, scale, **kw):
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    o, lse = fa.decode(qd, kd, vd, causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 17), (1, 128), (1, 129), (1, 1000), (1, 4097), (1, 20000),
                                   (2, 513), (5, 300), (31, 2048), (32, 32), (33, 700), (64, 5000), (40, 17)])
def test_decode_shapes(Sq, Sk, d, causal):
    dtype = "bf16" if (Sq + Sk) % 2 == 0 else "fp16"
    q, k, v = make_inputs_kv(2, 3, Sq, Sk, d, dtype, seed=80_000 + 17 * Sq + Sk + d)
    scale = default_scale(d)
    label = f"decode Sq={Sq} Sk={Sk} d={d} causal={causal} {dtype}"
    say(label)
    o, lse = run(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention_kv(to64(q), to64(k), to64(v), causal, scale, workers=8)
    compare(o, lse, o_ref, lse_ref, label)


def test_decode_no_keys():
    q = make_inputs_kv(1, 2, 3, 0, 128, "bf16", seed=80_500)[0].cuda()
    o = torch.full_like(q, float("nan"))
    lse = torch.zeros(1, 2, 3, device="cuda")
    need = fa.fa_fwd_decode_workspace_size(1, 2, 3, 0, 128)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    say("decode Sk=0")
    st = fa.fa_fwd_decode(q.data_ptr(), 0, 0, o.data_ptr(), lse.data_ptr(), 1, 2, 3, 0, 128, 1, 0.1,
                          fa.FA_DTYPE_BF16, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert (o.float() == 0).all().item() and torch.isneginf(lse).all().item()


def test_decode_one_row_no_keys():
    """S_q = 1 (the register-staged kernel) with S_k = 0: O = 0, LSE = -inf."""
    q = make_inputs_kv(2, 3, 1, 0, 64, "fp16", seed=80_550)[0].cuda()
    o = torch.full_like(q, float("nan"))
    lse = torch.zeros(2, 3, 1, device="cuda")
    need = fa.fa_fwd_decode_workspace_size(2, 3, 1, 0, 64)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    say("decode Sq=1 Sk=0")
    st = fa.fa_fwd_decode(q.data_ptr(), 0, 0, o.data_ptr(), lse.data_ptr(), 2, 3, 1, 0, 64, 0, 0.125,
                          fa.FA_DTYPE_FP16, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert (o.float() == 0).all().item() and torch.isneginf(lse).all().item()


@pytest.mark.parametrize("d", [64, 128])
def test_decode_rising_scores(d):
    """S_q = 1 with scores that climb by about 200 (natural units) along the
    keys, past what fp32 exponentials hold, so every stream moves its
    reference max many times and the splits' LSEs differ widely."""
    q, k, v = make_inputs_kv(2, 4, 1, 6000, d, "bf16", seed=80_650 + d)
    qf = q.float()
    ramp = torch.linspace(0.0, 1.0, 6000).view(1, 1, 6000, 1)
    scale = default_scale(d)
    # score_j = scale * q.k_j ~ 200 * j / Sk (natural units) on top of the noise
    k = (k.float() + ramp * qf * (200.0 / (scale * (qf * qf).sum(-1, keepdim=True)))).to(torch.bfloat16)
    say(f"decode rising d={d}")
    o, lse = run(q, k, v, False, scale)
    o_ref, lse_ref = oracle.attention_kv(to64(q), to64(k), to64(v), False, scale, workers=8)
    compare(o, lse, o_ref, lse_ref, f"decode rising d={d}")


def test_decode_scale_zero():
    q, k, v = make_inputs_kv(1, 2, 4, 3000, 64, "bf16", seed=80_600)
    say("decode scale 0")
    o, lse = run(q, k, v, True, 0.0)
    o_ref, lse_ref = oracle.attention_kv(to64(q), to64(k), to64(v), True, 0.0)
    compare(o, lse, o_ref, lse_ref, "decode scale 0")


def test_decode_peaky_keys():
    """One key per head dominates (scaled by 8): the merge must weight the
    split that holds it by its LSE."""
    q, k, v = make_inputs_kv(2, 4, 1, 9000, 128, "bf16", seed=80_700)
    k = k.float()
    for h in range(4):
        k[:, h, 1234 + 1000 * h] = 8.0 * q[:, h, 0].float()
    k = k.to(torch.bfloat16)
    scale = default_scale(128)
    say("decode peaky")
    o, lse = run(q, k, v, True, scale)
    o_ref, lse_ref = oracle.attention_kv(to64(q), to64(k), to64(v), True, scale)
    compare(o, lse, o_ref, lse_ref, "decode peaky")


@pytest.mark.parametrize("name", [w.name for w in DECODE])
def test_decode_workload_sampled(name):
    """Each decoding workload at full size, in the launch the benchmark times:
    every output finite; two heads of every fourth sequence against the
    oracle."""
    w = DECODE_BY_NAME[name]
    q, k, v = w.inputs()
    scale = default_scale(w.d)
    say(f"decode workload {name}")
    o, lse = run(q, k, v, w.causal, scale)
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rng = np.random.default_rng(w.seed)
    samples = [(b, h, i) for b in range(0, w.B, 4) for h in rng.choice(w.H, size=2, replace=False).tolist()
               for i in range(w.Sq)]
    so, sl = oracle.attention_kv_samples(to64(q), to64(k), to64(v), w.causal, scale, samples)
    got_o = np.stack([o[b, h, i] for (b, h, i) in samples])
    got_l = np.array([lse[b, h, i] for (b, h, i) in samples])
    compare(got_o, got_l, so, sl, name)


def test_decode_matches_forward_kv():
    """fa_fwd_decode and fa_fwd_kv agree to rounding on the same inputs."""
    q, k, v = (x.cuda() for x in make_inputs_kv(3, 5, 7, 3333, 128, "bf16", seed=80_800))
    say("decode vs fa_fwd_kv")
    o1, l1 = fa.forward(q, k, v, causal=True)
    o2, l2 = fa.decode(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2 * TOL_O
    assert (l1 - l2).abs().max().item() <= 2 * TOL_LSE


def test_decode_workspace_contract():
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 4, 3, 5000, 64, "bf16", seed=80_900))
    need = fa.fa_fwd_decode_workspace_size(2, 4, 3, 5000, 64)
    assert need > 0
    say("decode workspace contract")
    ws = torch.full((need,), 255, dtype=torch.uint8, device="cuda")  # NaN bit patterns
    o = torch.empty_like(q)
    lse = torch.empty(2, 4, 3, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    fa.decode(q, k, v, causal=False, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    first = (o.clone(), lse.clone())
    # reuse the same workspace for another shape in between
    q2, k2, v2 = (x.cuda() for x in make_inputs_kv(1, 2, 1, 700, 64, "bf16", seed=80_901))
    fa.decode(q2, k2, v2, workspace=ws)
    fa.decode(q, k, v, causal=False, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(first[0], o) and torch.equal(first[1], lse)
    with pytest.raises(fa.FaError) as e:
        fa.decode(q, k, v, workspace=ws[: need - 16])
    assert e.value.status == fa.FA_ERR_WORKSPACE
