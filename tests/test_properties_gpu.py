"""GPU properties of the HIP path that hold at any size (through the C ABI)."""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
from exact_attention_16_amd.inputs import Workload, default_scale, make_inputs
from tests.gpu_helpers import TOL_LSE, TOL_O, check_full, gpu_forward, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_row0_is_v0_bitwise(d, dtype):
    """Causal row 0 sees only key 0: its weight is exactly 1, so O_0 = v_0."""
    w = Workload("row0", 2, 3, 700, d, dtype, True, seed=31)
    q, k, v = make_inputs(w)
    say(f"row0 d={d} {dtype}")
    o, lse = gpu_forward(q, k, v, True, default_scale(d))
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])
    ref = default_scale(d) * (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1)
    assert float((lse[:, :, 0].cpu().double() - ref).abs().max()) <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_zero_query_gives_mean_of_values(d, causal):
    """Q = 0: uniform weights, O_i = mean of the allowed v_j, LSE_i = ln |A(i)|."""
    w = Workload("zeroq", 1, 2, 333, d, "bf16", causal, seed=32)
    _, k, v = make_inputs(w)
    q = torch.zeros_like(k)
    say(f"zero-q d={d} causal={causal}")
    o, lse = gpu_forward(q, k, v, causal, default_scale(d))
    vv = v.double()
    if causal:
        n = torch.arange(1, w.S + 1, dtype=torch.float64)
        mean = vv.cumsum(2) / n[:, None]
    else:
        n = torch.full((w.S,), float(w.S), dtype=torch.float64)
        mean = vv.mean(2, keepdim=True).expand_as(vv)
    assert float((o.cpu().double() - mean).abs().max()) <= TOL_O
    assert float((lse.cpu().double() - n.log()).abs().max()) <= TOL_LSE


def test_scale_zero_gives_uniform_weights():
    w = Workload("scale0", 1, 2, 200, 64, "fp16", False, seed=33)
    q, k, v = make_inputs(w)
    say("scale 0")
    o, lse = gpu_forward(q, k, v, False, 0.0)
    mean = v.double().mean(2, keepdim=True).expand(1, 2, 200, 64)
    assert float((o.cpu().double() - mean).abs().max()) <= TOL_O
    assert float((lse.cpu().double() - np.log(200)).abs().max()) <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_other_scales(causal):
    """Scale is an argument, not a constant: 0.5/sqrt(d) and 2/sqrt(d)."""
    w = Workload("scales", 1, 2, 300, 128, "bf16", causal, seed=34)
    q, k, v = make_inputs(w)
    for f in (0.5, 2.0):
        check_full(q, k, v, causal, float(np.float32(f * default_scale(128))), label=f"scale x{f}")


def test_deterministic_bitwise():
    w = Workload("det", 2, 4, 1100, 128, "bf16", True, seed=35)
    q, k, v = make_inputs(w)
    say("determinism")
    o1, l1 = gpu_forward(q, k, v, True, default_scale(128))
    o2, l2 = gpu_forward(q, k, v, True, default_scale(128))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_device_memory_allocated_and_outputs_overwritten():
    """Linear memory, no workspace: the call allocates nothing; every output
    element is written (outputs pre-filled with NaN)."""
    w = Workload("mem", 2, 2, 513, 64, "fp16", True, seed=36)
    q, k, v = (x.cuda() for x in make_inputs(w))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((2, 2, 513), float("nan"), device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    say("memory / NaN poison")
    fa.forward(q, k, v, causal=True, out=out, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.isfinite(out.float()).all().item() and torch.isfinite(lse).all().item()


def test_guard_bands_untouched():
    """Outputs placed inside larger buffers: the bytes around them stay intact
    (tail rows beyond S are dropped by the buffer range checks)."""
    B, H, S, d = 1, 3, 130, 128
    w = Workload("guard", B, H, S, d, "bf16", False, seed=37)
    q, k, v = (x.cuda() for x in make_inputs(w))
    n = B * H * S * d
    pad = 4096  # elements, 8 KiB on each side (keeps 16-byte alignment)
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((B * H * S + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    out = obuf[pad:pad + n].view(B, H, S, d)
    lse = lbuf[pad:pad + B * H * S].view(B, H, S)
    say("guard bands")
    fa.forward(q, k, v, causal=False, out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((obuf[:pad] == 7).all().item()) and bool((obuf[pad + n:] == 7).all().item())
    assert bool((lbuf[:pad] == 7).all().item()) and bool((lbuf[pad + B * H * S:] == 7).all().item())
    o_ref, l_ref = gpu_forward(q.cpu(), k.cpu(), v.cpu(), False, default_scale(d))
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)


def test_non_default_stream():
    w = Workload("stream", 1, 2, 400, 64, "bf16", True, seed=38)
    q, k, v = (x.cuda() for x in make_inputs(w))
    ref_o, ref_l = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    say("side stream")
    with torch.cuda.stream(s):
        o, l = fa.forward(q, k, v, causal=True)
    s.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_empty_problem():
    q = torch.empty((1, 2, 0, 64), dtype=torch.float16, device="cuda")
    say("empty")
    o, lse = fa.forward(q, q, q)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)


def test_binding_rejects_bad_arguments():
    q = torch.zeros((1, 1, 8, 96), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q, q)
    assert e.value.status == -3
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q, q, scale=-1.0)
    assert e.value.status == -5
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q, q, out=q)
    assert e.value.status == -7


def test_binding_rejects_host_outputs_and_scratch():
    """out, lse, delta, workspace and the gradients must be device tensors:
    host buffers are rejected before any launch."""
    say("host outputs rejected")
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, device="cuda")
    host = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    host_lse = torch.zeros((1, 1, 8), dtype=torch.float32)
    with pytest.raises(ValueError, match="out"):
        fa.forward(q, q, q, out=host)
    with pytest.raises(ValueError, match="lse"):
        fa.forward(q, q, q, lse=host_lse)
    with pytest.raises(ValueError, match="out"):
        fa.decode(q, q, q, out=host)
    with pytest.raises(ValueError, match="workspace"):
        fa.decode(q, q, q, workspace=torch.zeros(1 << 16, dtype=torch.uint8))
    o, lse = fa.forward(q, q, q)
    with pytest.raises(ValueError, match="lse"):
        fa.backward(q, q, q, o, host_lse, q)
    with pytest.raises(ValueError, match="delta"):
        fa.backward(q, q, q, o, lse, q, delta=host_lse)
    with pytest.raises(ValueError, match="dq"):
        fa.backward(q, q, q, o, lse, q, dq=host)
    torch.cuda.synchronize()
