"""GPU parity of the strided entry points (fa_fwd_strided, fa_fwd_decode_strided,
fa_bwd_strided) through the C ABI.

The strided kernels do the dense kernels' arithmetic in the same order, only
addressing rows through the caller's strides, so on the same values they must
give BITWISE the dense results; small cases are also compared with the fp64
oracle.  Layouts: [B, S, H, d] ("BSHD") storage viewed as [B, H, S, d], the
first Sk rows of a larger key/value cache, padded rows, mixed layouts, and an
output written into a view of a larger buffer whose other elements must stay
untouched.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, say, to64

pytestmark = pytest.mark.gpu


def bshd(x):
    """The same values stored [B, S, H, d], returned as a [B, H, S, d] view."""
    return x.transpose(1, 2).contiguous().transpose(1, 2)


def padded(x, pad=8):
    """The same values with every row padded by `pad` elements."""
    B, H, S, d = x.shape
    buf = torch.full((B, H, S, d + pad), float("nan"), dtype=x.dtype, device=x.device)
    buf[..., :d] = x
    return buf[..., :d]


def cache_slice(x, extra=37):
    """The same values as the first S rows of a [B, S + extra, H, d] cache."""
    B, H, S, d = x.shape
    cache = torch.randn(B, S + extra, H, d, device=x.device).to(x.dtype)
    cache[:, :S] = x.transpose(1, 2)
    return cache[:, :S].transpose(1, 2)


LAYOUTS = {"bshd": bshd, "padded": padded, "cache": cache_slice}


def check_oracle(o, lse, q, k, v, causal, scale, label):
    o_ref, l_ref = oracle.attention_kv(to64(q.cpu()), to64(k.cpu()), to64(v.cpu()), causal, scale, workers=8)
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    live = np.isfinite(l_ref)
    eo = float(np.max(np.abs(o - o_ref)))
    el = float(np.max(np.abs(lse[live] - l_ref[live]))) if live.any() else 0.0
    print(f"{label}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("Sq,Sk", [(300, 300), (100, 333), (333, 100), (1, 257)])
def test_forward_strided_equals_dense(Sq, Sk, layout, d, causal):
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 3, Sq, Sk, d, "bf16", seed=90_000 + Sq + 7 * Sk + d))
    scale = default_scale(d)
    label = f"strided fwd {layout} Sq={Sq} Sk={Sk} d={d} causal={causal}"
    say(label)
    o_dense, l_dense = fa.forward(q, k, v, causal=causal, scale=scale)
    f = LAYOUTS[layout]
    qs, ks, vs = f(q), f(k), f(v)
    assert not (qs.is_contiguous() and ks.is_contiguous())
    o, lse = fa.forward(qs, ks, vs, causal=causal, scale=scale)
    torch.cuda.synchronize()
    if layout == "bshd" and Sq > 1:
        assert o.stride() == qs.stride()  # a default out takes q's (dense) layout
    assert torch.equal(o, o_dense) and torch.equal(lse, l_dense), label
    check_oracle(o, lse, q, k, v, causal, scale, label)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk", [(1, 4097), (3, 1000), (40, 2500)])
def test_decode_strided_equals_dense(Sq, Sk, d, causal):
    """Decoding over the first Sk rows of a [B, S_max, H, d] cache, with q and
    o in [B, S, H, d] storage."""
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 4, Sq, Sk, d, "bf16", seed=91_000 + Sq + Sk + d))
    scale = default_scale(d)
    label = f"strided decode Sq={Sq} Sk={Sk} d={d} causal={causal}"
    say(label)
    o_dense, l_dense = fa.decode(q, k, v, causal=causal, scale=scale)
    o, lse = fa.decode(bshd(q), cache_slice(k), cache_slice(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dense) and torch.equal(lse, l_dense), label
    check_oracle(o, lse, q, k, v, causal, scale, label)


def test_output_view_leaves_the_rest_untouched():
    """o written through a [B, S, H, d] view of a buffer with an extra head and
    padded rows: only the viewed elements change."""
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 3, 200, 200, 64, "fp16", seed=92_000))
    say("strided output view")
    buf = torch.full((2, 200, 4, 72), 1234.0, dtype=torch.float16, device="cuda")
    out = buf[:, :, 1:, :64].transpose(1, 2)  # [2, 3, 200, 64] view
    o, lse = fa.forward(q, k, v, causal=True, out=out)
    o_dense, l_dense = fa.forward(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(out, o_dense) and torch.equal(lse, l_dense)
    mask = torch.ones_like(buf, dtype=torch.bool)
    mask[:, :, 1:, :64] = False
    assert (buf[mask] == 1234.0).all().item()


@pytest.mark.parametrize("S,causal", [(8192, True), (4096, False)])
def test_large_bshd_bitwise(S, causal):
    """Shapes with more query blocks than compute units (the long causal
    workload's, and a non-causal one; both run the persistent grid) in BSHD
    storage: bitwise the dense result."""
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 16, S, S, 128, "bf16", seed=93_000 + S))
    say(f"strided large bshd S={S} causal={causal}")
    o_dense, l_dense = fa.forward(q, k, v, causal=causal)
    o, lse = fa.forward(bshd(q), bshd(k), bshd(v), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_dense) and torch.equal(lse, l_dense)


def test_strided_binding_errors():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # head dimension not contiguous
        fa.forward(q.transpose(2, 3).contiguous().transpose(2, 3), q, q)
    buf = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    overlapped = buf.as_strided((1, 2, 8, 64), (1024, 0, 64, 1))  # both heads on one slab
    with pytest.raises(fa.FaError) as e:
        fa.forward(q, q, q, out=overlapped)
    assert e.value.status == fa.FA_ERR_STRIDE


def packed_qkv(q, k, v):
    """q, k, v as slices of one [B, S, 3, H, d] buffer (a fused QKV
    projection's output), each returned as a [B, H, S, d] view."""
    B, H, S, d = q.shape
    buf = torch.empty(B, S, 3, H, d, dtype=q.dtype, device=q.device)
    for i, x in enumerate((q, k, v)):
        buf[:, :, i] = x.transpose(1, 2)
    return tuple(buf[:, :, i].transpose(1, 2) for i in range(3))


def backward_inputs(B, H, S, d, dtype, seed):
    q, k, v = (x.cuda() for x in make_inputs_kv(B, H, S, S, d, dtype, seed=seed))
    g = torch.Generator().manual_seed(seed + 777_777)
    do = torch.randn(B, H, S, d, generator=g).to(q.dtype).cuda()
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", ["bshd", "padded", "packed"])
@pytest.mark.parametrize("S", [1, 200, 777])
def test_backward_strided_equals_dense(S, layout, d, causal):
    """Gradients through fa_bwd_strided are bitwise those of fa_bwd; the
    gradients allocated by the binding take q's layout."""
    q, k, v, do = backward_inputs(2, 3, S, d, "bf16", seed=94_000 + S + d)
    scale = default_scale(d)
    label = f"strided bwd {layout} S={S} d={d} causal={causal}"
    say(label)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    ref = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    if layout == "packed":
        qs, ks, vs = packed_qkv(q, k, v)
        os_, dos = bshd(o), bshd(do)
    else:
        f = LAYOUTS[layout]
        qs, ks, vs, os_, dos = f(q), f(k), f(v), f(o), f(do)
    got = fa.backward(qs, ks, vs, os_, lse, dos, causal=causal, scale=scale)
    torch.cuda.synchronize()
    if layout == "bshd" and S > 1:
        assert all(g.stride() == qs.stride() for g in got)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), f"{label}: {name} differs from the dense result"


def test_backward_strided_oracle_and_untouched():
    """Gradients written into [B, S, H, d] views of buffers with padded rows
    and an extra head: they match the fp64 oracle and leave every other
    element of the buffers untouched."""
    B, H, S, d = 1, 2, 300, 64
    q, k, v, do = backward_inputs(B, H, S, d, "fp16", seed=95_000)
    scale = default_scale(d)
    say("strided bwd gradient views")
    o, lse = fa.forward(bshd(q), bshd(k), bshd(v), causal=True, scale=scale)
    bufs = [torch.full((B, S, H + 1, d + 8), 4321.0, dtype=q.dtype, device="cuda") for _ in range(3)]
    dq, dk, dv = (b[:, :, 1:, :d].transpose(1, 2) for b in bufs)
    fa.backward(bshd(q), bshd(k), bshd(v), o, lse, bshd(do), causal=True, scale=scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    mask = torch.ones_like(bufs[0], dtype=torch.bool)
    mask[:, :, 1:, :d] = False
    for b in bufs:
        assert (b[mask] == 4321.0).all().item()
    ref = oracle.attention_backward(to64(q.cpu()), to64(k.cpu()), to64(v.cpu()), to64(do.cpu()), True, scale,
                                    workers=8)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        g = g.float().cpu().double().numpy()
        err, mag = float(np.max(np.abs(g - r))), float(np.max(np.abs(r)))
        print(f"strided bwd {name}: max|err|={err:.3e} max|ref|={mag:.3e}")
        assert err <= 2e-2 * mag + 1e-4


def test_backward_strided_binding_errors():
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 2, 8, dtype=torch.float32, device="cuda")
    buf = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16, device="cuda")
    shared = buf.as_strided((1, 2, 8, 64), (1024, 0, 64, 1))  # both heads' dk on one slab
    with pytest.raises(fa.FaError) as e:
        fa.backward(q, q, q, q, lse, q, dk=shared)
    assert e.value.status == fa.FA_ERR_STRIDE
    with pytest.raises(ValueError):  # head dimension not contiguous
        fa.backward(q.transpose(2, 3).contiguous().transpose(2, 3), q, q, q, lse, q)
    # gradients as slices of one packed buffer: their elements are disjoint but
    # their byte ranges overlap, which the library rejects
    dq, dk, dv = packed_qkv(q, q, q)
    with pytest.raises(fa.FaError) as e:
        fa.backward(q, q, q, q, lse, q, dq=dq, dk=dk, dv=dv)
    assert e.value.status == -7
