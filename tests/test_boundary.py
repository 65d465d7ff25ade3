"""The C-ABI library on the CPU: it loads, exports what include/fa.h declares,
and validates arguments before any HIP call (no kernel is launched here)."""

import ctypes
import os
import re

import pytest

import exact_attention_16_amd as fa
from exact_attention_16_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.library_path()):
        from exact_attention_16_amd.build import build
        build()
    return fa.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["fa_bwd", "fa_bwd_kv", "fa_bwd_strided", "fa_fwd", "fa_fwd_decode", "fa_fwd_decode_noalloc",
                                   "fa_fwd_decode_strided",
                                   "fa_fwd_decode_workspace_size", "fa_fwd_kv", "fa_fwd_strided",
                                   "fa_last_hip_error", "fa_status_string", "fa_version"]


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(binding.library_path())
    for name in declared_functions():
        assert hasattr(raw, name), f"libfa.so does not export {name}"


def test_status_strings(lib):
    for st in range(-11, 1):
        assert fa.fa_status_string(st)
    assert fa.fa_status_string(12345) == "unknown status"
    assert fa.fa_last_hip_error() == ""
    assert fa.fa_version() >= 200


# Fake, never-dereferenced device addresses: validation only looks at their
# values.  Each buffer is 1 MiB apart so nothing overlaps unless a test wants it.
BASE = 0x7F0000000000
Q, K, V, O, L = (BASE + i * (1 << 20) for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, S=64, d=64, causal=0, scale=0.125,
            dtype=fa.FA_DTYPE_BF16)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["S"], a["d"],
                     a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(o=0), -1), (dict(lse=0), -1),
    (dict(B=-1), -2), (dict(H=-3), -2), (dict(S=-1), -2), (dict(causal=2), -2),
    (dict(d=32), -3), (dict(d=96), -3), (dict(d=320), -3), (dict(d=0), -3),
    (dict(dtype=2), -4), (dict(dtype=-1), -4),
    (dict(scale=float("nan")), -5), (dict(scale=float("inf")), -5), (dict(scale=-0.5), -5),
    (dict(q=Q + 8), -6), (dict(v=V + 2), -6), (dict(o=O + 4), -6), (dict(lse=L + 2), -6),
    (dict(o=Q), -7), (dict(o=K + 64), -7), (dict(lse=V + 1024), -7), (dict(lse=O + 4096), -7),
    (dict(S=1 << 23, d=128, q=BASE, k=BASE + (1 << 40), v=BASE + (2 << 40), o=BASE + (3 << 40),
          lse=BASE + (4 << 40)), -8),
])
def test_validation_errors(lib, kw, status):
    assert call(**kw) == status, fa.fa_status_string(status)


def test_empty_problem_is_a_no_op(lib):
    # B*H*S == 0: nothing is read or written, NULL pointers are fine
    for dims in (dict(B=0), dict(H=0), dict(S=0)):
        assert call(q=0, k=0, v=0, o=0, lse=0, **dims) == 0
    # but the remaining arguments are still checked
    assert call(S=0, d=48) == -3
    assert call(S=0, scale=-1.0) == -5


# fa_bwd: ten buffers, each 1 MiB apart
BQ_, BK_, BV_, BO_, BL_, BDO, BDQ, BDK, BDV, BDL = (BASE + (16 + i) * (1 << 20) for i in range(10))
GOOD_BWD = dict(q=BQ_, k=BK_, v=BV_, o=BO_, lse=BL_, dout=BDO, dq=BDQ, dk=BDK, dv=BDV, delta=BDL,
                B=1, H=2, S=64, d=64, causal=0, scale=0.125, dtype=fa.FA_DTYPE_BF16)


def call_bwd(**kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"], a["delta"],
                     a["B"], a["H"], a["S"], a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(o=0), -1), (dict(lse=0), -1), (dict(dout=0), -1), (dict(dq=0), -1),
    (dict(dk=0), -1), (dict(dv=0), -1), (dict(delta=0), -1),
    (dict(B=-1), -2), (dict(causal=3), -2), (dict(d=80), -3), (dict(d=320), -3), (dict(dtype=7), -4),
    (dict(scale=float("nan")), -5), (dict(scale=-1.0), -5),
    (dict(dout=BDO + 8), -6), (dict(dq=BDQ + 2), -6), (dict(delta=BDL + 2), -6), (dict(lse=BL_ + 1), -6),
    (dict(dq=BQ_), -7), (dict(dk=BO_ + 64), -7), (dict(dv=BDO + 4096), -7), (dict(delta=BL_), -7),
    (dict(dk=BDQ + 256), -7), (dict(delta=BDV + 16), -7), (dict(dq=BDL - 256), -7),
    (dict(S=1 << 23, d=128, **{n: BASE + (i << 40) for i, n in enumerate(
        ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta"))}), -8),
])
def test_backward_validation_errors(lib, kw, status):
    assert call_bwd(**kw) == status, fa.fa_status_string(status)


def test_backward_empty_problem_is_a_no_op(lib):
    for dims in (dict(B=0), dict(H=0), dict(S=0)):
        assert call_bwd(**{n: 0 for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta")},
                        **dims) == 0
    assert call_bwd(S=0, d=48) == -3


# fa_fwd_kv: q, o, lse sized by Sq; k, v by Sk
GOOD_KV = dict(GOOD, Sq=64, Sk=200)
del GOOD_KV["S"]


def call_kv(**kw):
    a = dict(GOOD_KV)
    a.update(kw)
    return fa.fa_fwd_kv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"], a["Sk"], a["d"],
                        a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(o=0), -1), (dict(lse=0), -1),
    (dict(Sq=-1), -2), (dict(Sk=-1), -2), (dict(causal=5), -2), (dict(d=96), -3), (dict(dtype=3), -4),
    (dict(scale=float("inf")), -5), (dict(k=K + 8), -6), (dict(lse=L + 1), -6),
    # k spans B*H*Sk*d*2 = 51200 bytes
    (dict(o=K + 51184), -7), (dict(lse=V + 51196), -7), (dict(o=Q + 16), -7),
    (dict(Sk=1 << 23, d=128, k=BASE + (1 << 40), v=BASE + (2 << 40)), -8),
])
def test_kv_validation_errors(lib, kw, status):
    assert call_kv(**kw) == status, fa.fa_status_string(status)


def test_kv_empty_problem_is_a_no_op(lib):
    for dims in (dict(B=0), dict(H=0), dict(Sq=0)):
        assert call_kv(q=0, k=0, v=0, o=0, lse=0, **dims) == 0
    assert call_kv(Sq=0, d=48) == -3
    assert call_kv(Sq=0, Sk=-2) == -2


# fa_fwd_decode: fa_fwd_kv's checks, then the workspace
WS = BASE + 64 * (1 << 20)


def call_dec(ws=WS, ws_bytes=1 << 20, **kw):
    a = dict(GOOD_KV)
    a.update(kw)
    return fa.fa_fwd_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"], a["Sk"], a["d"],
                            a["causal"], a["scale"], a["dtype"], ws, ws_bytes, None)


def test_decode_workspace_size_is_a_pure_function(lib):
    n = fa.fa_fwd_decode_workspace_size(1, 2, 64, 200, 64)
    assert n > 0 and n == fa.fa_fwd_decode_workspace_size(1, 2, 64, 200, 64)
    # grows with the query rows and the heads; 0 for empty or invalid shapes
    assert fa.fa_fwd_decode_workspace_size(1, 2, 128, 200, 64) > n
    assert fa.fa_fwd_decode_workspace_size(2, 2, 64, 200, 64) > n
    assert fa.fa_fwd_decode_workspace_size(1, 2, 64, 200, 256) > n  # fp32 partials grow with d
    for bad in ((0, 2, 64, 200, 64), (1, 2, 0, 200, 64), (1, 2, 64, -1, 64), (1, 2, 64, 200, 80),
                (-1, 2, 64, 200, 64)):
        assert fa.fa_fwd_decode_workspace_size(*bad) == 0
    # one query over 8192 keys, d = 128: the split count keeps it small
    assert fa.fa_fwd_decode_workspace_size(16, 16, 1, 8192, 128) < (1 << 22)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(Sk=-1), -2), (dict(d=96), -3), (dict(dtype=9), -4), (dict(scale=-1.0), -5),
    (dict(o=O + 2), -6), (dict(o=Q), -7),
    (dict(ws=0), -10), (dict(ws_bytes=16), -10), (dict(ws=WS + 8), -10),
    (dict(ws=Q + 4096), -7), (dict(ws=O - 16), -7), (dict(ws=L - 4096), -7), (dict(ws=K + 1024), -7),
])
def test_decode_validation_errors(lib, kw, status):
    assert call_dec(**kw) == status, fa.fa_status_string(status)


def test_decode_empty_problem_is_a_no_op(lib):
    for dims in (dict(B=0), dict(H=0), dict(Sq=0)):
        assert call_dec(q=0, k=0, v=0, o=0, lse=0, ws=0, ws_bytes=0, **dims) == 0


# fa_fwd_strided / fa_fwd_decode_strided: dense-equivalent strides by default
D64 = [2 * 64 * 64, 64 * 64, 64]          # q, o: B=1, H=2, Sq=64, d=64
K64 = [2 * 200 * 64, 200 * 64, 64]        # k, v: Sk=200


def call_st(strides=None, **kw):
    a = dict(GOOD_KV)
    a.update(kw)
    st = strides if strides is not None else D64 + K64 + K64 + D64
    return fa.fa_fwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"], a["Sk"], a["d"],
                             st, a["causal"], a["scale"], a["dtype"], None)


def with_stride(i, value):
    st = D64 + K64 + K64 + D64
    st[i] = value
    return st


@pytest.mark.parametrize("strides,status", [
    (with_stride(2, -64), -11), (with_stride(5, 32), -11), (with_stride(11, 0), -11),  # row stride < d
    (with_stride(0, -1), -11),
    (with_stride(1, 68), -6), (with_stride(8, 100), -6),                                 # not 16-byte rows
    (with_stride(10, 64 * 32), -11),  # o's two heads overlap (head stride < 64 rows)
    (with_stride(5, 1 << 22), -8),    # 32-bit row offsets exceeded
])
def test_strided_validation_errors(lib, strides, status):
    assert call_st(strides) == status, fa.fa_status_string(status)


def test_strided_null_and_alias(lib):
    assert fa.fa_fwd_strided(Q, K, V, O, L, 1, 2, 64, 200, 64, None, 0, 0.125, fa.FA_DTYPE_BF16, None) == -1
    # o placed inside k's strided extent (k spans 2*(200*64 + 199*64 + 64) bytes)
    assert call_st(o=K + 4096) == -7
    # a padded q row stride widens q's extent: an o right after the dense extent now overlaps
    assert call_st(strides=[2 * 64 * 72, 64 * 72, 72] + K64 + K64 + D64, o=Q + 2 * 2 * 64 * 64) == -7


def test_decode_strided_validation(lib):
    st = D64 + K64 + K64 + D64
    bad = list(st)
    bad[5] = 8
    args = (Q, K, V, O, L, 1, 2, 64, 200, 64)
    assert fa.fa_fwd_decode_strided(*args, bad, 0, 0.125, fa.FA_DTYPE_BF16, WS, 1 << 20, None) == -11
    assert fa.fa_fwd_decode_strided(*args, st, 0, 0.125, fa.FA_DTYPE_BF16, 0, 0, None) == -10
    assert fa.fa_fwd_decode_strided(*args, None, 0, 0.125, fa.FA_DTYPE_BF16, WS, 1 << 20, None) == -1


# fa_bwd_strided: dense-equivalent strides (B=1, H=2, S=64, d=64) for all eight tensors
DENSE_BWD = D64 * 8


def call_bwd_st(strides=None, **kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    st = strides if strides is not None else DENSE_BWD
    return fa.fa_bwd_strided(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                             a["delta"], a["B"], a["H"], a["S"], a["S"], a["d"], st, a["causal"], a["scale"],
                             a["dtype"], None)


def bwd_stride(i, value):
    st = list(DENSE_BWD)
    st[i] = value
    return st


def test_backward_strided_empty_problem(lib):
    assert call_bwd_st(B=0) == 0 and call_bwd_st(S=0, d=48) == -3


# Every case fails validation, so nothing is launched on these fake addresses.
@pytest.mark.parametrize("strides,kw,status", [
    (bwd_stride(2, 32), {}, -11), (bwd_stride(14, 0), {}, -11),          # row stride < d (q, dout)
    (bwd_stride(3, -8), {}, -11),                                         # negative stride (k)
    (bwd_stride(7, 68), {}, -6), (bwd_stride(23, 100), {}, -6),           # not 16-byte rows (v, dv)
    (bwd_stride(16, 64 * 32), {}, -11),   # dq's two heads overlap
    (bwd_stride(19, 0), {}, -11),         # dk's two heads written to one place
    (bwd_stride(22, 64 * 63), {}, -11),   # dv's heads interleave rows
    (bwd_stride(5, 1 << 22), {}, -8),     # 32-bit row offsets exceeded
    # o's heads may share storage (it is only read): the layout passes and the
    # later alias check is what fails
    (bwd_stride(10, 0), dict(dq=BQ_), -7),
    (None, dict(dq=BQ_), -7),
])
def test_backward_strided_validation_errors(lib, strides, kw, status):
    assert call_bwd_st(strides, **kw) == status, fa.fa_status_string(status)


def test_backward_strided_null_and_alias(lib):
    assert fa.fa_bwd_strided(BQ_, BK_, BV_, BO_, BL_, BDO, BDQ, BDK, BDV, BDL, 1, 2, 64, 64, 64, None, 0, 0.125,
                             fa.FA_DTYPE_BF16, None) == -1
    # dk 20000 bytes before dv: the dense dk (16 KiB) fits, a padded one
    # (row stride 128, 32640 bytes) reaches into dv
    dk = BDV - 20000
    padded = list(DENSE_BWD)
    padded[18:21] = [2 * 64 * 128, 64 * 128, 128]
    assert call_bwd_st(padded, dk=dk) == -7
    # dq as the first and dk as the second half of each 128-element row of one
    # buffer: disjoint elements but overlapping byte ranges, which validation
    # rejects
    inter = list(DENSE_BWD)
    inter[15:18] = [2 * 64 * 128, 64 * 128, 128]
    inter[18:21] = [2 * 64 * 128, 64 * 128, 128]
    assert call_bwd_st(inter, dk=BDQ + 128) == -7


# fa_bwd_kv: q-side tensors sized by Sq, k-side by Sk
GOOD_BWD_KV = dict(GOOD_BWD, Sq=64, Sk=200)
del GOOD_BWD_KV["S"]


def call_bwd_kv(**kw):
    a = dict(GOOD_BWD_KV)
    a.update(kw)
    return fa.fa_bwd_kv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
                        a["delta"], a["B"], a["H"], a["Sq"], a["Sk"], a["d"], a["causal"], a["scale"], a["dtype"],
                        None)


# Every case fails validation, so nothing is launched on these fake addresses.
@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(k=0), -1), (dict(dk=0), -1), (dict(delta=0), -1), (dict(lse=0), -1),
    (dict(Sq=-1), -2), (dict(Sk=-1), -2), (dict(causal=2), -2), (dict(d=96), -3), (dict(dtype=5), -4),
    (dict(scale=-1.0), -5), (dict(dk=BDK + 8), -6), (dict(delta=BDL + 2), -6),
    # dk spans 2 * 200 * 64 * 2 bytes = 50 KiB: dv 32 KiB after it overlaps
    (dict(dv=BDK + 32768), -7),
    # dq spans only 2 * 64 * 64 * 2 = 16 KiB (Sq rows): dk 20 KiB after it is fine, so the
    # next failure is the alias of dk with dv placed inside it
    (dict(dk=BDQ + 20480, dv=BDQ + 20480 + 4096), -7),
    (dict(Sk=1 << 23, d=128, **{n: BASE + (i << 40) for i, n in enumerate(
        ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta"))}), -8),
])
def test_backward_kv_validation_errors(lib, kw, status):
    assert call_bwd_kv(**kw) == status, fa.fa_status_string(status)


def test_backward_kv_empty_sides(lib):
    # B*H == 0 or Sq = Sk = 0: no-op with every pointer NULL
    nulls = {n: 0 for n in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "delta")}
    assert call_bwd_kv(B=0, **nulls) == 0
    assert call_bwd_kv(Sq=0, Sk=0, **nulls) == 0
    # Sq = 0 still writes dk and dv: those (and k, v) must be present
    assert call_bwd_kv(Sq=0, q=0, o=0, lse=0, dout=0, dq=0, delta=0, dk=0) == -1
    # Sk = 0 still writes dq and delta: those must be present
    assert call_bwd_kv(Sk=0, k=0, v=0, dk=0, dv=0, dq=0) == -1
    # a bad argument is still reported on an empty side
    assert call_bwd_kv(Sq=0, d=48) == -3


def test_grid_check_follows_the_kernel_choice(lib):
    # causal S = 129 at d = 64 runs the in-order kernel (128-row blocks: 2 per
    # head); 2^30 heads then need 2^31 work-groups, one more than a launch can
    # take.  Non-causal runs 256-row blocks (1 per head) and passes the grid
    # check, failing later on the (fake) pointers' overlap instead.
    big = dict(B=1 << 15, H=1 << 15, S=129, d=64)
    assert call(causal=1, **big) == -8
    assert call(causal=0, **big) == -7


def test_binding_rejects_host_tensors_before_any_call(monkeypatch):
    """Every tensor the kernels touch must be device memory on q's device:
    the binding raises ValueError before reaching any C entry point (a host
    pointer passed through would fault the GPU)."""
    import types

    import torch

    def no_call(*a, **k):
        raise AssertionError("the C entry point must not be reached")

    for name in ("fa_fwd", "fa_fwd_kv", "fa_fwd_strided", "fa_fwd_decode", "fa_fwd_decode_strided", "fa_bwd",
                 "fa_bwd_kv", "fa_bwd_strided"):
        monkeypatch.setattr(binding, name, no_call)
    monkeypatch.setattr(binding, "fa_fwd_decode_workspace_size", lambda *a: 1024)
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16)
    lse = torch.zeros((1, 1, 8), dtype=torch.float32)
    with pytest.raises(ValueError):
        binding.forward(q, q, q)
    with pytest.raises(ValueError):
        binding.decode(q, q, q)
    with pytest.raises(ValueError):
        binding.backward(q, q, q, q, lse, q)

    # the per-tensor check itself, with a stand-in for a device tensor
    dev = torch.device("cuda", 0)
    on_gpu = types.SimpleNamespace(is_cuda=True, device=dev)
    binding._on_device(dev, out=on_gpu, lse=on_gpu)
    for bad in (torch.zeros(4), types.SimpleNamespace(is_cuda=True, device=torch.device("cuda", 1))):
        for name in ("out", "lse", "delta", "workspace", "dq"):
            with pytest.raises(ValueError, match=name):
                binding._on_device(dev, **{name: bad})


# fa_fwd_decode_noalloc: fa_fwd_decode's validation without the workspace,
# then a size check against the library's scratch array -- all before any
# HIP call.
def call_noalloc(**kw):
    a = dict(GOOD_KV)
    a.update(kw)
    return fa.fa_fwd_decode_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Sq"], a["Sk"],
                                    a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), -1), (dict(Sk=-1), -2), (dict(d=96), -3), (dict(dtype=9), -4), (dict(scale=-1.0), -5),
    (dict(o=O + 2), -6), (dict(o=Q), -7),
])
def test_noalloc_validation_errors(lib, kw, status):
    assert call_noalloc(**kw) == status, fa.fa_status_string(status)


def test_noalloc_scratch_limit_and_empty_problem(lib):
    big = dict(B=64, H=64, Sq=64, Sk=2048, d=64)
    assert fa.fa_fwd_decode_workspace_size(64, 64, 64, 2048, 64) > fa.FA_DECODE_NOALLOC_MAX_BYTES
    far = {n: BASE + i * (1 << 32) for i, n in enumerate(("q", "k", "v", "o", "lse"))}
    assert call_noalloc(**big, **far) == fa.FA_ERR_SCRATCH
    assert "scratch" in fa.fa_status_string(fa.FA_ERR_SCRATCH)
    for dims in (dict(B=0), dict(H=0), dict(Sq=0)):
        assert call_noalloc(q=0, k=0, v=0, o=0, lse=0, **dims) == 0
