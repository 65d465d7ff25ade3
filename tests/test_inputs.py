"""The seeded input generator: determinism, recipe and rounding."""

import numpy as np
import torch

from exact_attention_16_amd.inputs import (WORKLOADS, WORKLOADS_BY_NAME, default_scale,
                                           make_inputs, peaky_rows)


def test_five_workloads_as_described():
    shapes = [(w.B, w.H, w.S, w.d, w.dtype, w.causal) for w in WORKLOADS]
    assert shapes == [
        (1, 2, 128, 64, "fp16", False),
        (32, 32, 512, 64, "bf16", False),
        (8, 16, 2048, 128, "bf16", True),
        (2, 16, 8192, 128, "bf16", True),
        (1, 32, 16384, 64, "fp16", False),
    ]
    # 16k tokens per batch for every benchmark-sized workload
    assert all(w.B * w.S == 16384 for w in WORKLOADS[1:])


def test_same_seed_same_bytes():
    w = WORKLOADS_BY_NAME["tiny"]
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.float16 and x.is_contiguous()
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    c = make_inputs(w, seed=w.seed + 1)
    assert not torch.equal(a[0], c[0])


def test_scale_is_fp32_inverse_sqrt():
    assert default_scale(64) == 0.125
    assert default_scale(128) == float(np.float32(1 / np.sqrt(128)))
    assert np.float32(default_scale(128)) == default_scale(128)


def test_peaky_rows_recipe():
    w = WORKLOADS_BY_NAME["long_seq_causal"].scaled(B=1, H=3, S=1000)
    g = torch.Generator().manual_seed(7)
    rows = peaky_rows(w, g)
    assert rows.shape == (1, 3, 10)
    for h in range(3):
        assert len(set(rows[0, h].tolist())) == 10
    # the full workload scales exactly 82 rows per head by 8
    full = WORKLOADS_BY_NAME["long_seq_causal"]
    assert int(round(full.peaky_frac * full.S)) == 82
    small = full.scaled(B=1, H=2, S=512)  # 5 rows per head at this length
    q, k, v = make_inputs(small)
    g = torch.Generator().manual_seed(small.seed)
    shape = (1, 2, 512, small.d)
    torch.randn(shape, generator=g)            # Q
    k32 = torch.randn(shape, generator=g)      # K before scaling
    torch.randn(shape, generator=g)            # V
    picks = peaky_rows(small, g)
    for h in range(2):
        ratio = k[0, h].float().abs().amax(dim=1) / k32[0, h].to(torch.bfloat16).float().abs().amax(dim=1)
        assert torch.all(ratio[picks[0, h]] == 8.0)
        others = torch.ones(512, dtype=torch.bool)
        others[picks[0, h]] = False
        assert torch.all(ratio[others] == 1.0)


def _rne_bits(x32: np.ndarray, mant_drop: int) -> np.ndarray:
    """Round-to-nearest-even of float32 bit patterns by dropping mantissa bits
    (bf16: 16 bits); returns the rounded float32 values."""
    u = x32.view(np.uint32).astype(np.uint64)
    half = np.uint64(1 << (mant_drop - 1))
    lsb = (u >> np.uint64(mant_drop)) & np.uint64(1)
    r = (u + half - np.uint64(1) + lsb) >> np.uint64(mant_drop) << np.uint64(mant_drop)
    return r.astype(np.uint32).view(np.float32)


def test_bf16_cast_is_round_to_nearest_even():
    x = torch.randn(1_000_000, generator=torch.Generator().manual_seed(3)) * 4
    x[:4] = torch.tensor([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 1.0 + 2**-9])
    got = x.to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got, _rne_bits(x.numpy().copy(), 16))


def test_fp16_cast_is_round_to_nearest_even():
    x = torch.randn(1_000_000, generator=torch.Generator().manual_seed(4)) * 4
    got = x.to(torch.float16).numpy()
    np.testing.assert_array_equal(got, x.numpy().astype(np.float16))


def test_separate_length_inputs():
    from exact_attention_16_amd.inputs import make_inputs_kv

    q, k, v = make_inputs_kv(2, 3, 5, 17, 64, "bf16", seed=7)
    assert q.shape == (2, 3, 5, 64) and k.shape == v.shape == (2, 3, 17, 64)
    assert q.dtype == k.dtype == v.dtype == torch.bfloat16
    # the same recipe as make_inputs: draws in the order Q, K, V
    g = torch.Generator().manual_seed(7)
    rq = torch.randn((2, 3, 5, 64), generator=g).to(torch.bfloat16)
    rk = torch.randn((2, 3, 17, 64), generator=g).to(torch.bfloat16)
    assert torch.equal(q, rq) and torch.equal(k, rk)
    q2, _, _ = make_inputs_kv(2, 3, 5, 17, 64, "bf16", seed=7)
    assert torch.equal(q, q2)


def test_decoding_and_wide_workloads():
    from exact_attention_16_amd.inputs import DECODE, WIDE

    for w in DECODE:
        assert w.Sq == 1 and w.causal and w.dtype == "bf16"
        assert w.H * w.d == 2048                              # the grid's model width
        assert w.B * w.H * w.Sk * w.d * 2 * 2 == 1 << 30      # 1 GiB of K and V
    for w in WIDE:
        assert w.d in (192, 256) and w.B * w.S == 16384
