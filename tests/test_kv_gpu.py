"""GPU parity of separate query and key lengths: fa_fwd_kv (through the C ABI)
against the fp64 oracle ``oracle.attention_kv``.

The causal mask is the end-aligned one (query row i sits at key position
i + Sk - Sq); rows that see no key must come back as O = 0 and LSE = -inf
exactly.  Shapes cover Sq < Sk (prefill of a chunk after a cached prefix, one
query, a few queries), Sq > Sk (rows without keys when causal), ragged lengths
around the 64-key and 256-row tiles, and Sk = 0.  Tolerances as for fa_fwd:
max-abs 2e-2 on O and 1e-3 on LSE.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, gpu_forward, say, to64

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1), (1, 17), (1, 300), (1, 4097), (5, 300), (17, 64), (64, 17), (200, 65), (65, 200),
          (300, 1000), (1000, 300), (256, 257), (257, 256), (31, 2048)]


def compare(o, lse, o_ref, lse_ref, label):
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    dead = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), dead), f"{label}: rows without keys differ"
    assert (o[dead] == 0).all(), f"{label}: a row without keys has O != 0"
    live = ~dead
    eo = float(np.max(np.abs(o[live] - o_ref[live]))) if live.any() else 0.0
    el = float(np.max(np.abs(lse[live] - lse_ref[live]))) if live.any() else 0.0
    print(f"{label}: max|dO|={eo:.3e} max|dLSE|={el:.3e} rows without keys={int(dead.sum())}")
    assert np.isfinite(o).all() and np.isfinite(lse[live]).all()
    assert eo <= TOL_O and el <= TOL_LSE, (label, eo, el)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Sq,Sk", SHAPES)
def test_kv_shapes(Sq, Sk, d, causal):
    dtype = "bf16" if (Sq + Sk + d) % 2 == 0 else "fp16"
    q, k, v = make_inputs_kv(1, 2, Sq, Sk, d, dtype, seed=70_000 + 13 * Sq + Sk + d)
    scale = default_scale(d)
    label = f"kv Sq={Sq} Sk={Sk} d={d} causal={causal} {dtype}"
    say(label)
    o, lse = gpu_forward(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention_kv(to64(q), to64(k), to64(v), causal, scale, workers=8)
    compare(o, lse, o_ref, lse_ref, label)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_square_matches_fa_fwd_bitwise(causal):
    """fa_fwd_kv with Sq = Sk is the same kernel work as fa_fwd."""
    q, k, v = (x.cuda() for x in make_inputs_kv(2, 3, 777, 777, 128, "bf16", seed=70_500 + causal))
    scale = default_scale(128)
    say(f"kv square bitwise causal={causal}")
    o1, l1 = fa.forward(q, k, v, causal=causal, scale=scale)
    o2 = torch.empty_like(q)
    l2 = torch.empty(2, 3, 777, device="cuda")
    st = fa.fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(), 2, 3, 777, 777, 128,
                      int(causal), scale, fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_no_keys(causal):
    """Sk = 0: every row has an empty key set (k and v are never read)."""
    q = make_inputs_kv(1, 2, 70, 0, 64, "bf16", seed=70_600)[0].cuda()
    o = torch.full_like(q, float("nan"))
    lse = torch.zeros(1, 2, 70, device="cuda")
    say(f"kv Sk=0 causal={causal}")
    st = fa.fa_fwd_kv(q.data_ptr(), 0, 0, o.data_ptr(), lse.data_ptr(), 1, 2, 70, 0, 64, int(causal), 0.125,
                      fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert (o.float() == 0).all().item() and torch.isneginf(lse).all().item()


def test_kv_scale_zero_rows_without_keys():
    """scale = 0 with rows that see no key: the live rows average their keys'
    values, the others stay O = 0, LSE = -inf."""
    q, k, v = make_inputs_kv(1, 2, 300, 100, 64, "bf16", seed=70_700)
    say("kv scale 0")
    o, lse = gpu_forward(q, k, v, True, 0.0)
    o_ref, lse_ref = oracle.attention_kv(to64(q), to64(k), to64(v), True, 0.0)
    compare(o, lse, o_ref, lse_ref, "kv scale 0")


@pytest.mark.parametrize("B,H,Sq,Sk,d,causal", [
    (2, 16, 2048, 8192, 128, True),   # a prompt chunk after a cached 6k prefix
    (4, 32, 512, 16384, 64, False),
    (1, 8, 8192, 1024, 128, True),    # more queries than keys: 7168 rows per head see none
    # more query blocks than compute units: the persistent grid, each block's
    # Q rows loaded during the previous block
    (2, 32, 4096, 6144, 128, False),
    (2, 32, 4096, 6144, 128, True),
])
def test_kv_large_sampled(B, H, Sq, Sk, d, causal):
    q, k, v = make_inputs_kv(B, H, Sq, Sk, d, "bf16", seed=70_800 + Sq + Sk)
    scale = default_scale(d)
    label = f"kv large B={B} H={H} Sq={Sq} Sk={Sk} d={d} causal={causal}"
    say(label)
    o, lse = gpu_forward(q, k, v, causal, scale)
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    assert np.isfinite(o).all()
    rng = np.random.default_rng(Sq + Sk)
    rows = sorted({0, 1, 255, 256, Sq // 2, Sq - 1, max(0, Sq - Sk - 1), min(Sq - 1, max(0, Sq - Sk))}
                  | set(rng.choice(Sq, size=8, replace=False).tolist()))
    samples = [(b, h, i) for b in range(B) for h in rng.choice(H, size=2, replace=False).tolist() for i in rows]
    so, sl = oracle.attention_kv_samples(to64(q), to64(k), to64(v), causal, scale, samples)
    got_o = np.stack([o[b, h, i] for (b, h, i) in samples])
    got_l = np.array([lse[b, h, i] for (b, h, i) in samples])
    compare(torch.tensor(got_o), torch.tensor(got_l), so, sl, label)
