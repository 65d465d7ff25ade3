"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

* small and medium shapes, compared element by element, spanning several
  key and query tiles and ragged tails (S not a multiple of any tile size);
* the five benchmark workloads and the 24 shapes of the pages' benchmark grid
  at full size, in the same launch the benchmark times: every output checked
  for finiteness and the value-hull property, and every element of O and LSE
  against the oracle;
* d = 64 causal problems long enough for the ping-pong kernel, in full.
"""

import pytest
import torch

import oracle
from exact_attention_16_amd.inputs import (SWEEP, SWEEP_BY_NAME, WORKLOADS, WORKLOADS_BY_NAME,
                                           Workload, default_scale, make_inputs)
from tests.gpu_helpers import TOL_LSE, TOL_O, check_full, errors, gpu_forward, oracle_workers, say, to64

pytestmark = pytest.mark.gpu

SEQ = [1, 2, 17, 63, 64, 65, 127, 128, 129, 255, 300, 1000]


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("S", SEQ)
def test_edge_lengths(S, d, causal, dtype):
    w = Workload("edge", 1, 2, S, d, dtype, causal, seed=10_000 + S * 7 + d + causal)
    q, k, v = make_inputs(w)
    check_full(q, k, v, causal, default_scale(d), label=f"edge S={S}")


@pytest.mark.parametrize("B,H,S,d,dtype,causal", [
    (2, 3, 777, 128, "bf16", True),
    (3, 2, 1029, 64, "fp16", False),
    (1, 4, 2048, 128, "fp16", True),
    (2, 2, 1536, 64, "bf16", True),
    (1, 1, 4099, 128, "bf16", False),
])
def test_multi_tile_ragged(B, H, S, d, dtype, causal):
    w = Workload("ragged", B, H, S, d, dtype, causal, seed=20_000 + S)
    q, k, v = make_inputs(w)
    check_full(q, k, v, causal, default_scale(d), label="ragged")


def test_peaky_keys_medium():
    """The long-sequence recipe (1 % of key rows x8) at a size the oracle
    finishes in full."""
    w = WORKLOADS_BY_NAME["long_seq_causal"].scaled(B=1, H=3, S=1500)
    q, k, v = make_inputs(w)
    check_full(q, k, v, True, default_scale(w.d), label="peaky")


def _level_inputs(shape, S, d, dtype, seed):
    """q, k, v whose scores follow a chosen level L_j (in binary orders of
    magnitude, c * s) along the key axis, plus noise of about one order.

    q rows are 1 + 0.25 N(0,1) and key row j is t_j + 0.5 N(0,1) with
    t_j = L_j / (log2(e) sqrt(d)), so with the default scale c * s_ij is about
    L_j.  "rising" climbs 40 orders per 64 keys, "valley" falls by that much
    and climbs back, "cliff" jumps by 300 orders (2^300 overflows fp32) at key
    500.  Inputs are rounded to the dtype before anything sees them.
    """
    g = torch.Generator().manual_seed(seed)
    j = torch.arange(S, dtype=torch.float64)
    if shape == "rising":
        level = 40.0 * torch.floor(j / 64)
    elif shape == "valley":
        level = 40.0 * torch.abs(torch.floor(j / 64) - 7)
    else:
        level = torch.where(j < 500, 0.0, 300.0)
    t = level / (1.4426950408889634 * d ** 0.5)
    q = 1.0 + 0.25 * torch.randn(1, 2, S, d, generator=g, dtype=torch.float64)
    k = t[None, None, :, None] + 0.5 * torch.randn(1, 2, S, d, generator=g, dtype=torch.float64)
    v = torch.randn(1, 2, S, d, generator=g, dtype=torch.float64)
    tdt = torch.float16 if dtype == "fp16" else torch.bfloat16
    return tuple(x.to(tdt) for x in (q, k, v))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", ["rising", "valley", "cliff"])
def test_moving_row_max(shape, d, causal, dtype):
    """Row maxima that move by tens to hundreds of binary orders of magnitude
    from tile to tile: the online softmax must move its reference max and
    rescale the partial output many times (weights past the fp16 and bf16
    bounds, and past fp32's range) and still match the oracle."""
    S = 1000
    q, k, v = _level_inputs(shape, S, d, dtype, seed=30_000 + 10 * d + causal)
    check_full(q, k, v, causal, default_scale(d), label=f"level {shape}")


def _compare_whole(w, label):
    """Every element of O and LSE of workload ``w``, from the launch the
    benchmark times, against the oracle on the same inputs."""
    scale = default_scale(w.d)
    q, k, v = make_inputs(w)
    say(f"{label} {w.name} B={w.B} H={w.H} S={w.S} d={w.d} {w.dtype} causal={w.causal}")
    o, lse = gpu_forward(q, k, v, w.causal, scale)

    # properties over every output: finite; each O_i inside the per-head
    # coordinatewise range of V (exact attention averages value rows; P is
    # rounded to the input dtype before the PV product and O to the dtype on
    # output, hence the margin)
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    vd = v.cuda().float()
    lo = vd.amin(dim=2, keepdim=True)
    hi = vd.amax(dim=2, keepdim=True)
    of = o.float()
    margin = 0.05
    assert bool(((of >= lo - margin) & (of <= hi + margin)).all().item())
    del vd, lo, hi, of

    o_cpu = o.float().cpu().double().numpy()
    lse_cpu = lse.cpu().double().numpy()
    del o, lse
    o_ref, lse_ref = oracle.attention(to64(q), to64(k), to64(v), w.causal, scale, workers=oracle_workers())
    eo, el = errors(o_cpu, lse_cpu, o_ref, lse_ref)
    print(f"{w.name}: all {o_cpu.size} O and {lse_cpu.size} LSE elements max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE, (w.name, eo, el)


@pytest.mark.parametrize("name", [w.name for w in WORKLOADS])
def test_full_size_workload(name):
    """The five benchmark workloads at full size, every output element."""
    _compare_whole(WORKLOADS_BY_NAME[name], "workload")


@pytest.mark.parametrize("name", [w.name for w in SWEEP])
def test_sweep_full(name):
    """The pages' kernel-benchmark grid (S 512..16k x d 64/128 x causal, 16k
    tokens per batch), in the launch the benchmark times, every output
    element.  The grid reaches every forward instantiation at bf16: the
    ping-pong kernel at d = 64 / 128 with and without the causal mask, and the
    in-order kernel that short causal problems use."""
    _compare_whole(SWEEP_BY_NAME[name], "sweep")


@pytest.mark.parametrize("B,H,S,dtype", [(1, 2, 4096, "bf16"), (1, 2, 4096, "fp16"), (1, 1, 8192, "fp16"),
                                         (2, 1, 6144, "bf16")])
def test_causal_d64_long(B, H, S, dtype):
    """d = 64 causal problems longer than 2048 keys run the ping-pong kernel
    (shorter ones the in-order kernel); every element against the oracle."""
    w = Workload("causal_d64_long", B, H, S, 64, dtype, True, seed=40_000 + S + B)
    _compare_whole(w, "causal d64")
