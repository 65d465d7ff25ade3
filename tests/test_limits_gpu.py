"""GPU parity at the ends of the size range, through the C ABI.

* one head of 2^20 rows (a million-token context; per-head byte offsets of
  256 MiB, far past every tile and XCD-mapping boundary), checked on sampled
  rows against the fp64 oracle, causal and not;
* one query per head over a 2^20-key cache through both the decoding pass
  and the forward pass;
* a grid of many small ragged heads (B*H = 12300, not a multiple of the eight
  XCDs, S below one tile) checked head by head.
"""

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, say, to64

pytestmark = pytest.mark.gpu

MILLION = 1 << 20


def sampled_rows(S, rng, extra=10):
    rows = {0, 1, 31, 32, 127, 128, 255, 256, S // 2, S - 257, S - 256, S - 2, S - 1}
    rows |= set(rng.choice(S, size=extra, replace=False).tolist())
    return sorted(r for r in rows if 0 <= r < S)


@pytest.mark.parametrize("causal", [False, True])
def test_million_row_head(causal):
    S, d = MILLION, 128
    q, k, v = make_inputs_kv(1, 1, S, S, d, "bf16", seed=96_000 + causal)
    scale = default_scale(d)
    say(f"limits: one head S={S} d={d} causal={causal}")
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    rows = sampled_rows(S, np.random.default_rng(S + causal))
    samples = [(0, 0, i) for i in rows]
    so, sl = oracle.attention_samples(to64(q), to64(k), to64(v), causal, scale, samples)
    got_o = o[0, 0, rows].float().cpu().double().numpy()
    got_l = lse[0, 0, rows].cpu().double().numpy()
    eo, el = float(np.abs(got_o - so).max()), float(np.abs(got_l - sl).max())
    print(f"S={S} causal={causal}: {len(rows)} rows max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


def test_one_query_over_a_million_keys():
    B, H, Sk, d = 2, 2, MILLION, 128
    q, k, v = make_inputs_kv(B, H, 1, Sk, d, "bf16", seed=96_100)
    scale = default_scale(d)
    say(f"limits: decode Sq=1 Sk={Sk}")
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o_dec, l_dec = fa.decode(qd, kd, vd, causal=True, scale=scale)
    o_fwd, l_fwd = fa.forward(qd, kd, vd, causal=True, scale=scale)
    torch.cuda.synchronize()
    samples = [(b, h, 0) for b in range(B) for h in range(H)]
    so, sl = oracle.attention_kv_samples(to64(q), to64(k), to64(v), True, scale, samples)
    for name, o, lse in (("decode", o_dec, l_dec), ("forward", o_fwd, l_fwd)):
        got_o = o[:, :, 0].float().cpu().double().numpy().reshape(B * H, d)
        got_l = lse[:, :, 0].cpu().double().numpy().reshape(B * H)
        eo, el = float(np.abs(got_o - so).max()), float(np.abs(got_l - sl).max())
        print(f"{name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
        assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("S,d,causal", [(45, 64, True), (129, 128, False)])
def test_many_small_heads(S, d, causal):
    B, H = 300, 41
    q, k, v = make_inputs_kv(B, H, S, S, d, "fp16", seed=96_200 + S)
    scale = default_scale(d)
    say(f"limits: B={B} H={H} S={S} d={d} causal={causal}")
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all().item() and torch.isfinite(lse).all().item()
    o_cpu, l_cpu = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
    rng = np.random.default_rng(S)
    heads = [(0, 0), (B - 1, H - 1), (B // 2, 7)]
    heads += [(int(b), int(h)) for b, h in zip(rng.integers(0, B, 29), rng.integers(0, H, 29))]
    worst_o = worst_l = 0.0
    for b, h in heads:
        oh, lh = oracle.attention_head(to64(q[b, h]), to64(k[b, h]), to64(v[b, h]), causal, scale)
        worst_o = max(worst_o, float(np.abs(o_cpu[b, h] - oh).max()))
        worst_l = max(worst_l, float(np.abs(l_cpu[b, h] - lh).max()))
    print(f"{len(heads)} heads: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O and worst_l <= TOL_LSE
