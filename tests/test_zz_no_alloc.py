"""fa_fwd_decode_noalloc (the decoding pass for callers that cannot
allocate: its partial results live in the library's own scratch array)
against fa_fwd_decode with a caller workspace, on the GPU through the C ABI.

Two calls in a row, the second smaller than the first (the array keeps the
first call's contents), each bitwise equal to fa_fwd_decode (same kernels,
same key split) and within the oracle's tolerances; torch allocates nothing
during the calls; shapes beyond the array's size are rejected before any
launch."""

import gc

import numpy as np
import pytest
import torch

import exact_attention_16_amd as fa
import oracle
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import TOL_LSE, TOL_O, say

pytestmark = pytest.mark.gpu


def _compare(B, H, Sq, Sk, d, dtype, causal, seed):
    say(f"noalloc B={B} H={H} Sq={Sq} Sk={Sk} d={d} {dtype} causal={causal}")
    q, k, v = make_inputs_kv(B, H, Sq, Sk, d, dtype, seed)
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    scale = default_scale(d)
    o_ref_gpu, l_ref_gpu = fa.decode(qd, kd, vd, causal=causal, scale=scale)
    out = torch.full_like(qd, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    # nothing is allocated during the call: the peak stays at the level it
    # starts from (collected first, so that no earlier test's tensors are
    # freed meanwhile)
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    fa.decode_noalloc(qd, kd, vd, out, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
    assert torch.equal(out, o_ref_gpu) and torch.equal(lse, l_ref_gpu)
    o_ref, l_ref = oracle.attention_kv(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal, scale)
    eo = float(np.abs(out.float().cpu().double().numpy() - o_ref).max())
    el = float(np.abs(lse.cpu().double().numpy() - l_ref).max())
    print(f"noalloc: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE, (eo, el)


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    _compare(4, 8, 3, 5000, 128, "bf16", True, seed=5101)   # several key splits per head
    _compare(2, 4, 1, 777, 64, "fp16", False, seed=5102)    # smaller, ragged, one split


def test_noalloc_rejects_shapes_beyond_the_scratch():
    say("noalloc oversize")
    B, H, Sq, Sk, d = 64, 64, 64, 256, 64
    assert fa.fa_fwd_decode_workspace_size(B, H, Sq, Sk, d) > fa.FA_DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((B, H, Sq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Sk, d), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Sq), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.decode_noalloc(q, k, k, out, lse)
    assert e.value.status == fa.FA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all().item() and torch.isnan(lse).all().item()
