"""The library's launches inside a captured HIP graph, and on a non-default
stream.

A serving or training loop may capture a step into a HIP graph and replay it.
The entry points allocate nothing and record only kernel launches (no memset
or copy nodes), so a captured forward + backward + decoding step must give,
on every replay, bitwise the results of the same calls made eagerly.  Each
replay is preceded by eager work of the program's own (new inputs copied into
the captured buffers, an unrelated kernel) and followed by a synchronisation.
"""

import pytest
import torch

import exact_attention_16_amd as fa
from exact_attention_16_amd.inputs import default_scale, make_inputs_kv
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu


def _inputs(seed):
    q, k, v = make_inputs_kv(2, 4, 300, 300, 128, "bf16", seed=seed)
    g = torch.Generator().manual_seed(seed + 1)
    do = torch.randn(2, 4, 300, 128, generator=g).to(torch.bfloat16)
    qt, kc, vc = make_inputs_kv(2, 4, 1, 3000, 128, "bf16", seed=seed + 2)
    return [x.cuda() for x in (q, k, v, do, qt, kc, vc)]


def _step(bufs, outs, causal):
    q, k, v, do, qt, kc, vc = bufs
    o, lse, dq, dk, dv, delta, ot, lt, ws = outs
    scale = default_scale(128)
    fa.forward(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta)
    fa.decode(qt, kc, vc, causal=causal, scale=scale, out=ot, lse=lt, workspace=ws)


def _outs(bufs):
    q, k, v, do, qt, kc, vc = bufs
    B, H, S, d = q.shape
    n = fa.fa_fwd_decode_workspace_size(B, H, 1, kc.shape[2], d)
    return [torch.empty_like(q), torch.empty(B, H, S, device="cuda"), torch.empty_like(q), torch.empty_like(k),
            torch.empty_like(v), torch.empty(B, H, S, device="cuda"), torch.empty_like(qt),
            torch.empty(B, H, 1, device="cuda"), torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")]


@pytest.mark.parametrize("causal", [False, True])
def test_graph_replays_match_eager(causal):
    say(f"graph capture causal={causal}")
    bufs = _inputs(110_000)
    outs = _outs(bufs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        _step(bufs, outs, causal)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(bufs, outs, causal)
    torch.cuda.synchronize()
    for rep in range(3):
        new = _inputs(111_000 + rep)
        for b, n in zip(bufs, new):
            b.copy_(n)
        junk = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs[:8]]
        ref_outs = _outs(new)
        _step(new, ref_outs, causal)
        torch.cuda.synchronize()
        for i, (g, r) in enumerate(zip(got, ref_outs[:8])):
            assert torch.equal(g, r), f"replay {rep}: output {i} differs from the eager call"
        del junk


def test_backward_and_decode_on_a_side_stream():
    say("side stream backward + decode")
    bufs = _inputs(112_000)
    ref = _outs(bufs)
    _step(bufs, ref, True)
    torch.cuda.synchronize()
    outs = _outs(bufs)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _step(bufs, outs, True)
    s.synchronize()
    for i, (g, r) in enumerate(zip(outs[:8], ref[:8])):
        assert torch.equal(g, r), f"output {i} differs on a side stream"
