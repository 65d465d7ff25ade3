"""Shared helpers of the GPU parity tests (test-side only).

The HIP path is always reached through the C ABI (``exact_attention_16_amd``'s
ctypes binding); the expected values always come from the CPU oracle.
"""

import os
import sys

import numpy as np
import torch

import exact_attention_16_amd as fa
import oracle

# Tolerances: max-abs error of O (upcast to float32) and of the logsumexp
# against the fp64 oracle, for fp16/bf16 inputs with fp32 accumulation.
TOL_O = 2e-2
TOL_LSE = 1e-3


def oracle_workers() -> int:
    """Threads for the oracle: the host cores this process may use, at most
    16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def say(msg):
    """Name the case on stdout before each GPU step (flushed)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def gpu_forward(q, k, v, causal, scale, **kw):
    qd, kd, vd = (x.cuda() for x in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale, **kw)
    torch.cuda.synchronize()
    return o, lse


def to64(x):
    return x.double().numpy()


def errors(o_gpu, lse_gpu, o_ref, lse_ref):
    eo = float(np.max(np.abs(o_gpu - o_ref))) if o_ref.size else 0.0
    el = float(np.max(np.abs(lse_gpu - lse_ref))) if lse_ref.size else 0.0
    return eo, el


def check_full(q, k, v, causal, scale, label=""):
    """Whole-tensor parity: every element of O and LSE against the oracle."""
    say(f"full {label} shape={tuple(q.shape)} dtype={q.dtype} causal={causal}")
    o, lse = gpu_forward(q, k, v, causal, scale)
    o_ref, lse_ref = oracle.attention(to64(q), to64(k), to64(v), causal, scale, workers=oracle_workers())
    eo, el = errors(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), o_ref, lse_ref)
    assert np.isfinite(eo) and np.isfinite(el), (eo, el)
    assert eo <= TOL_O, f"{label}: max |O - O_ref| = {eo}"
    assert el <= TOL_LSE, f"{label}: max |LSE - LSE_ref| = {el}"
    return eo, el
