"""Attention-forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--no-per-config] [--no-parity]
                    [--no-sweep] [--no-backward] [--no-decode] [--no-wide]
                    [--decode NAMES] [--backward NAMES] [--copy-calibration]

One step is one exact-attention forward pass (every step of the method, one
kernel launch) over one batch of the workload's synthetic inputs, already
resident in device memory.  The default workload is the short-sequence batch
(B=32, H=32, S=512, d=64, bf16, no mask: 16k tokens).  All five workloads are
also timed (at least 20 launches each) and reported under "per_config", the
last key of the line: each with min / median / p90 launch times, its
roofline, and the max-abs errors of its outputs against the whole fp64 oracle,
which is timed on the host cores beside it.  The pages' benchmark grid
(S 512..16k x d 64/128 x causal, 16k tokens, bf16) under "sweep", and the
gradients (fa_bwd) of the five workloads under "backward", and the split-key
decoding pass (fa_fwd_decode) over three 1 GiB K/V caches under "decode", and
wide heads (d = 192, 256) under "wide".
Rank 0 prints ONE JSON line.

The timed region is bracketed by torch.cuda.synchronize(); the launches go on
torch's current stream and are timed with HIP events recorded on that same
stream.  The CPU baseline runs the fp64 oracle, untuned, on a bounded sample of
the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
RIDGE = PEAK_MFMA_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per byte
# The recorded HBM counters belong to one binary: its kernel sources and the
# build script that holds the compiler flags.
BUILD_SCRIPT = os.path.join(ROOT, "exact_attention_16_amd", "build.py")
KERNEL_SOURCES = [os.path.join(ROOT, "exact_attention_16_amd", "csrc", f)
                  for f in ("fa_fwd.hip", "fa_fwd_wide.hip", "fa_fwd_wave.h", "fa_device.h", "fa_launch.h")] + [BUILD_SCRIPT]
DECODE_SOURCES = [os.path.join(ROOT, "exact_attention_16_amd", "csrc", f)
                  for f in ("fa_decode.hip", "fa_fwd_wave.h", "fa_device.h", "fa_launch.h")] + [BUILD_SCRIPT]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_fa_fwd.md")
DECODE_TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "hbm_traffic_fa_decode.md")


def flops(w) -> float:
    """Attention-forward FLOPs: 4 B H S^2 d, halved for the causal mask."""
    f = 4.0 * w.B * w.H * w.S * w.S * w.d
    return f / 2 if w.causal else f


def algorithmic_bytes(w) -> int:
    """Compulsory HBM bytes: read Q, K, V; write O (2 bytes each) and the fp32 LSE."""
    n = w.B * w.H * w.S * w.d
    return 4 * n * 2 + w.B * w.H * w.S * 4


def kernel_hash(sources=None) -> str:
    """Identifies the kernel source the recorded HBM counters belong to."""
    h = hashlib.sha256()
    for path in sources or KERNEL_SOURCES:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, record: str = TRAFFIC_RECORD, sources=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    if not os.path.exists(record):
        return None
    sha = kernel_hash(sources)
    for line in open(record):
        if line.startswith("traffic-record:"):
            rec = json.loads(line.split(":", 1)[1])
            if rec.get("workload") == workload and rec.get("kernel_sha") == sha:
                return rec.get("bytes_per_launch")
    return None


def progress(msg: str) -> None:
    """One line per finished piece of work, on stderr (stdout holds only the
    JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def time_workload(w, steps: int, warmup: int, per_launch: bool = False, keep_outputs: bool = False):
    """Time `steps` forward launches of workload `w` (inputs and outputs
    resident in device memory).

    total_ms: K back-to-back launches between two events on the launch stream
    (the step time; no marker between launches).  With per_launch, a second
    sequence of K launches has an event before and after each launch
    (K + 1 events, still back to back apart from the markers): min / median /
    p90 / mean of those per-launch durations.  keep_outputs returns O (fp32)
    and LSE of the last launch as host arrays, for the parity check."""
    import torch

    import exact_attention_16_amd as fa
    from exact_attention_16_amd.inputs import default_scale, make_inputs

    q, k, v = (x.cuda() for x in make_inputs(w))
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device=q.device)
    scale = default_scale(w.d)
    stream = torch.cuda.current_stream()
    torch.cuda.reset_peak_memory_stats()
    for _ in range(warmup):
        fa.forward(q, k, v, causal=w.causal, scale=scale, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fa.forward(q, k, v, causal=w.causal, scale=scale, out=out, lse=lse, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    launch_stats = None
    if per_launch:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            fa.forward(q, k, v, causal=w.causal, scale=scale, out=out, lse=lse, stream=stream)
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
        launch_stats = {"min_ms": per[0], "median_ms": per[len(per) // 2],
                        "p90_ms": per[min(len(per) - 1, int(0.9 * len(per)))], "mean_ms": sum(per) / steps}
    ok = bool(torch.isfinite(lse).all().item())
    res = dict(total_ms=total_ms, wall_s=wall, finite=ok, launch_stats=launch_stats,
               peak_mem_mib=torch.cuda.max_memory_allocated() / 2**20)
    if keep_outputs:
        res["o"] = out.float().cpu().numpy()
        res["lse"] = lse.cpu().numpy()
    del q, k, v, out, lse
    progress(f"forward {w.name}: {total_ms / steps:.4f} ms per launch over {steps}")
    return res


def time_backward(w, steps: int, warmup: int):
    """fa_bwd on the workload: inputs, o, lse, dO and every output buffer
    resident in device memory before the timed region."""
    import torch

    import exact_attention_16_amd as fa
    from exact_attention_16_amd.inputs import default_scale, make_inputs

    q, k, v = (x.cuda() for x in make_inputs(w))
    g = torch.Generator().manual_seed(w.seed + 777_777)
    do = torch.randn(q.shape, generator=g, dtype=torch.float32).to(q.dtype).cuda()
    scale = default_scale(w.d)
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=scale)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty_like(lse)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fa.backward(q, k, v, o, lse, do, causal=w.causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta,
                    stream=stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fa.backward(q, k, v, o, lse, do, causal=w.causal, scale=scale, dq=dq, dk=dk, dv=dv, delta=delta,
                    stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    ok = all(bool(torch.isfinite(t.float()).all().item()) for t in (dq, dk, dv))
    progress(f"backward {w.name}: {start.elapsed_time(end) / steps:.4f} ms per step")
    return dict(total_ms=start.elapsed_time(end), finite=ok)


def decode_bytes(w) -> int:
    """Compulsory HBM bytes of a decoding call: read K and V (Sk rows) and Q,
    write O (2 bytes each) and the fp32 LSE."""
    return w.B * w.H * (2 * w.Sk * w.d * 2 + 2 * w.Sq * w.d * 2 + w.Sq * 4)


def time_decode(w, steps: int, warmup: int):
    """fa_fwd_decode (split pass + merge) with inputs, outputs and workspace
    resident in device memory before the timed region."""
    import torch

    import exact_attention_16_amd as fa
    from exact_attention_16_amd.inputs import default_scale

    q, k, v = (x.cuda() for x in w.inputs())
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(16, fa.fa_fwd_decode_workspace_size(w.B, w.H, w.Sq, w.Sk, w.d)), dtype=torch.uint8,
                     device=q.device)
    scale = default_scale(w.d)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fa.decode(q, k, v, causal=w.causal, scale=scale, out=out, lse=lse, workspace=ws, stream=stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fa.decode(q, k, v, causal=w.causal, scale=scale, out=out, lse=lse, workspace=ws, stream=stream)
    end.record(stream)
    torch.cuda.synchronize()
    ok = bool(torch.isfinite(lse).all().item()) and bool(torch.isfinite(out.float()).all().item())
    del q, k, v
    progress(f"decode {w.name}: {start.elapsed_time(end) / steps:.4f} ms per call")
    return dict(total_ms=start.elapsed_time(end), finite=ok, workspace_bytes=ws.numel())


def cpu_baseline(w, budget_heads: int, min_seconds: float = 10.0):
    """The fp64 oracle, as it stands, on the first `budget_heads` (b, h) heads."""
    import numpy as np

    import oracle
    from exact_attention_16_amd.inputs import default_scale, make_inputs

    q, k, v = make_inputs(w)
    n_heads = min(budget_heads, w.B * w.H)
    b_n = max(1, n_heads // w.H)
    h_n = w.H if n_heads >= w.H else n_heads
    qs, ks, vs = (x[:b_n, :h_n].double().numpy() for x in (q, k, v))
    try:
        workers = len(os.sched_getaffinity(0))
    except AttributeError:
        workers = os.cpu_count() or 1
    workers = max(1, min(workers, 16))
    runs, t0 = 0, time.perf_counter()
    while True:  # repeat the sample until about min_seconds of CPU work
        o, l = oracle.attention(qs, ks, vs, w.causal, default_scale(w.d), workers=workers)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    assert np.isfinite(o).all() and np.isfinite(l).all()
    progress(f"cpu baseline: {runs} oracle run(s) in {dt:.1f} s")
    sample = w.scaled(B=b_n, H=h_n)
    return {
        "value": runs * flops(sample) / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{b_n * h_n} of {w.B * w.H} (b, h) heads of {w.name} (S={w.S}, d={w.d}), "
                  f"fp64 numpy, {runs} run(s) in {dt:.1f} s wall",
        "seconds": dt,
    }


def copy_calibration(steps: int):
    """A plain 256 MiB device-to-device copy, for scaling the HBM counters."""
    import torch

    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    return {"copy_bytes": n, "copies": steps}


def _r(x, nd=4):
    """A float rounded to `nd` significant digits (keeps the JSON line short)."""
    if x is None:
        return None
    return float(f"{x:.{nd}g}")


def roofline(w, launch_ms: float) -> dict:
    """The roofline object of one forward workload: its bound by arithmetic
    intensity against the ridge point, the achieved rate on the algorithmic
    work per launch, and the recorded HBM traffic (null once the kernel
    source changed since the counters were taken)."""
    f, nbytes = flops(w), algorithmic_bytes(w)
    t = launch_ms * 1e-3
    if f / nbytes < RIDGE:
        achieved = nbytes / t / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    else:
        achieved = f / t / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_MFMA_TFLOPS}
    roof["traffic"] = recorded_traffic(w.name)
    return roof


def oracle_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def oracle_parity(w, o_gpu, lse_gpu) -> dict:
    """The whole fp64 oracle on the workload's inputs (timed on the host
    cores), and the max-abs errors of the GPU's O and LSE against it:
    err_o, err_lse, ok (both within 2e-2 / 1e-3), oracle_s, cores."""
    import numpy as np

    import oracle
    from exact_attention_16_amd.inputs import default_scale, make_inputs

    q, k, v = (x.double().numpy() for x in make_inputs(w))
    workers = oracle_workers()
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attention(q, k, v, w.causal, default_scale(w.d), workers=workers)
    dt = time.perf_counter() - t0
    eo = float(np.abs(o_gpu.astype(np.float64) - o_ref).max())
    el = float(np.abs(lse_gpu.astype(np.float64) - lse_ref).max())
    progress(f"oracle {w.name}: {dt:.1f} s on {workers} threads, max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    return {"err_o": eo, "err_lse": el, "ok": bool(eo <= 2e-2 and el <= 1e-3), "oracle_s": dt, "cores": workers}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="short_seq_batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the per-config oracle runs")
    ap.add_argument("--no-sweep", action="store_true", help="skip the S x d x causal grid")
    ap.add_argument("--no-backward", action="store_true", help="skip the gradient timings")
    ap.add_argument("--no-decode", action="store_true", help="skip the split-key decoding timings")
    ap.add_argument("--no-wide", action="store_true", help="skip the wide-head (d = 192, 256) timings")
    ap.add_argument("--decode", default="", help="comma-separated decoding workloads (default: all)")
    ap.add_argument("--backward", default="", help="comma-separated workloads for the gradient timings (default: all)")
    ap.add_argument("--cpu-heads", type=int, default=1024)
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library runs the attention forward of one "
              "GPU's share of (batch, head) pairs, and multi-GPU sharding is not implemented. "
              "Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_16_amd as fa
    from exact_attention_16_amd.inputs import DECODE, SWEEP, WIDE, WORKLOADS, WORKLOADS_BY_NAME

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    fa.load_library()  # fail loudly if the HIP library is missing

    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.steps)), flush=True)
        return

    # the headline workload: one of the five, or any shape of the grid or the
    # wide heads (for profiling a single kernel instantiation)
    every = {**WORKLOADS_BY_NAME, **{x.name: x for x in SWEEP + WIDE}}
    w = every[args.workload]
    torch.cuda.synchronize()
    r = time_workload(w, args.steps, args.warmup, per_launch=True)
    torch.cuda.synchronize()
    ms = r["total_ms"] / args.steps
    f = flops(w)
    value = f / (ms * 1e-3) / 1e12
    # back-to-back launches run contiguously (rocprofv3 trace), so the step
    # time is the kernel's average launch duration
    roof = roofline(w, ms)
    roof["algorithmic_bytes"] = algorithmic_bytes(w)
    roof["flops"] = f
    roof["mfma_frac"] = value / PEAK_MFMA_TFLOPS
    in_order = w.d > 128 or (w.causal and w.S <= (2048 if w.d == 64 else 512))
    roof["kernel"] = "fa::detail::fwd_wide_kernel" if in_order else "fa::detail::fwd_kernel"
    roof["launch_ms"] = ms
    roof["launch_stats"] = r["launch_stats"]

    def time_list(workloads):
        out = {}
        for wc in workloads:
            steps = max(5, min(args.steps, int(2e9 / max(1.0, flops(wc) / 1e3))))
            rc = time_workload(wc, steps, args.warmup)
            msc = rc["total_ms"] / steps
            tf = flops(wc) / (msc * 1e-3) / 1e12
            out[wc.name] = {"ms": _r(msc), "tflops": _r(tf), "pct": _r(100.0 * tf / PEAK_MFMA_TFLOPS),
                            "steps": steps, "finite": rc["finite"]}
        return out

    # Gradients of every workload (fa_bwd, two kernels per step).  FLOPs by
    # the usual count for the attention backward: 2.5x the forward (five
    # S x S x d products instead of two); the kernels recompute S and dP once
    # more, which the count does not credit.
    backward = {}
    if not args.no_backward:
        only = [n for n in args.backward.split(",") if n]
        for wc in WORKLOADS + (() if args.no_wide else WIDE):
            if only and wc.name not in only:
                continue
            steps = max(5, min(args.steps, int(2e9 / max(1.0, 2.5 * flops(wc) / 1e3))))
            rb = time_backward(wc, steps, args.warmup)
            msb = rb["total_ms"] / steps
            tf = 2.5 * flops(wc) / (msb * 1e-3) / 1e12
            backward[wc.name] = {"ms": _r(msb), "tflops": _r(tf), "pct": _r(100.0 * tf / PEAK_MFMA_TFLOPS),
                                 "steps": steps, "finite": rb["finite"]}
    # The pages' kernel-benchmark grid (S 512..16k x d 64/128 x causal, 16k
    # tokens per batch), bf16.
    sweep = {} if args.no_sweep else time_list(SWEEP)
    # Wide heads (d = 192, 256: four-wavefront work-groups), beyond the grid.
    wide = {} if args.no_wide else time_list(WIDE)
    # Token-by-token decoding (fa_fwd_decode: split pass + merge per step),
    # bound by HBM: reported against the 8 TB/s peak.
    decode = {}
    if not args.no_decode:
        names = [n for n in args.decode.split(",") if n]
        for wd in DECODE:
            if names and wd.name not in names:
                continue
            steps = max(10, args.steps)
            rd = time_decode(wd, steps, args.warmup)
            msd = rd["total_ms"] / steps
            gbs = decode_bytes(wd) / (msd * 1e-3) / 1e9
            tr = recorded_traffic(wd.name, DECODE_TRAFFIC_RECORD, DECODE_SOURCES)
            decode[wd.name] = {"ms": _r(msd), "gbs": _r(gbs), "frac_hbm": _r(gbs / PEAK_HBM_GBS),
                               "algorithmic_bytes": decode_bytes(wd), "traffic": _r(tr), "steps": steps,
                               "finite": rd["finite"]}

    # The five workloads, each: >= 20 timed back-to-back launches (their mean
    # is the step time "ms") and a second marked sequence for min / median /
    # p90; its roofline (achieved in the bound's unit: GB/s for "hbm",
    # TFLOP/s for "mfma"; traffic = recorded HBM bytes per launch); peak
    # device memory; the outputs of the timed launches against the whole
    # fp64 oracle, which is timed on the host cores (oracle_s on `cores`
    # threads; it computes every score, causal or not).  GPU timings come
    # first, the oracle runs after all of them.
    per_config = []
    if not args.no_per_config:
        outs = []
        for wc in WORKLOADS:
            steps = max(20, args.steps)
            rc = time_workload(wc, steps, args.warmup, per_launch=True, keep_outputs=not args.no_parity)
            msc = rc["total_ms"] / steps
            tf = flops(wc) / (msc * 1e-3) / 1e12
            roof_c = roofline(wc, msc)
            st = rc["launch_stats"]
            per_config.append({
                "workload": wc.name, "shape": f"B{wc.B} H{wc.H} S{wc.S} d{wc.d}", "dtype": wc.dtype,
                "causal": wc.causal, "steps": steps, "ms": _r(msc), "ms_min": _r(st["min_ms"]),
                "ms_median": _r(st["median_ms"]), "ms_p90": _r(st["p90_ms"]), "tflops": _r(tf),
                "pct_peak": _r(100.0 * tf / PEAK_MFMA_TFLOPS),
                "roofline": {"bound": roof_c["bound"], "achieved": _r(roof_c["achieved"]),
                             "frac": _r(roof_c["frac"]), "traffic": _r(roof_c["traffic"])},
                "mem_mib": _r(rc["peak_mem_mib"])})
            outs.append((rc.get("o"), rc.get("lse")))
        if not args.no_parity:
            for entry, wc, (o_gpu, lse_gpu) in zip(per_config, WORKLOADS, outs):
                par = oracle_parity(wc, o_gpu, lse_gpu)
                entry.update({k: (_r(v, 3) if isinstance(v, float) else v) for k, v in par.items()})
            del outs

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_heads)

    props = torch.cuda.get_device_properties(0)
    line = {
        "metric": "attention fwd TFLOPs/s and % of MI355X dense bf16 MFMA peak per config",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs, rounded to the dtype)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "d": w.d,
                   "causal": w.causal, "input_dtype": w.dtype, "tokens": w.B * w.S,
                   "pct_of_mfma_peak": 100.0 * value / PEAK_MFMA_TFLOPS},
        "roofline": roof,
        "cpu_baseline": cpu,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", ""), "rocm": torch.version.hip},
        "wall_s_timed_region": r["wall_s"],
        "outputs_finite": r["finite"],
        "sweep": sweep,
        "backward": backward,
        "decode": decode,
        "wide": wide,
        # last, so that a reader of the line's tail sees the five workloads
        "per_config": per_config,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
