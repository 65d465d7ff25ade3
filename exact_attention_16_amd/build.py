"""Build libfa.so in-tree with hipcc for gfx950.

    python -m exact_attention_16_amd.build [--verbose]

Every HIP source is compiled with ``-Xclang -target-feature -Xclang
-packed-fp32-ops`` so that the compiler emits no packed-fp32 VALU instructions.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
ARCH = "gfx950"

# (source, extra flags).  The kernels are built with -fno-honor-nans: the
# softmax's fmaxf then lowers to plain v_max/v_max3 without the NaN
# canonicalisation that otherwise doubles the row-max instructions (NaN
# inputs give unspecified results).  The host front end keeps IEEE semantics
# for its argument checks (isfinite on the scale).
SOURCES = [("fa_api.cpp", []), ("fa_fwd.hip", ["-fno-honor-nans"]), ("fa_bwd.hip", ["-fno-honor-nans"]), ("fa_decode.hip", ["-fno-honor-nans"]),
           ("fa_fwd_wide.hip", ["-fno-honor-nans"])]
COMMON = ["-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every source for gfx950 (in parallel, one hipcc per source) and
    link libfa.so in-tree."""
    from concurrent.futures import ThreadPoolExecutor

    cc = hipcc()
    obj_dir = os.path.join(PKG, "_obj")
    os.makedirs(obj_dir, exist_ok=True)
    cmds, objs = [], []
    for src, flags in SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".o")
        cmds.append([cc, f"--offload-arch={ARCH}", *COMMON, *flags, "-I", INCLUDE, "-I", CSRC,
                     "-c", os.path.join(CSRC, src), "-o", obj] + list(extra or []))
        objs.append(obj)
    jobs = jobs or max(1, min(len(cmds), os.cpu_count() or 1, 8))
    with ThreadPoolExecutor(jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()  # re-raises the first failure
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
