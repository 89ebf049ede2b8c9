"""Build libfa.so (the HIP library behind the C ABI in include/fa.h) for gfx950.

    python -m exact_attention_forward_fwd_amd.build

compiles csrc/*.hip with hipcc into exact_attention_forward_fwd_amd/libfa.so.
Packed fp32 VALU instructions are disabled (-packed-fp32-ops) for all device code.

fa_fwd.hip is compiled twice. As a whole it uses the compiler's maximum-ILP machine
scheduler, which measured +1.1% to +1.6% on the non-causal d = 64 tiles and up to
+1.5% on the d = 128 pipelined kernel; with FA_FWD_DEFAULT_SCHED_UNIT defined it holds
only the four-wave kernel under a causal mask and its two-wave tiles, which keep the
default scheduler (the maximum-ILP one cost them 1% to 2%). fa_bwd.hip keeps the
default scheduler as well.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
FWD = os.path.join(PKG_DIR, "csrc", "fa_fwd.hip")
BWD = os.path.join(PKG_DIR, "csrc", "fa_bwd.hip")
# (source, object name, extra flags): one object per compilation unit
UNITS = [
    (FWD, "fa_fwd.o", ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]),
    (FWD, "fa_fwd_default_sched.o", ["-DFA_FWD_DEFAULT_SCHED_UNIT"]),
    (BWD, "fa_bwd.o", []),
]
LIB_PATH = os.path.join(PKG_DIR, "libfa.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-mllvm", "--amdgpu-mfma-vgpr-form",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32-ops feature: harmless
    noise = ("packed-fp32-ops", "not a recognized feature", "warning generated", "warnings generated")
    err = "\n".join(l for l in res.stderr.splitlines() if not any(n in l for n in noise))
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stderr}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory() as objdir:
        objs = []
        jobs = []
        for src, obj, extra in UNITS:
            out = os.path.join(objdir, obj)
            objs.append(out)
            jobs.append([hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", out])
        # the units compile independently: run them side by side
        with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as pool:
            for f in [pool.submit(_run, cmd, verbose) for cmd in jobs]:
                f.result()
        _run([hipcc, f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
