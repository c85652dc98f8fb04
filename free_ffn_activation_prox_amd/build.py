"""Build the Prox HIP library (libprox_hip.so) in-tree for gfx950.

    python -m free_ffn_activation_prox_amd.build

Compiles every .hip source under csrc/ (in parallel) and links one shared library with hipcc.
Packed-fp32 instructions are disabled for all device code.
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
LIB = os.path.join(PKG, "libprox_hip.so")
ARCH = os.environ.get("PROX_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _flags(debug: bool):
    return [
        f"--offload-arch={ARCH}", "-std=c++17", "-fPIC",
        "-O1" if debug else "-O3",
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    if verbose and r.stderr.strip():
        # the host pass warns about the gfx-only target feature; keep other output visible
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            print("\n".join(lines))


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every csrc/*.hip to an object (in parallel), then link them."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(f)[:-4] + ".o") for f in srcs]
    jobs = [[cc] + _flags(debug) + ["-c", src, "-o", obj] for src, obj in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    out_tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", out_tmp] + objs, verbose)
    os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
