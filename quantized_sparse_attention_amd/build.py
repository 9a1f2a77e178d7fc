"""Build libqsa.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m quantized_sparse_attention_amd.build

Compiles every csrc/*.hip to an object (in parallel) and links them into
quantized_sparse_attention_amd/libqsa.so; the benchmark's MFMA-rate probe
(probe/*.hip) goes into a library of its own, libqsa_probe.so.  Always
recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libqsa.so")
PROBE_DIR = os.path.join(PKG, "probe")
PROBE_LIB = os.path.join(PKG, "libqsa_probe.so")
OBJ_DIR = os.path.join(PKG, "_build")

ARCH = "gfx950"

# Numerics flags: IEEE fp32 division (the quantiser's codes depend on it),
# fp32 denormals kept, no fast-math; contraction only where a file allows it.
# Packed-fp32 instructions are disabled for the device.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=fast-honor-pragmas",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libqsa.so)")


def sources(folder: str = CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def _compile(src: str, verbose: bool) -> str:
    sub = "probe_" if os.path.dirname(src) == PROBE_DIR else ""
    obj = os.path.join(OBJ_DIR, sub + os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def _link(objs, out: str, verbose: bool) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs, probe = sources(), sources(PROBE_DIR)
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs) + len(probe))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + probe))
    _link(objs[:len(srcs)], LIB, verbose)
    _link(objs[len(srcs):], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
