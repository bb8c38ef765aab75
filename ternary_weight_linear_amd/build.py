"""Build libtern.so (gfx950 kernels + host C ABI) in-tree with hipcc.

Usage: ``python -m ternary_weight_linear_amd.build`` (or ``build()``). Always
recompiles. The result is ``ternary_weight_linear_amd/libtern.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libtern.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Device code: MI355X only. Packed-fp32 VALU ops are disabled (hipcc hands the
# target feature to the host pass as well, which ignores it with a warning that
# _run drops); fp32 division is the correctly rounded IEEE one (the s8
# quantisation relies on it); fp32 denormals are kept.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-ffp-contract=off", "-Wall",
]
# The host pass's note that it does not know the gfx950 feature above.
_HOST_FEATURE_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "".join(line for line in r.stdout.splitlines(keepends=True)
                  if line.strip() != _HOST_FEATURE_NOTE)
    if out:
        print(out, end="", flush=True)
    if r.returncode:
        raise subprocess.CalledProcessError(r.returncode, cmd)


# The s8 contraction reads every MFMA accumulator in its fp32 epilogue: keep
# MFMA results in VGPRs (no accumulator-register round trips).
S8_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


# (source, extra flags) of every translation unit; the host ABI layer is
# plain C++ and builds with g++.
UNITS = [
    ("tern_kernels.hip", []),
    ("tern_s8.hip", S8_FLAGS),
    ("tern_s8mma.hip", S8_FLAGS),
    ("tern_b16mma.hip", []),
    ("tern_tile.hip", []),
    ("tern_limb.hip", []),
    ("tern_limbtile.hip", S8_FLAGS),
    ("tern_probe.hip", []),
    ("tern_noalloc.hip", []),
    ("tern_chain.hip", []),
    ("tern_narrow.hip", []),
]


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n or (os.cpu_count() or 1), 16))


def build(verbose: bool = True) -> str:
    """Compile every unit (in parallel, up to MAX_JOBS or the CPU count, at
    most 16 at once) and link libtern.so."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    cmds, objs = [], []
    for src, extra in UNITS:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmds.append([HIPCC, *HIP_FLAGS, *extra, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    h_obj = os.path.join(BUILD, "tern_host.o")
    cmds.append(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_host.cpp"), "-o", h_obj])
    objs.append(h_obj)
    with ThreadPoolExecutor(max_workers=_jobs()) as ex:
        for f in [ex.submit(_run, c) for c in cmds]:
            f.result()  # re-raises the first failure
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
