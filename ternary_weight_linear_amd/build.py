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


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include")]
    k_obj = os.path.join(BUILD, "tern_kernels.o")
    s8_obj = os.path.join(BUILD, "tern_s8.o")
    t_obj = os.path.join(BUILD, "tern_tile.o")
    limb_obj = os.path.join(BUILD, "tern_limb.o")
    s8m_obj = os.path.join(BUILD, "tern_s8mma.o")
    b16_obj = os.path.join(BUILD, "tern_b16mma.o")
    lt_obj = os.path.join(BUILD, "tern_limbtile.o")
    pr_obj = os.path.join(BUILD, "tern_probe.o")
    na_obj = os.path.join(BUILD, "tern_noalloc.o")
    ch_obj = os.path.join(BUILD, "tern_chain.o")
    nw_obj = os.path.join(BUILD, "tern_narrow.o")
    h_obj = os.path.join(BUILD, "tern_host.o")
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_kernels.hip"), "-o", k_obj])
    _run([HIPCC, *HIP_FLAGS, *S8_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_s8.hip"), "-o", s8_obj])
    _run([HIPCC, *HIP_FLAGS, *S8_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_s8mma.hip"), "-o", s8m_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_b16mma.hip"), "-o", b16_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_tile.hip"), "-o", t_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_limb.hip"), "-o", limb_obj])
    _run([HIPCC, *HIP_FLAGS, *S8_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_limbtile.hip"), "-o", lt_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_probe.hip"), "-o", pr_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_noalloc.hip"), "-o", na_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_chain.hip"), "-o", ch_obj])
    _run([HIPCC, *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_narrow.hip"), "-o", nw_obj])
    _run(["g++", *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "tern_host.cpp"), "-o", h_obj])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, k_obj, s8_obj, s8m_obj, b16_obj, t_obj, limb_obj, lt_obj,
          pr_obj, na_obj, ch_obj, nw_obj, h_obj])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
