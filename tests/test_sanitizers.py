"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): tern_host.cpp (argument validation, tern_pack / tern_unpack, the
dispatcher and its dry run) and the oracle, each rebuilt with
-fsanitize=address,undefined into a scratch copy of the package, then the
host ABI tests and the oracle pins run against those builds in a child
process. Any out-of-bounds access, use after free or undefined behaviour
aborts the child. The kernels' objects are linked unchanged (no GPU code is
instrumented and none is launched)."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "ternary_weight_linear_amd")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
KERNEL_OBJS = ("tern_kernels", "tern_s8", "tern_s8mma", "tern_b16mma", "tern_tile", "tern_limb",
               "tern_limbtile", "tern_probe", "tern_noalloc", "tern_chain", "tern_narrow")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def test_host_code_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    objs = [os.path.join(PKG, "_build", f + ".o") for f in KERNEL_OBJS]
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("kernel objects not built (run the package build first)")
    tree = tmp_path / "tree"
    shutil.copytree(os.path.join(ROOT, "tern_synth"), tree / "tern_synth",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "include"), tree / "include")
    shutil.copytree(os.path.join(ROOT, "tests"), tree / "tests",
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), tree)
    os.makedirs(tree / "oracle")
    for f in ("__init__.py", "oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", f), tree / "oracle")
    os.makedirs(tree / "ternary_weight_linear_amd")
    shutil.copy(os.path.join(PKG, "__init__.py"), tree / "ternary_weight_linear_amd")
    # the oracle with the flags of oracle/__init__.py plus the sanitizers
    import oracle as ora
    flags = [f for f in ora.GCC_FLAGS if f != "-O2"] + ["-O1", "-g"]
    subprocess.check_call(["gcc", *flags, *SAN, "-o", str(tree / "oracle" / "liboracle.so"),
                           str(tree / "oracle" / "oracle.c"), "-lm"])
    # the host side of libtern.so, linked with the unchanged kernel objects
    host_o = str(tmp_path / "tern_host.o")
    subprocess.check_call(["g++", "-O1", "-g", "-std=c++17", "-fPIC", *SAN, "-I",
                           os.path.join(ROOT, "include"), "-c",
                           os.path.join(PKG, "csrc", "tern_host.cpp"), "-o", host_o])
    subprocess.check_call(["g++", "-shared", *SAN, "-o", str(tree / "ternary_weight_linear_amd" / "libtern.so"),
                           host_o, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"])
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", PYTHONPATH=str(tree),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # -s: a sanitizer report goes to the child's stderr, not into pytest's capture
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-s", "-p", "no:cacheprovider",
                        "-m", "not gpu", "tests/test_host_abi.py", "tests/test_oracle_pins.py"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
    assert " passed" in r.stdout, tail
