"""CPU oracle for the ternary-weight linear layer.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
and its Python binding never import, link or call it, and it imports nothing
from them: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, fp64 / exact integer); this
module only compiles it with gcc, marshals numpy arrays and checks shapes.
Sources, cited by page title and section:

* "NInfer sm_89 fork" article, section 9 item 2 (ternary weights, one fp16
  scale per 128 weights, int8 prefill contraction) and section 7 (int8
  activation artifact).
* "NINFER ternary perf-tuning" notes, section 2 (rung map: s8 from T = 17)
  and section 4 (numeric gate: only the s8 rung changes numerics).

Array conventions: bf16 and fp16 values travel as their uint16 bit patterns;
``x`` is ``[T, K]``, ``w`` is int8 ``[N, K]`` in {-1, 0, +1}, scales are
``[N, K // G]`` with group ``g`` covering ``k in [g*G, (g+1)*G)``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-std=gnu11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
             "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU, no HIP)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        lib = ctypes.CDLL(_SO)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        for name, args in {
            "oracle_linear_bf16": [p, i64, i64, p, p, i64, i64, p],
            "oracle_quant_s8": [p, i64, i64, p, p],
            "oracle_s8_acc": [p, i64, i64, p, i64, i64, p],
            "oracle_linear_s8": [p, p, i64, i64, p, p, i64, i64, p],
            "oracle_linear_s8_fp32_ordered": [p, p, i64, i64, p, p, i64, i64, p],
            "oracle_unpack_layout_v1": [p, p, i64, i64, i64, p, p],
            "oracle_unpack_layout_t5": [p, p, i64, i64, i64, p, p],
            "oracle_rotate_f32": [p, i64, i64, p],
            "oracle_quant_s8_rot": [p, i64, i64, p, p],
        }.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        _lib = lib
    return _lib


_ERRORS = {-1: "bad arguments", -2: "weight outside {-1,0,+1} (or invalid code)",
           -3: "non-finite input"}


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _group(K: int, s: np.ndarray) -> int:
    ng = s.shape[1]
    if ng <= 0 or K % ng:
        raise ValueError(f"scale columns {ng} do not divide K={K}")
    return K // ng


def linear_bf16(x: np.ndarray, w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 reference of the bf16-activation rungs: y[t, n] (float64 [T, N])."""
    x = _c(x, np.uint16)
    w = _c(w, np.int8)
    s = _c(s, np.uint16)
    T, K = x.shape
    N = w.shape[0]
    assert w.shape == (N, K) and s.shape[0] == N
    G = _group(K, s)
    y = np.empty((T, N), np.float64)
    _check(_load().oracle_linear_bf16(_ptr(x), T, K, _ptr(w), _ptr(s), N, G, _ptr(y)),
           "linear_bf16")
    return y


def quant_s8(x: np.ndarray):
    """Per-token int8 codes and scales: (q int8 [T, K], scale float32 [T])."""
    x = _c(x, np.uint16)
    T, K = x.shape
    q = np.empty((T, K), np.int8)
    sc = np.empty((T,), np.float32)
    _check(_load().oracle_quant_s8(_ptr(x), T, K, _ptr(q), _ptr(sc)), "quant_s8")
    return q, sc


def rotate_f32(x: np.ndarray) -> np.ndarray:
    """Blockwise (1024) orthonormal Hadamard rotation of bf16 x [T, K] in fp32
    (fast Walsh-Hadamard butterflies, strides 1, 2, ..., 512): float32 [T, K]."""
    x = _c(x, np.uint16)
    T, K = x.shape
    xr = np.empty((T, K), np.float32)
    _check(_load().oracle_rotate_f32(_ptr(x), T, K, _ptr(xr)), "rotate_f32")
    return xr


def quant_s8_rot(x: np.ndarray):
    """Rotated per-token int8 quantisation: quant_s8's rule applied to
    rotate_f32(x). Returns (q int8 [T, K], scale float32 [T])."""
    x = _c(x, np.uint16)
    T, K = x.shape
    q = np.empty((T, K), np.int8)
    sc = np.empty((T,), np.float32)
    _check(_load().oracle_quant_s8_rot(_ptr(x), T, K, _ptr(q), _ptr(sc)), "quant_s8_rot")
    return q, sc


def s8_acc(q: np.ndarray, w: np.ndarray, G: int) -> np.ndarray:
    """Integer group accumulators acc[t, n, g] (int32 [T, N, K // G])."""
    q = _c(q, np.int8)
    w = _c(w, np.int8)
    T, K = q.shape
    N = w.shape[0]
    assert w.shape == (N, K) and K % G == 0
    acc = np.empty((T, N, K // G), np.int32)
    _check(_load().oracle_s8_acc(_ptr(q), T, K, _ptr(w), N, G, _ptr(acc)), "s8_acc")
    return acc


def linear_s8(q: np.ndarray, scale: np.ndarray, w: np.ndarray, s: np.ndarray) -> np.ndarray:
    """Exactly rounded s8 output y[t, n] (float32 [T, N])."""
    q = _c(q, np.int8)
    scale = _c(scale, np.float32)
    w = _c(w, np.int8)
    s = _c(s, np.uint16)
    T, K = q.shape
    N = w.shape[0]
    assert w.shape == (N, K) and scale.shape == (T,) and s.shape[0] == N
    G = _group(K, s)
    y = np.empty((T, N), np.float32)
    _check(_load().oracle_linear_s8(_ptr(q), _ptr(scale), T, K, _ptr(w), _ptr(s), N, G,
                                    _ptr(y)), "linear_s8")
    return y


def linear_s8_fp32_ordered(q: np.ndarray, scale: np.ndarray, w: np.ndarray,
                           s: np.ndarray) -> np.ndarray:
    """s8 output in the canonical fp32 order (groups ascending, one fmaf each,
    then one multiply by the token scale): the bitwise reference for kernels
    that keep that order."""
    q = _c(q, np.int8)
    scale = _c(scale, np.float32)
    w = _c(w, np.int8)
    s = _c(s, np.uint16)
    T, K = q.shape
    N = w.shape[0]
    G = _group(K, s)
    y = np.empty((T, N), np.float32)
    _check(_load().oracle_linear_s8_fp32_ordered(_ptr(q), _ptr(scale), T, K, _ptr(w), _ptr(s),
                                                 N, G, _ptr(y)), "linear_s8_fp32_ordered")
    return y


def unpack_layout_v1(codes: np.ndarray, scales_packed: np.ndarray, N: int, K: int, G: int):
    """Independent reader of packed layout v1: returns (w int8 [N, K], s uint16 [N, K//G])."""
    codes = _c(codes, np.uint8).reshape(-1)
    scales_packed = _c(scales_packed, np.uint16).reshape(-1)
    assert codes.size == N * K // 4 and scales_packed.size == N * (K // G)
    w = np.empty((N, K), np.int8)
    s = np.empty((N, K // G), np.uint16)
    _check(_load().oracle_unpack_layout_v1(_ptr(codes), _ptr(scales_packed), N, K, G, _ptr(w),
                                           _ptr(s)), "unpack_layout_v1")
    return w, s


def unpack_layout_t5(codes: np.ndarray, scales_packed: np.ndarray, N: int, K: int, G: int):
    """Independent reader of the base-3 layout t5 (five weights per byte):
    returns (w int8 [N, K], s uint16 [N, K//G])."""
    codes = _c(codes, np.uint8).reshape(-1)
    scales_packed = _c(scales_packed, np.uint16).reshape(-1)
    assert codes.size == N * (K // 1024) * 208 and scales_packed.size == N * (K // G)
    w = np.empty((N, K), np.int8)
    s = np.empty((N, K // G), np.uint16)
    _check(_load().oracle_unpack_layout_t5(_ptr(codes), _ptr(scales_packed), N, K, G, _ptr(w),
                                           _ptr(s)), "unpack_layout_t5")
    return w, s
