"""Host-side checks of the C ABI that need no GPU: the library loads and
exports every declared symbol, the offline relayout round-trips and agrees
with the oracle's independent layout reader and with hand-worked bytes, and
every invalid argument is rejected before any HIP call.
"""
from __future__ import annotations

import json
import os
import re
import subprocess
import sys

import numpy as np
import pytest

import oracle
import tern_synth as ts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tern.h")


@pytest.fixture(scope="module")
def tl():
    import ternary_weight_linear_amd as tl
    tl.lib()
    return tl


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tern_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function(tl):
    names = declared_functions()
    assert len(names) >= 14
    for name in names:
        assert hasattr(tl.lib(), name), name
    assert set(names) == set(tl.EXPORTS)
    assert tl.lib().tern_abi_version() == 1


def test_header_compiles_as_c():
    src = '#include "tern.h"\nint main(void){ tern_weights w; (void)w; return TERN_OK; }\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-x", "c", "-", "-o", os.devnull], input=src.encode(),
                       capture_output=True)
    assert r.returncode == 0, r.stderr.decode()


@pytest.mark.parametrize("n,k,G", [(16, 256, 64), (32, 512, 128), (128, 256, 64), (48, 768, 128)])
def test_pack_roundtrip_and_independent_reader(tl, n, k, G):
    rng = np.random.default_rng(n * 1000 + k)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.draw_scales(rng, n, k, G)
    codes, sp = tl.pack(w, s)
    assert codes.size == n * k // 4 and sp.size == n * (k // G)
    w2, s2 = tl.unpack(codes, sp, n, k, G)
    assert np.array_equal(w2, w) and np.array_equal(s2, s)
    w3, s3 = oracle.unpack_layout_v1(codes, sp, n, k, G)
    assert np.array_equal(w3, w) and np.array_equal(s3, s)


def test_pack_matches_hand_worked_bytes(tl):
    with open(os.path.join(ROOT, "tests", "golden", "hand_cases.json")) as f:
        c = json.load(f)["layout_v1"]
    N, K, G = c["N"], c["K"], c["G"]
    s = np.zeros((N, K // G), np.uint16)
    for case in c["cases"]:
        w = np.zeros((N, K), np.int8)
        w[case["n"], case["k"]] = case["w"]
        codes, _ = tl.pack(w, s)
        nz = np.flatnonzero(codes)
        assert nz.tolist() == [case["byte"]], case["derivation"]
        assert codes[case["byte"]] == int(case["value"], 16), case["derivation"]
    for sc in c["scale_cases"]:
        s = np.zeros((N, K // G), np.uint16)
        s[sc["n"], sc["g"]] = 0x3C00
        _, sp = tl.pack(np.zeros((N, K), np.int8), s)
        assert np.flatnonzero(sp).tolist() == [sc["index"]], sc["derivation"]


def test_code_10_is_never_written(tl):
    rng = np.random.default_rng(3)
    w = ts.draw_weights(rng, 64, 1024, 0.2)
    codes, _ = tl.pack(w, ts.draw_scales(rng, 64, 1024, 128))
    c = codes.view(np.uint8)
    for shift in (0, 2, 4, 6):
        assert not np.any(((c >> shift) & 3) == 2)


def test_pack_rejects_bad_values_and_shapes(tl):
    s = np.zeros((16, 2), np.uint16)
    w = np.zeros((16, 256), np.int8)
    w[3, 7] = 2
    with pytest.raises(tl.TernError) as e:
        tl.pack(w, s)
    assert e.value.status_name == "TERN_ERR_VALUE"
    for n, k, g in [(8, 256, 128), (16, 200, 100), (16, 256, 32), (17, 256, 128)]:
        with pytest.raises(tl.TernError) as e:
            tl.pack(np.zeros((n, k), np.int8), np.zeros((n, k // g), np.uint16))
        assert e.value.status_name == "TERN_ERR_SHAPE"


def test_unpack_rejects_code_10(tl):
    codes = np.zeros(16 * 256 // 4, np.uint8)
    codes[3] = 0x80
    with pytest.raises(tl.TernError) as e:
        tl.unpack(codes, None, 16, 256, 128)
    assert e.value.status_name == "TERN_ERR_VALUE"


def test_default_rung_map(tl):
    # "NINFER ternary perf-tuning" notes, section 2: 1 / 2..8 / 9..16 / >= 17
    expect = {1: "gemv", 2: "small_t", 8: "small_t", 9: "small_t_tiled", 16: "small_t_tiled",
              17: "s8", 36: "s8", 2048: "s8"}
    for T, r in expect.items():
        assert tl.resolve_rung(T) == r, T
    assert tl.resolve_rung(5, "s8") == "s8"
    assert tl.resolve_rung(40, "small_t_tiled") == "small_t_tiled"
    with pytest.raises(tl.TernError):
        tl.resolve_rung(17, "small_t")  # one 16-token tile only
    with pytest.raises(tl.TernError):
        tl.resolve_rung(0)


def test_workspace_sizes(tl):
    assert tl.workspace_bytes(1, 128, 256, 64) == 0
    assert tl.workspace_bytes(1, 5120, 17408, 128) == 0  # gemv
    assert tl.workspace_bytes(4, 128, 256, 64) == 0  # one k-tile: K is not split
    # the per-wave small-T kernel (narrow layers: T <= 8, or K <= 8192) and
    # the activation-tiled kernel of wide layers (no K split) keep no partial sums
    assert tl.workspace_bytes(16, 5120, 5120, 128) == 0
    assert tl.workspace_bytes(4, 5120, 17408, 128) == 0
    assert tl.workspace_bytes(8, 34816, 5120, 128) == 0
    # wide layers at T <= 4 run the limb path with the limbs made in the kernel
    assert tl.workspace_bytes(4, 34816, 5120, 128) == 0
    assert tl.workspace_bytes(2, 34816, 5120, 128, "small_t_tiled") == 0
    # the activation-tiled kernel splits a long K over workgroups: fp32
    # partials of one 16-token tile per K part
    ws16 = tl.workspace_bytes(16, 5120, 17408, 128)
    assert ws16 > 0 and ws16 % (16 * 5120 * 4) == 0
    # above one 16-token tile small_t_tiled runs the prefill kernel: no K split
    assert tl.workspace_bytes(40, 5120, 17408, 128, "small_t_tiled") == 0
    need = tl.workspace_bytes(17, 5120, 5120, 128)
    assert need >= 17 * 5120 + 17 * 4
    assert tl.workspace_bytes(3, 5120, 5120, 128, "s8") >= 3 * 5120 + 12
    with pytest.raises(tl.TernError):
        tl.workspace_bytes(1, 100, 256, 128)


def _call_linear_raw(tl, x_ptr, T, W, y_ptr, rung, ws, ws_bytes):
    return tl.lib().tern_linear(x_ptr, T, W, y_ptr, rung, ws, ws_bytes, None)


def test_linear_validation_happens_before_any_hip_call(tl):
    """Every call here is invalid, so none of them reaches a kernel launch
    (there is no GPU in this process)."""
    import ctypes
    L = tl.lib()
    good = tl._Weights(0x100000, 0x200000, 5120, 5120, 128, tl.LAYOUT_V1)
    ref = ctypes.byref(good)
    status = lambda *a: tl.STATUS[_call_linear_raw(tl, *a)]  # noqa: E731
    assert status(None, 1, ref, 0x300000, 0, None, 0) == "TERN_ERR_NULL"
    assert status(0x400000, 1, None, 0x300000, 0, None, 0) == "TERN_ERR_NULL"
    bad = tl._Weights(0x100000, 0x200000, 5120, 5000, 128, tl.LAYOUT_V1)
    assert status(0x400000, 1, ctypes.byref(bad), 0x300000, 0, None, 0) == "TERN_ERR_SHAPE"
    bad = tl._Weights(0x100000, 0x200000, 5120, 5120, 96, tl.LAYOUT_V1)
    assert status(0x400000, 1, ctypes.byref(bad), 0x300000, 0, None, 0) == "TERN_ERR_SHAPE"
    bad = tl._Weights(0x100000, 0x200000, 5120, 5120, 128, 0x1234)
    assert status(0x400000, 1, ctypes.byref(bad), 0x300000, 0, None, 0) == "TERN_ERR_LAYOUT"
    bad = tl._Weights(0x100004, 0x200000, 5120, 5120, 128, tl.LAYOUT_V1)
    assert status(0x400000, 1, ctypes.byref(bad), 0x300000, 0, None, 0) == "TERN_ERR_ALIGN"
    assert status(0x400002, 1, ref, 0x300000, 0, None, 0) == "TERN_ERR_ALIGN"
    assert status(0x400000, 0, ref, 0x300000, 0, None, 0) == "TERN_ERR_SHAPE"
    assert status(0x400000, 1, ref, 0x300000, 9, None, 0) == "TERN_ERR_RUNG"
    assert status(0x400000, 20, ref, 0x300000, tl.RUNG_ID["small_t"], None, 0) == "TERN_ERR_RUNG"
    # s8 without (enough) workspace fails loudly instead of falling back
    assert status(0x400000, 17, ref, 0x300000, 0, None, 0) == "TERN_ERR_WORKSPACE"
    assert status(0x400000, 17, ref, 0x300000, 0, 0x500000, 100) == "TERN_ERR_WORKSPACE"
    assert "workspace" in L.tern_last_error().decode()
    # nothing was counted by the probe
    assert all(v == 0 for v in tl.probe_snapshot().values())
    assert tl.last_rung() == "auto"
    assert L.tern_quant_act_s8(None, 1, 256, 0x100000, 0x200000, 0, None) == 1
    assert L.tern_quant_act_s8(0x100000, 1, 100, 0x200000, 0x300000, 0, None) == 2
    assert L.tern_quant_act_s8(0x100000, 1, 72, 0x200000, 0x300000, 1, None) == 2  # 64 | K
    assert L.tern_quant_act_s8(0x100000, 1, 256, 0x200000, 0x300000, 7, None) == 4
    # rotated quantisation: 1024-wide blocks, K in [1024, 32768]
    assert L.tern_quant_act_s8_rot(None, 1, 1024, 0x100000, 0x200000, 0, None) == 1
    for k in (256, 1536, 0, 65536):
        assert L.tern_quant_act_s8_rot(0x100000, 1, k, 0x200000, 0x300000, 0, None) == 2
    assert L.tern_quant_act_s8_rot(0x100000, 0, 1024, 0x200000, 0x300000, 0, None) == 2
    assert L.tern_quant_act_s8_rot(0x100000, 1, 1024, 0x200000, 0x300000, 7, None) == 4
    assert L.tern_quant_act_s8_rot(0x100008, 1, 1024, 0x200000, 0x300000, 0, None) == 3
    # streaming-read ceiling probe: size, depth, waves and alignment checked first
    assert L.tern_stream_read(None, 1024, 8, 8, 0x200000, None) == 1
    assert L.tern_stream_read(0x100000, 1024, 8, 8, None, None) == 1
    for nbytes in (0, 512, 1536):
        assert L.tern_stream_read(0x100000, nbytes, 8, 8, 0x200000, None) == 2
    for depth, waves in ((2, 8), (32, 8), (8, 0), (8, 33)):
        assert L.tern_stream_read(0x100000, 1024, depth, waves, 0x200000, None) == 4
    assert L.tern_stream_read(0x100008, 1024, 8, 8, 0x200000, None) == 3
    assert L.tern_stream_read(0x100000, 1024, 8, 8, 0x200002, None) == 3


def test_unfused_limb_path_declares_its_workspace():
    """With the limbs made by the separate prep kernel (TERN_TUNE_SMALLT=limb2)
    the workspace holds one row block of 16 int8 limb rows and the per-token
    k-tile exponents, each 256-byte aligned; two row blocks above 4 tokens."""
    out = _run_env({"TERN_TUNE_SMALLT": "limb2"},
                   "import ternary_weight_linear_amd as tl\n"
                   "print(tl.workspace_bytes(4, 34816, 5120, 128), tl.workspace_bytes(8, 34816, 5120, 128))")
    assert out.split() == [str(16 * 5120 + 512), str(32 * 5120 + 768)]


def _run_env(env_extra: dict, code: str) -> str:
    env = dict(os.environ)
    env.update(env_extra)
    env["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout.strip()


PROBE = ("import ternary_weight_linear_amd as tl\n"
         "out=[]\n"
         "for T in (1,4,12,17,100):\n"
         "    try: out.append(tl.resolve_rung(T))\n"
         "    except tl.TernError as e: out.append(e.status_name)\n"
         "print(','.join(out))\n")


def test_env_knobs_steer_the_dispatcher():
    assert _run_env({}, PROBE) == "gemv,small_t,small_t_tiled,s8,s8"
    assert _run_env({"TERN_S8": "0"}, PROBE) == "gemv,small_t,small_t_tiled,small_t_tiled,small_t_tiled"
    assert _run_env({"TERN_S8_MIN_T": "33"}, PROBE) == "gemv,small_t,small_t_tiled,small_t_tiled,s8"
    assert _run_env({"TERN_SMALL_T_MAX": "16"}, PROBE) == "gemv,small_t,small_t,s8,s8"
    assert _run_env({"TERN_RUNG": "s8"}, PROBE) == "s8,s8,s8,s8,s8"
    assert _run_env({"TERN_RUNG": "small_t"}, PROBE) == ("small_t,small_t,small_t,"
                                                         "TERN_ERR_RUNG,TERN_ERR_RUNG")


@pytest.mark.parametrize("env", [{"TERN_RUNG": "fast"}, {"TERN_S8": "2"}, {"TERN_S8_MIN_T": "x"},
                                 {"TERN_SMALL_T_MAX": "17"}, {"TERN_DEBUG": "yes"}])
def test_invalid_env_fails_every_call(env):
    assert _run_env(env, PROBE) == ",".join(["TERN_ERR_CONFIG"] * 5)
    code = ("import ternary_weight_linear_amd as tl, ctypes\n"
            "w=tl._Weights(0x100000,0x200000,5120,5120,128,tl.LAYOUT_V1)\n"
            "print(tl.STATUS[tl.lib().tern_linear(0x400000,1,ctypes.byref(w),0x300000,0,None,0,None)])\n"
            "print(tl.lib().tern_last_error().decode())\n")
    out = _run_env(env, code).splitlines()
    assert out[0] == "TERN_ERR_CONFIG" and "invalid" in out[1]


def test_env_is_read_once():
    code = ("import os, ternary_weight_linear_amd as tl\n"
            "a = tl.resolve_rung(4)\n"
            "os.environ['TERN_RUNG'] = 's8'\n"
            "print(a, tl.resolve_rung(4))\n")
    assert _run_env({}, code) == "small_t small_t"
