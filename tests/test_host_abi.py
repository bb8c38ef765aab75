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
    # the per-wave small-T kernel (o_proj up to 12 tokens) and the
    # activation-tiled kernel of wide layers (no K split) keep no partial sums
    assert tl.workspace_bytes(12, 5120, 5120, 128) == 0
    assert tl.workspace_bytes(8, 34816, 5120, 128) == 0
    # the narrow-layer kernel: the counter header, then 6 K parts of fp32
    # partials of T x N
    assert tl.workspace_bytes(4, 5120, 17408, 128) == 4096 + 6 * 4 * 5120 * 4
    assert tl.workspace_bytes(16, 5120, 5120, 128) == 4096 + 6 * 16 * 5120 * 4
    # wide layers at T <= 4 run the limb path with the limbs made in the kernel
    assert tl.workspace_bytes(4, 34816, 5120, 128) == 0
    assert tl.workspace_bytes(2, 34816, 5120, 128, "small_t_tiled") == 0
    # the activation-tiled kernel (forced) splits a long K over workgroups:
    # fp32 partials of one 16-token tile per K part, after the 4096-byte
    # header every non-empty workspace starts with
    ws16 = tl.workspace_bytes(16, 5120, 17408, 128)
    assert ws16 > 4096 and (ws16 - 4096) % (16 * 5120 * 4) == 0
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
    k-tile exponents, each 256-byte aligned; two row blocks above 4 tokens
    (after the 4096-byte header of every non-empty workspace)."""
    out = _run_env({"TERN_TUNE_SMALLT": "limb2"},
                   "import ternary_weight_linear_amd as tl\n"
                   "print(tl.workspace_bytes(4, 34816, 5120, 128), tl.workspace_bytes(8, 34816, 5120, 128))")
    assert out.split() == [str(4096 + 16 * 5120 + 512), str(4096 + 32 * 5120 + 768)]


def test_narrow_path_plan_and_workspace():
    """The narrow-layer kernel (forced with TERN_TUNE_SMALLT=narrow; at T = 1
    with TERN_TUNE_GEMV=narrow): one kernel, about one workgroup per CU (down:
    40 blocks of 8 strips, K in 6 parts), and a workspace of the 4096-byte
    counter header plus Pk fp32 partials of T x N; none without a K split."""
    out = _run_env({"TERN_TUNE_SMALLT": "narrow", "TERN_TUNE_GEMV": "narrow"},
                   "import ternary_weight_linear_amd as tl\n"
                   "print(tl.workspace_bytes(16, 5120, 17408, 128), tl.workspace_bytes(4, 5120, 5120, 128),\n"
                   "      tl.workspace_bytes(1, 5120, 17408, 128), tl.workspace_bytes(4, 128, 256, 64))\n"
                   "print(*tl.plan_kernels(4, 5120, 17408, 128, 'small_t'), *tl.plan_kernels(1, 5120, 5120, 128, 'gemv'),\n"
                   "      *tl.plan_kernels(4, 34816, 5120, 128, 'small_t'))")
    sizes, kernels = out.split("\n")
    assert sizes.split() == [str(4096 + 6 * 16 * 5120 * 4), str(4096 + 6 * 4 * 5120 * 4),
                             str(4096 + 6 * 1 * 5120 * 4), "0"]
    # forced, it takes wide layers too (272 blocks: one K part, no workspace)
    assert kernels.split() == ["smallt_narrow"] * 3


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


# ------------------------------------------------ kernel choice (dry run)

# Kernels the dispatcher runs by default, per layer shape (N, K) and T: the
# map that the measurements on the part chose (resident limbs on wide layers
# up to 6 tokens and on narrow ones up to 3 where they fit; the tiled kernel
# on wide layers above; on narrow ones the narrow-layer kernel with its
# in-launch K split from 3 tokens on down's long K and above 12 tokens on
# o_proj, the per-wave kernel between; s8 with a K split on short prefills
# of narrow layers).
DEFAULT_KERNELS = {
    (34816, 5120): {1: "gemv_limb", 2: "smallt_resident", 6: "smallt_resident", 8: "smallt_resident",
                    9: "smallt_tile", 16: "smallt_tile", 17: "quant_s8,s8_mma", 2048: "quant_s8,s8_mma"},
    (5120, 17408): {1: "gemv_limb", 2: "smallt_resident", 3: "smallt_narrow", 8: "smallt_narrow",
                    9: "smallt_narrow", 16: "smallt_narrow",
                    17: "quant_s8,s8_mma,s8_reduce", 2048: "quant_s8,s8_mma"},
    (5120, 5120): {1: "gemv_limb", 3: "smallt_resident", 4: "smallt_wave", 12: "smallt_wave",
                   13: "smallt_narrow", 16: "smallt_narrow",
                   36: "quant_s8,s8_mma,s8_reduce", 2048: "quant_s8,s8_mma"},
}


def test_plan_kernels_default_map(tl):
    for (n, k), by_t in DEFAULT_KERNELS.items():
        for T, names in by_t.items():
            assert ",".join(tl.plan_kernels(T, n, k, 128)) == names, (n, k, T)
    # forced rungs: small_t_tiled above one 16-token tile is the bf16 prefill
    assert tl.plan_kernels(100, 34816, 5120, 128, "small_t_tiled") == ["b16_prefill"]
    assert tl.plan_kernels(4, 34816, 5120, 128, "s8") == ["quant_s8", "s8_mma"]
    assert tl.plan_kernels(1, 5120, 5120, 128, "small_t") == ["smallt_resident"]
    with pytest.raises(tl.TernError):
        tl.plan_kernels(20, 5120, 5120, 128, "small_t")  # one 16-token tile at most
    with pytest.raises(tl.TernError):
        tl.plan_kernels(1, 100, 256, 128)


PLAN = ("import ternary_weight_linear_amd as tl\n"
        "print(';'.join(','.join(tl.plan_kernels(T, n, k, 128)) for T, n, k in "
        "((1, 34816, 5120), (4, 34816, 5120), (12, 5120, 17408), (2, 5120, 5120))))\n")


def test_tune_knobs_steer_the_kernel_choice():
    """TERN_TUNE_* arms select other kernels for the same rung; the dry run
    (and so the kernel probe) names them."""
    assert _run_env({}, PLAN) == "gemv_limb;smallt_resident;smallt_narrow;smallt_resident"
    assert _run_env({"TERN_TUNE_GEMV": "bf16"}, PLAN).split(";")[0] == "gemv_bf16"
    assert _run_env({"TERN_TUNE_SMALLT": "tile"}, PLAN).split(";")[1] == "smallt_tile"
    assert _run_env({"TERN_TUNE_SMALLT": "wave"}, PLAN).split(";")[1] == "smallt_wave"
    assert _run_env({"TERN_TUNE_SMALLT": "limb"}, PLAN).split(";")[1] == "smallt_limb_fused"
    assert _run_env({"TERN_TUNE_SMALLT": "limb2"}, PLAN).split(";")[1] == ("smallt_limb_prep,"
                                                                           "smallt_limb_tile")


def test_gemv_with_limbs_beyond_lds_runs_the_bf16_kernel(tl):
    # K = 16384 on a wide layer: the limbs and scales exceed the limb
    # kernel's LDS, so the gemv runs the bf16 kernel with one-token rows; at
    # K = 32768 the bf16 row no longer fits its LDS either and the 16-token
    # per-wave kernel runs (its absent rows read as zeros).
    assert tl.plan_kernels(1, 16384, 12288, 128) == ["gemv_limb"]
    assert tl.plan_kernels(1, 16384, 16384, 128) == ["gemv_bf16"]
    assert tl.plan_kernels(1, 16384, 32768, 128) == ["smallt_wave"]


@pytest.mark.parametrize("n", [16384, 34816])
def test_resident_choice_takes_the_group_size(tl, n):
    """The resident limb kernel keeps the workgroup's scales in LDS next to the
    limbs, twice the bytes at G = 64: the dispatcher must size its plan with
    the call's G, and a shape whose G = 64 plan does not fit must go to
    another kernel rather than fail at launch. The dry run and the launch
    share the plan, so this checks that the choice is made per G."""
    for k in range(7680, 16641, 768):
        for T in (4, 5, 6):
            a, b = tl.plan_kernels(T, n, k, 64), tl.plan_kernels(T, n, k, 128)
            assert len(a) >= 1 and len(b) >= 1


def test_tiled_max_knob():
    assert _run_env({"TERN_SMALL_T_TILED_MAX": "32"}, PROBE) == "gemv,small_t,small_t_tiled,small_t_tiled,s8"
    assert _run_env({"TERN_SMALL_T_TILED_MAX": "12"}, PROBE) == "gemv,small_t,small_t_tiled,s8,s8"
    # consistent with TERN_S8_MIN_T: accepted
    assert _run_env({"TERN_SMALL_T_TILED_MAX": "32", "TERN_S8_MIN_T": "33"}, PROBE) == \
        "gemv,small_t,small_t_tiled,small_t_tiled,s8"


@pytest.mark.parametrize("env", [{"TERN_SMALL_T_TILED_MAX": "x"}, {"TERN_SMALL_T_TILED_MAX": "0"},
                                 {"TERN_SMALL_T_TILED_MAX": "4"},  # below TERN_SMALL_T_MAX
                                 {"TERN_SMALL_T_TILED_MAX": "32", "TERN_S8_MIN_T": "20"}])
def test_invalid_tiled_max_fails_every_call(env):
    assert _run_env(env, PROBE) == ",".join(["TERN_ERR_CONFIG"] * 5)


def test_shape_limits_of_the_kernels(tl):
    """K above 2^20 or N above 2^24 would overflow the kernels' 32-bit
    offsets: rejected before any launch."""
    import ctypes
    L = tl.lib()
    assert L.tern_scale_count(16, 1 << 20, 128) == (16 * (1 << 20)) // 128
    assert L.tern_scale_count(16, (1 << 20) + 256, 128) == 0
    assert L.tern_scale_count(1 << 24, 256, 128) == (1 << 24) * 2
    assert L.tern_scale_count((1 << 24) + 16, 256, 128) == 0
    for n, k in (((1 << 24) + 16, 256), (16, (1 << 20) + 256)):
        w = tl._Weights(0x100000, 0x200000, n, k, 128, tl.LAYOUT_V1)
        st = L.tern_linear(0x400000, 1, ctypes.byref(w), 0x300000, 0, None, 0, None)
        assert tl.STATUS[st] == "TERN_ERR_SHAPE", (n, k)
        assert "above the supported" in L.tern_last_error().decode()
    assert L.tern_quant_act_s8(0x100000, 1, (1 << 20) + 64, 0x200000, 0x300000, 1, None) == 2


def test_kernel_probe_starts_empty_and_names_every_kernel(tl):
    L = tl.lib()
    tl.probe_reset()
    assert all(v == 0 for v in tl.kernel_probe_snapshot().values())
    assert tl.last_kernels() == []
    names = [L.tern_kernel_name(i).decode() for i in range(len(tl.KERNELS))]
    assert tuple(names) == tl.KERNELS
    assert L.tern_kernel_name(len(tl.KERNELS)).decode() == "invalid"
    src = open(HEADER).read()
    assert len(re.findall(r"^\s+TERN_KERNEL_[A-Z0-9_]+(?: = 0)?,", src, re.M)) == len(tl.KERNELS)


# ------------------------------------------------------ base-3 layout t5


@pytest.mark.parametrize("n,k,G", [(16, 1024, 128), (32, 2048, 64), (48, 3072, 128)])
def test_pack_t5_roundtrip_and_independent_reader(tl, n, k, G):
    rng = np.random.default_rng(n * 7 + k)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.draw_scales(rng, n, k, G)
    codes, sp = tl.pack(w, s, layout="t5")
    assert codes.size == n * (k // 1024) * 208 == tl.lib().tern_packed_code_bytes_t5(n, k)
    assert codes.size * 64 == n * k * 13 // 4 * 4  # 13 bytes per 64 weights
    w2, s2 = tl.unpack(codes, sp, n, k, G, layout="t5")
    assert np.array_equal(w2, w) and np.array_equal(s2, s)
    w3, s3 = oracle.unpack_layout_t5(codes, sp, n, k, G)
    assert np.array_equal(w3, w) and np.array_equal(s3, s)
    # the scales are re-laid exactly as for v1
    assert np.array_equal(sp, tl.pack(w, s)[1])


def test_pack_t5_hand_bytes(tl):
    """tern_pack_t5 writes the hand-worked bytes of the golden file."""
    with open(os.path.join(ROOT, "tests", "golden", "hand_cases.json")) as f:
        c = json.load(f)["layout_t5"]
    N, K, G = c["N"], c["K"], c["G"]
    s = np.zeros((N, K // G), np.uint16)
    zero, _ = tl.pack(np.zeros((N, K), np.int8), s, layout="t5")
    blocks = zero.reshape(-1, 3328)
    assert np.all(blocks[:, :3072] == int(c["zero_main"], 16)) and np.all(blocks[:, 3072:] == int(c["zero_tail"], 16))
    for case in c["cases"]:
        w = np.zeros((N, K), np.int8)
        w[case["n"], case["k"]] = case["w"]
        codes, _ = tl.pack(w, s, layout="t5")
        diff = np.flatnonzero(codes != zero)
        assert diff.tolist() == [case["byte"]], case["derivation"]
        assert codes[case["byte"]] == int(case["value"], 16), case["derivation"]


def test_t5_rejects_bad_input(tl):
    L = tl.lib()
    s = np.zeros((16, 8), np.uint16)
    with pytest.raises(tl.TernError):  # K not a multiple of 1024
        tl.pack(np.zeros((16, 512), np.int8), np.zeros((16, 4), np.uint16), layout="t5")
    w = np.zeros((16, 1024), np.int8)
    w[3, 5] = 2
    with pytest.raises(tl.TernError):
        tl.pack(w, s, layout="t5")
    codes, sp = tl.pack(np.zeros((16, 1024), np.int8), s, layout="t5")
    bad = codes.copy()
    bad[7] = 1  # not ceil(256 v / 243) of any v
    with pytest.raises(tl.TernError):
        tl.unpack(bad, sp, 16, 1024, 128, layout="t5")
    bad = codes.copy()
    bad[3072] = 0x57  # tail trit 3
    with pytest.raises(tl.TernError):
        tl.unpack(bad, sp, 16, 1024, 128, layout="t5")
    assert L.tern_packed_code_bytes_t5(16, 1536) == 0


def test_t5_dispatch(tl):
    """t5 weights run the gemv rung only; any other rung is an error, never a
    fallback."""
    import ctypes
    assert tl.plan_kernels(1, 34816, 5120, 128, layout="t5") == ["gemv_t5"]
    assert tl.plan_kernels(1, 5120, 17408, 128, "gemv", layout="t5") == ["gemv_t5"]
    for T, rung in ((4, "auto"), (1, "small_t"), (20, "auto"), (1, "s8")):
        with pytest.raises(tl.TernError) as e:
            tl.plan_kernels(T, 34816, 5120, 128, rung, layout="t5")
        assert "layout t5" in str(e.value)
    with pytest.raises(tl.TernError):
        tl.plan_kernels(1, 5120, 5376, 128, layout="t5")  # K % 1024
    W = tl._Weights(0x100000, 0x200000, 5120, 5120, 128, tl.LAYOUT_T5)
    st = tl.lib().tern_linear(0x400000, 4, ctypes.byref(W), 0x300000, 0, None, 0, None)
    assert tl.STATUS[st] == "TERN_ERR_LAYOUT"
    W = tl._Weights(0x100000, 0x200000, 5120, 5376, 128, tl.LAYOUT_T5)
    st = tl.lib().tern_linear(0x400000, 1, ctypes.byref(W), 0x300000, 0, None, 0, None)
    assert tl.STATUS[st] == "TERN_ERR_SHAPE"


# ------------------------------------------------------ decode chain (host)


def _chain(tl, shapes, afters, group=128, layout=None):
    arr = (tl._ChainItem * len(shapes))()
    for i, ((n, k), a) in enumerate(zip(shapes, afters)):
        arr[i].W = tl._Weights(0x100000, 0x200000, n, k, group, layout or tl.LAYOUT_V1)
        arr[i].x, arr[i].y, arr[i].y_bf16, arr[i].after = 0x300000, 0x400000, None, a
    return arr


def test_chain_table_bytes_and_validation(tl):
    """The table holds a header, the entries, the offsets of the record lists
    of up to 512 workgroups of 12 waves, and room for their records: every
    task and unit end, a switch per workgroup run of each item (at most one
    run per unit) and a signal per workgroup after every item that is
    waited on, the last two for each wave; invalid chains are refused before
    any HIP call."""
    L = tl.lib()
    shapes = [(5120, 5120), (34816, 5120), (5120, 17408)]
    arr = _chain(tl, shapes, [-1, 0, 1])
    # units: 320 strips in threes (K in 4 shares: 12 records a unit), 2176
    # single strips (K whole), 320 strips in twos (K in 6 shares); items 0
    # and 1 signal
    P, W = 512, 12
    records = (107 * W + W * 107 + W * P) + (2176 + W * P + W * P) + (160 * W + W * 160)
    assert L.tern_chain_table_bytes(arr, 3) == 16 + 3 * 80 + (P * W + 4) * 4 + 16 * records
    assert L.tern_chain_table_bytes(_chain(tl, shapes, [-1, 2, 1]), 3) == 0  # after must be earlier
    assert "after" in L.tern_last_error().decode()
    assert L.tern_chain_table_bytes(_chain(tl, shapes, [-1, -1, -1], layout=tl.LAYOUT_T5), 3) == 0
    mixed = _chain(tl, [(5120, 5120), (256, 256)], [-1, -1])
    mixed[1].W.group = 64
    assert L.tern_chain_table_bytes(mixed, 2) == 0 and "group" in L.tern_last_error().decode()
    bad = _chain(tl, shapes, [-1, -1, -1])
    bad[1].y = 0x400004
    assert L.tern_chain_table_bytes(bad, 3) == 0 and "aligned" in L.tern_last_error().decode()
    assert L.tern_chain_table_bytes(arr, 0) == 0
    plan = tl._ChainPlan(3, 128, 256, 4096, 1)
    assert tl.STATUS[L.tern_linear_chain(None, 0x100000, 0x200000, 16, 0x300000, 10, None)] == "TERN_ERR_NULL"
    import ctypes
    st = L.tern_linear_chain(ctypes.byref(plan), 0x100000, 0x200000, 8, 0x300000, 10, None)
    assert tl.STATUS[st] == "TERN_ERR_WORKSPACE"  # 4 counters + done needed
    st = L.tern_linear_chain(ctypes.byref(plan), 0x100000, 0x200000, 16, 0x300000, 0, None)
    assert tl.STATUS[st] == "TERN_ERR_VALUE"  # spin limit
