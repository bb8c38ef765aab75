"""Pins for the CPU oracle, checked against things other than the oracle.

Each test pins one oracle function to hand-worked values, closed forms,
invariants, an independent library routine (numpy BLAS / int64 einsum) or an
exact rational computation, so that a dropped term, a wrong sign, a
transposed operand or a different rounding rule fails at least one of them.
CPU only.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import tern_synth as ts
from tests import exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


@pytest.fixture(scope="module")
def hand():
    with open(GOLDEN) as f:
        return json.load(f)


def bf16(a) -> np.ndarray:
    return ts.f32_to_bf16_bits(np.asarray(a, np.float32))


def f16(a) -> np.ndarray:
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


# ------------------------------------------------------------ hand-worked


def test_hand_linear_bf16(hand):
    c = hand["linear_bf16"]
    x = bf16(c["x"])
    assert np.array_equal(ts.bf16_bits_to_f32(x), np.asarray(c["x"], np.float32))
    y = oracle.linear_bf16(x, np.asarray(c["w"], np.int8), f16(c["s"]))
    assert np.array_equal(y, np.asarray(c["y"], np.float64))


def test_hand_quant_s8(hand):
    for c in hand["quant_s8"]:
        x = bf16([c["x"]])
        q, sc = oracle.quant_s8(x)
        assert exact.f32_bits(float(sc[0])) == int(c["scale_bits"], 16), c["derivation"]
        assert q[0].tolist() == c["q"], c["derivation"]


def test_hand_s8_acc_and_linear(hand):
    c = hand["s8_linear"]
    q = np.asarray([c["q"]], np.int8)
    w = np.asarray(c["w"], np.int8)
    acc = oracle.s8_acc(q, w, c["G"])
    assert acc[0].tolist() == c["acc"]
    y = oracle.linear_s8(q, np.asarray([c["scale"]], np.float32), w, f16(c["s"]))
    assert y[0].tolist() == c["y"]


def test_hand_layout_reader(hand):
    c = hand["layout_v1"]
    N, K, G = c["N"], c["K"], c["G"]
    sp = np.zeros(N * (K // G), np.uint16)
    for case in c["cases"]:
        codes = np.zeros(N * K // 4, np.uint8)
        codes[case["byte"]] = int(case["value"], 16)
        w, _ = oracle.unpack_layout_v1(codes, sp, N, K, G)
        nz = np.argwhere(w != 0)
        assert nz.tolist() == [[case["n"], case["k"]]], case["derivation"]
        assert w[case["n"], case["k"]] == case["w"], case["derivation"]
    codes = np.zeros(N * K // 4, np.uint8)
    for sc in c["scale_cases"]:
        sp = np.zeros(N * (K // G), np.uint16)
        sp[sc["index"]] = 0x3C00  # fp16 1.0
        _, s = oracle.unpack_layout_v1(codes, sp, N, K, G)
        assert np.argwhere(s != 0).tolist() == [[sc["n"], sc["g"]]], sc["derivation"]


def _t5_zero(N, K):
    """An all-zero t5 matrix: main bytes 0x80 (five trits 1), tails 0x55."""
    codes = np.full(N * (K // 1024) * 208, 0x80, np.uint8)
    blocks = codes.reshape(-1, 3328)
    blocks[:, 3072:] = 0x55
    return codes


def test_hand_layout_t5_reader(hand):
    c = hand["layout_t5"]
    N, K, G = c["N"], c["K"], c["G"]
    sp = np.zeros(N * (K // G), np.uint16)
    assert c["zero_main"] == "0x80" and c["zero_tail"] == "0x55"
    w, _ = oracle.unpack_layout_t5(_t5_zero(N, K), sp, N, K, G)
    assert not w.any()
    for case in c["cases"]:
        codes = _t5_zero(N, K)
        codes[case["byte"]] = int(case["value"], 16)
        w, _ = oracle.unpack_layout_t5(codes, sp, N, K, G)
        assert np.argwhere(w != 0).tolist() == [[case["n"], case["k"]]], case["derivation"]
        assert w[case["n"], case["k"]] == case["w"], case["derivation"]


def test_layout_t5_every_byte_value():
    """Every canonical main byte ceil(256 v / 243), v = 0..242, decodes to the
    five base-3 digits of v (most significant first) minus one, at the
    weights of register 0..4 of lane 0, byte 0 (k = 32, 34, 36, 38 of k-block
    0 and 32 of k-block 1); every other byte value is rejected."""
    N, K, G = 16, 1024, 128
    sp = np.zeros(N * (K // G), np.uint16)
    canonical = {-(-256 * v // 243): v for v in range(243)}
    for b in range(256):
        codes = _t5_zero(N, K)
        codes[0] = b
        if b not in canonical:
            with pytest.raises(ValueError):
                oracle.unpack_layout_t5(codes, sp, N, K, G)
            continue
        v = canonical[b]
        digits = [(v // 3 ** (4 - d)) % 3 for d in range(5)]
        w, _ = oracle.unpack_layout_t5(codes, sp, N, K, G)
        assert w[0, [32, 34, 36, 38, 96]].tolist() == [d - 1 for d in digits], b
        assert np.count_nonzero(w) == sum(d != 1 for d in digits)


def test_layout_t5_rejects_tail_trit_3():
    N, K, G = 16, 1024, 128
    codes = _t5_zero(N, K)
    codes[3072] = 0x57  # bits 1:0 = 11
    with pytest.raises(ValueError):
        oracle.unpack_layout_t5(codes, np.zeros(N * (K // G), np.uint16), N, K, G)


def test_layout_reader_rejects_code_10():
    codes = np.zeros(16 * 256 // 4, np.uint8)
    codes[3] = 0x80  # bits 31:30 of lane 0 word 0 = 10
    with pytest.raises(ValueError):
        oracle.unpack_layout_v1(codes, np.zeros(16 * 2, np.uint16), 16, 256, 128)


# ------------------------------------------------------- closed forms


def _small_case(seed=7, T=3, N=16, K=256, G=64):
    rng = np.random.default_rng(seed)
    w = ts.draw_weights(rng, N, K, 1.0 / 3.0)
    s = ts.draw_scales(rng, N, K, G)
    x = bf16(rng.standard_normal((T, K)).astype(np.float32) * 3)
    return x, w, s


def test_zero_weights_give_zero():
    x, w, s = _small_case()
    y = oracle.linear_bf16(x, np.zeros_like(w), s)
    assert np.all(y == 0.0)
    q, sc = oracle.quant_s8(x)
    assert np.all(oracle.linear_s8(q, sc, np.zeros_like(w), s) == 0.0)
    assert np.all(oracle.s8_acc(q, np.zeros_like(w), 64) == 0)


@pytest.mark.parametrize("sign", [1, -1])
def test_all_same_sign_weights_give_group_sums(sign):
    # Integer x and power-of-two scales make every sum exact, so the closed
    # form y = sign * sum_g s[n, g] * (sum of x over group g) holds bit for bit.
    T, N, K, G = 2, 16, 256, 64
    x = ts.integer_activations(K, T, seed=11)
    s = ts.pow2_scales(N, K, G, seed=12)
    w = np.full((N, K), sign, np.int8)
    y = oracle.linear_bf16(x, w, s)
    xs = ts.bf16_bits_to_f32(x).astype(np.float64).reshape(T, K // G, G).sum(-1)  # [T, NG]
    sv = s.view(np.float16).astype(np.float64)  # [N, NG]
    expect = sign * (xs @ sv.T)
    assert np.array_equal(y, expect)


def test_single_nonzero_weight_picks_one_product():
    x, w, s = _small_case(T=2)
    w = np.zeros_like(w)
    w[5, 77] = -1
    y = oracle.linear_bf16(x, w, s)
    xf = ts.bf16_bits_to_f32(x).astype(np.float64)
    sv = s.view(np.float16).astype(np.float64)
    expect = np.zeros_like(y)
    expect[:, 5] = -sv[5, 77 // 64] * xf[:, 77]
    assert np.array_equal(y, expect)


# ---------------------------------------------------------- invariants


def test_linear_bf16_is_linear_in_x():
    T, N, K, G = 3, 32, 512, 128
    rng = np.random.default_rng(5)
    w = ts.draw_weights(rng, N, K, 0.4)
    s = ts.pow2_scales(N, K, G, seed=6)
    xi = rng.integers(-50, 51, size=(T, K)).astype(np.float32)
    x = bf16(xi)
    y = oracle.linear_bf16(x, w, s)
    assert np.array_equal(oracle.linear_bf16(bf16(2 * xi), w, s), 2 * y)
    assert np.array_equal(oracle.linear_bf16(bf16(-xi), w, s), -y)
    mask = rng.random(K) < 0.5  # disjoint supports: x1 + x2 is exact
    x1 = np.where(mask, xi, 0).astype(np.float32)
    x2 = np.where(mask, 0, xi).astype(np.float32)
    y12 = oracle.linear_bf16(bf16(x1), w, s) + oracle.linear_bf16(bf16(x2), w, s)
    assert np.array_equal(y12, y)


def test_quant_s8_invariances():
    x, _, _ = _small_case(T=4, K=512)
    xf = ts.bf16_bits_to_f32(x)
    q, sc = oracle.quant_s8(x)
    q2, sc2 = oracle.quant_s8(bf16(2 * xf))
    assert np.array_equal(q2, q) and np.array_equal(sc2, 2 * sc)
    qn, scn = oracle.quant_s8(bf16(-xf))
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)
    assert q.min() >= -127 and q.max() <= 127
    # the absmax element maps to +-127 exactly
    am = np.abs(xf).argmax(axis=1)
    assert np.array_equal(np.abs(q[np.arange(4), am]), np.full(4, 127, np.int8))


def test_linear_s8_sign_symmetry_bitwise():
    x, w, s = _small_case(T=3, N=32, K=512, G=128)
    q, sc = oracle.quant_s8(x)
    y = oracle.linear_s8(q, sc, w, s)
    yn = oracle.linear_s8(-q, sc, w, s)
    assert np.array_equal(yn.view(np.uint32), (-y).view(np.uint32))


def test_batch_invariance():
    x, w, s = _small_case(T=5)
    y = oracle.linear_bf16(x, w, s)
    q, sc = oracle.quant_s8(x)
    ys8 = oracle.linear_s8(q, sc, w, s)
    for t in range(5):
        assert np.array_equal(oracle.linear_bf16(x[t:t + 1], w, s)[0], y[t])
        qt, st = oracle.quant_s8(x[t:t + 1])
        assert np.array_equal(qt[0], q[t]) and st[0] == sc[t]
        assert np.array_equal(oracle.linear_s8(qt, st, w, s)[0].view(np.uint32),
                              ys8[t].view(np.uint32))


# ------------------------------------------------- library routines


def test_linear_bf16_matches_numpy_blas_on_dequantised_matrix():
    x, w, s = _small_case(T=4, N=64, K=1024, G=128)
    y = oracle.linear_bf16(x, w, s)
    xf = ts.bf16_bits_to_f32(x).astype(np.float64)
    W = w.astype(np.float64) * np.repeat(s.view(np.float16).astype(np.float64), 128, axis=1)
    y_np = xf @ W.T
    bound = 1e-13 * (np.abs(xf) @ np.abs(W).T)
    assert np.all(np.abs(y - y_np) <= bound)
    # a transposed/misaligned scale would be visibly off
    W_bad = w.astype(np.float64) * np.tile(s.view(np.float16).astype(np.float64), (1, 128))
    assert not np.allclose(xf @ W_bad.T, y)


def test_s8_acc_matches_int64_einsum():
    x, w, s = _small_case(T=4, N=48, K=512, G=64)
    q, _ = oracle.quant_s8(x)
    acc = oracle.s8_acc(q, w, 64)
    ref = np.einsum("tgk,ngk->tng", q.astype(np.int64).reshape(4, 8, 64),
                    w.astype(np.int64).reshape(48, 8, 64))
    assert np.array_equal(acc, ref)


# --------------------------------------------------- exact rationals


def test_linear_s8_is_exactly_rounded():
    x, w, s = _small_case(T=3, N=24, K=512, G=128)
    q, sc = oracle.quant_s8(x)
    y = oracle.linear_s8(q, sc, w, s)
    acc = oracle.s8_acc(q, w, 128)
    for t in range(3):
        st = exact.f32_to_fraction(float(sc[t]))
        for n in range(24):
            tot = sum(exact.half_bits_to_fraction(int(s[n, g])) * int(acc[t, n, g])
                      for g in range(4))
            assert exact.f32_bits(float(y[t, n])) == exact.fraction_to_f32_bits(st * tot)


def test_linear_s8_within_gate_of_fp32_order():
    # The fixed fp32-order diagnostic differs from the exactly rounded value
    # by accumulated fp32 rounding only (far below the 1e-6 relative gate).
    x, w, s = _small_case(T=4, N=64, K=2048, G=128)
    q, sc = oracle.quant_s8(x)
    y = oracle.linear_s8(q, sc, w, s).astype(np.float64)
    yo = oracle.linear_s8_fp32_ordered(q, sc, w, s).astype(np.float64)
    assert np.linalg.norm(yo - y) / np.linalg.norm(y) < 1e-6


def _runs(runs, dtype) -> np.ndarray:
    return np.concatenate([np.full(n, v, dtype) for v, n in runs])


def test_hand_s8_fp32_ordered(hand):
    """The canonical fp32 epilogue order, pinned on hand-worked cases where
    it differs from descending groups, from a separate multiply and add and
    from an fp64 accumulator (derivations in the golden file)."""
    for c in hand["s8_fp32_ordered"]["cases"]:
        q = _runs(c["q_runs"], np.int8)[None, :]
        w = _runs(c["w_runs"], np.int8)[None, :]
        s = f16([c["s"]])
        assert oracle.s8_acc(q, w, c["G"])[0, 0].tolist() == c["acc"], c["derivation"]
        sc = np.asarray([c["scale"]], np.float32)
        yo = oracle.linear_s8_fp32_ordered(q, sc, w, s)
        assert exact.f32_bits(float(yo[0, 0])) == int(c["y_ordered_bits"], 16), c["derivation"]
        ye = oracle.linear_s8(q, sc, w, s)
        assert exact.f32_bits(float(ye[0, 0])) == int(c["y_exact_bits"], 16), c["derivation"]


def test_s8_fp32_order_step_by_step_in_rationals():
    """The same order on random data, every step evaluated exactly in
    rationals and rounded once to fp32 (an fma is one rounding of
    acc * s + total; the final product one rounding of total * scale)."""
    x, w, s = _small_case(seed=21, T=4, N=16, K=8192, G=128)
    q, sc = oracle.quant_s8(x)
    yo = oracle.linear_s8_fp32_ordered(q, sc, w, s)
    acc = oracle.s8_acc(q, w, 128)
    for t in range(4):
        st = exact.f32_to_fraction(float(sc[t]))
        for n in range(16):
            tot = Fraction(0)
            for g in range(64):
                r = exact.half_bits_to_fraction(int(s[n, g])) * int(acc[t, n, g]) + tot
                tot = exact.f32_to_fraction(exact.bits_f32(exact.fraction_to_f32_bits(r)))
            assert exact.f32_bits(float(yo[t, n])) == exact.fraction_to_f32_bits(tot * st)


def _all_positive_bf16_upto(a: float) -> np.ndarray:
    b = np.arange(1, 0x7F80, dtype=np.uint32).astype(np.uint16)  # positive finite
    v = ts.bf16_bits_to_f32(b)
    return b[v <= a]


@pytest.mark.parametrize("absmax", [1.0, 3.0, 7.5, 20.0, 37.25, 51.5, 100.0, 126.0, 254.0,
                                    0.1875, 1e-3, 6.0e4])
def test_quant_code_rule_brute_force(absmax):
    """Every positive finite bf16 <= absmax (and its negation) against the
    exactly computed double rounding fl32(x / fl32(absmax / 127)) -> nearest
    even integer -> clamp."""
    a_bits = int(bf16([absmax])[0])
    a = exact.bf16_bits_to_fraction(a_bits)
    vals = _all_positive_bf16_upto(float(exact.bits_f32(a_bits << 16)))
    row = np.concatenate([[a_bits], vals, vals | 0x8000]).astype(np.uint16)[None, :]
    q, sc = oracle.quant_s8(row)
    sbits = exact.f32_bits(float(sc[0]))
    assert sbits == exact.quant_scale_exact(a)
    # the exact rule for every element
    cache = {}
    for i, b in enumerate(row[0].tolist()):
        key = b & 0x7FFF
        if key not in cache:
            cache[key] = exact.quant_code_exact(exact.bf16_bits_to_fraction(key), sbits)
        expect = cache[key] if not (b & 0x8000) else -cache[key]
        assert q[0, i] == expect, (hex(b), q[0, i], expect)


def test_quant_double_rounding_differs_from_single_rounding_somewhere():
    """The spec rounds twice (quotient to fp32, then to an integer). Over a
    range of scales this must differ from rounding the exact quotient once in
    at least one case; otherwise the brute-force test above could not tell
    the two rules apart."""
    diffs = 0
    for absmax in [3.0, 7.5, 20.0, 37.25, 51.5, 100.0]:
        a_bits = int(bf16([absmax])[0])
        sbits = exact.quant_scale_exact(exact.bf16_bits_to_fraction(a_bits))
        sc = exact.f32_to_fraction(exact.bits_f32(sbits))
        for b in _all_positive_bf16_upto(absmax).tolist():
            xv = exact.bf16_bits_to_fraction(b)
            once = max(-127, min(127, exact.rne_to_int(xv / sc)))
            if once != exact.quant_code_exact(xv, sbits):
                diffs += 1
    assert diffs > 0


# ------------------------------------- rotated activations (1024-wide blocks)
#
# oracle.rotate_f32 / quant_s8_rot: the blockwise Hadamard rotation that the
# "NInfer sm_89 fork" article (section 9 item 2) folds into the activation
# quantisation, on the 1024-wide blocks of the "NINFER ternary perf-tuning"
# notes (section 6, constants table). Pinned to the Hadamard matrix from
# scipy, closed forms, invariants and a hand-worked fp32 case.


def _sylvester(n):
    from scipy.linalg import hadamard
    return hadamard(n).astype(np.float64)


def test_rotation_matches_hadamard_matrix_within_fp32_bound():
    """fp64 product with scipy's Hadamard matrix: the fp32 butterflies may
    differ only by rounding, at most 10 stages x 2^-24 of the magnitude sum."""
    rng = np.random.default_rng(21)
    T, K = 3, 3072
    xf = rng.standard_normal((T, K)).astype(np.float32)
    xf[:, rng.choice(K, 30, replace=False)] *= 20.0
    x = bf16(xf)
    xd = ts.bf16_bits_to_f32(x).astype(np.float64)
    H = _sylvester(1024) / 32.0
    got = oracle.rotate_f32(x).astype(np.float64)
    for b in range(K // 1024):
        blk = slice(1024 * b, 1024 * (b + 1))
        want = xd[:, blk] @ H.T
        bound = 10 * 2.0 ** -24 * np.abs(xd[:, blk]).sum(axis=1, keepdims=True) / 32.0 * 2
        assert np.all(np.abs(got[:, blk] - want) <= bound)
    rel = np.linalg.norm(got - np.concatenate([xd[:, 1024 * b:1024 * (b + 1)] @ H.T
                                               for b in range(K // 1024)], axis=1)) / np.linalg.norm(got)
    assert rel < 1e-6


def test_rotation_exact_on_small_integers():
    """Integer inputs up to 16 in magnitude keep every partial sum an integer
    below 2^15: the fp32 butterflies are exact and equal the matrix product."""
    rng = np.random.default_rng(22)
    xi = rng.integers(-16, 17, size=(4, 2048)).astype(np.float32)
    got = oracle.rotate_f32(bf16(xi))
    H = _sylvester(1024)
    want = np.concatenate([xi[:, :1024] @ H.T, xi[:, 1024:] @ H.T], axis=1) / 32.0
    assert np.array_equal(got.astype(np.float64), want)


def test_rotation_closed_forms():
    """e_j goes to column j of H / 32; a block of ones to 32 e_0; blocks do
    not mix."""
    K = 2048
    for j in (0, 1, 3, 5, 511, 1000, 1023):
        x = np.zeros((1, K), np.uint16)
        x[0, 1024 + j] = 0x3F80  # 1.0 in the second block
        got = oracle.rotate_f32(x)[0]
        assert not got[:1024].any()
        i = np.arange(1024)
        sign = 1 - 2 * (np.array([bin(v & j).count("1") for v in i]) & 1)
        assert np.array_equal(got[1024:], (sign / 32.0).astype(np.float32))
    ones = np.full((1, 1024), 0x3F80, np.uint16)
    z = oracle.rotate_f32(ones)[0]
    assert z[0] == 32.0 and not z[1:].any()


def test_rotation_is_an_involution_and_odd():
    """H H = 1024 I: rotating the rotated unit vectors (values +-1/32, exact
    in bf16) gives them back exactly; rotate(-x) = -rotate(x) bitwise."""
    for j in (0, 7, 640):
        x = np.zeros((1, 1024), np.uint16)
        x[0, j] = 0x3F80
        z = oracle.rotate_f32(x)
        back = oracle.rotate_f32(bf16(z))[0]
        e = np.zeros(1024, np.float32)
        e[j] = 1.0
        assert np.array_equal(back, e)
    x, _, _ = _small_case(T=2, K=1024)
    z = oracle.rotate_f32(x)
    zn = oracle.rotate_f32(x ^ np.uint16(0x8000))
    assert np.array_equal(zn.view(np.uint32), (-z).view(np.uint32))


def test_rotation_stage_order_hand_worked():
    """Hand-worked fp32 case. x = (2^24, 1, 1, 1, 0, ...). Strides ascending:
    h=1 gives (2^24 + 1 -> 2^24 [tie to even], 2^24 - 1, 2, 0); h=2 gives
    (2^24 + 2, 2^24 - 1, 2^24 - 2, 2^24 - 1); later strides pair with zeros,
    so z[i] = that value at i mod 4, over 32. The exactly rounded sums would
    give (2^24 + 4)/32 at i = 0, and strides descending would swap the values
    at 1 and 2: either mistake fails this test."""
    x = np.zeros((1, 1024), np.uint16)
    x[0, 0] = 0x4B80  # 2^24
    x[0, 1:4] = 0x3F80
    z = oracle.rotate_f32(x)[0].astype(np.float64)
    want4 = np.array([2.0 ** 24 + 2, 2.0 ** 24 - 1, 2.0 ** 24 - 2, 2.0 ** 24 - 1]) / 32.0
    assert np.array_equal(z, np.tile(want4, 256))


def test_quant_s8_rot_equals_quant_of_exact_rotation():
    """Where every rotated value is exact in bf16 (inputs in {0, +-1} on
    four positions of a block: rotated values in {0, +-1/32, ..., +-4/32}),
    the rotated quantisation must equal quant_s8 of the rotated values, whose
    rule is pinned by brute force above."""
    rng = np.random.default_rng(23)
    T, K = 6, 3072
    xf = np.zeros((T, K), np.float32)
    for t in range(T):
        for b in range(K // 1024):
            pos = 1024 * b + rng.choice(1024, 4, replace=False)
            xf[t, pos] = rng.integers(-1, 2, size=4)
    xf[0, :] = 0.0  # an all-zero token
    x = bf16(xf)
    z = oracle.rotate_f32(x)
    zb = bf16(z)
    assert np.array_equal(ts.bf16_bits_to_f32(zb), z)
    q, sc = oracle.quant_s8_rot(x)
    q2, sc2 = oracle.quant_s8(zb)
    assert np.array_equal(q, q2) and np.array_equal(sc.view(np.uint32), sc2.view(np.uint32))
    assert sc[0] == 0.0 and not q[0].any()


def test_quant_s8_rot_invariances():
    x, _, _ = _small_case(T=4, K=2048)
    xf = ts.bf16_bits_to_f32(x)
    q, sc = oracle.quant_s8_rot(x)
    q2, sc2 = oracle.quant_s8_rot(bf16(2 * xf))
    assert np.array_equal(q2, q) and np.array_equal(sc2, 2 * sc)
    qn, scn = oracle.quant_s8_rot(x ^ np.uint16(0x8000))
    assert np.array_equal(qn, -q) and np.array_equal(scn, sc)
    # the largest rotated magnitude maps to +-127
    z = oracle.rotate_f32(x)
    am = np.abs(z).argmax(axis=1)
    assert np.array_equal(np.abs(q[np.arange(4), am]), np.full(4, 127, np.int8))
    for t in range(4):
        qt, st = oracle.quant_s8_rot(x[t:t + 1])
        assert np.array_equal(qt[0], q[t]) and st[0] == sc[t]


def test_rotation_rejects_ragged_blocks():
    with pytest.raises(ValueError):
        oracle.rotate_f32(np.zeros((1, 1536), np.uint16))
    with pytest.raises(ValueError):
        oracle.quant_s8_rot(np.zeros((1, 512), np.uint16))
