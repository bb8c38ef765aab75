"""GPU parity: every rung of the HIP library against the CPU oracle.

Gates: bf16-activation rungs (gemv, small_t, small_t_tiled) within 2e-3
relative L2 of the fp64 oracle; s8 int8 codes, scales and int32 group
accumulators bit-exact; s8 fp32 output within 1e-6 relative L2 of the exactly
rounded oracle. Integer-valued inputs with power-of-two scales make every
fp32 step exact, so there the bf16 rungs must match bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tern_synth as ts

pytestmark = pytest.mark.gpu

BF16_GATE = 2e-3
S8_GATE = 1e-6
RUNGS = ("gemv", "small_t", "small_t_tiled", "s8")


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def tl(torch):
    import ternary_weight_linear_amd as tl
    tl.lib()
    return tl


def rel_l2(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return np.linalg.norm(y - ref) / (den if den > 0 else 1.0)


def to_dev_bf16(torch, xbits):
    return torch.from_numpy(xbits.view(np.int16)).cuda().view(torch.bfloat16)


def rung_ok(rung, T):
    return not (rung == "small_t" and T > 16)


def check_kernels(tl, T, W, rung):
    """The kernels the last call launched are the ones the dispatcher's dry
    run names for it, each launched once (kernel probe and per-call set)."""
    plan = tl.plan_kernels(T, W.n, W.k, W.group, rung, layout=W.layout)
    assert tl.last_kernels() == plan, (T, W.n, W.k, rung, tl.last_kernels(), plan)
    snap = tl.kernel_probe_snapshot()
    assert {k: v for k, v in snap.items() if v} == {k: 1 for k in plan}, snap
    return plan


def run(tl, torch, x_dev, W, rung):
    tl.probe_reset()
    y = tl.linear(x_dev, W, rung=rung)
    torch.cuda.synchronize()
    snap = tl.probe_snapshot()
    expect = rung if rung != "auto" else tl.resolve_rung(x_dev.shape[0])
    assert snap[expect] == 1 and sum(snap.values()) == 1, snap
    assert tl.last_rung() == expect
    check_kernels(tl, x_dev.shape[0], W, rung)
    return y.cpu().numpy()


def operand_order(q):
    """Rearrange row-major int8 codes into the documented s8 operand order:
    byte 64b + 16g + 4i + e of a row holds k = 64b + 8g + m(i, e)."""
    T, K = q.shape
    src = np.empty(64, np.int64)
    for g in range(4):
        for i in range(4):
            for e, m in enumerate((32 + 2 * i, 2 * i, 33 + 2 * i, 2 * i + 1)):
                src[16 * g + 4 * i + e] = 8 * g + m
    assert sorted(src.tolist()) == list(range(64))
    idx = (np.arange(K // 64)[:, None] * 64 + src[None, :]).reshape(-1)
    return q[:, idx]


def s8_splits_k(tl, T, W):
    """True when tern_linear's s8 rung splits K over workgroups for this call
    (its workspace then holds fp32 partials beyond q and the token scales)."""
    base = -(-T * W.k // 256) * 256 + -(-4 * T // 256) * 256
    return tl.workspace_bytes(T, W.n, W.k, W.group, "s8") > base


def check_s8(tl, torch, xbits, x_dev, W, w, s, y, rows=None):
    """q/scale bit-exact, acc bit-exact, y within 1e-6, and bit-exact to the
    fixed fp32 order the kernel documents (ascending groups). When the s8 rung
    splits K over workgroups, tern_linear adds the parts' fp32 totals instead:
    a different fixed order, held to the 1e-6 gate; the unsplit contraction
    (tern_linear_s8_q) is still checked bitwise."""
    q_ref, sc_ref = oracle.quant_s8(xbits)
    q, sc = tl.quant_act_s8(x_dev)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), sc_ref.view(np.uint32))
    ws, ss = (w, s) if rows is None else (w[rows], s[rows])
    ycols = y if rows is None else y[:, rows]
    ref = oracle.linear_s8(q_ref, sc_ref, ws, ss)
    assert rel_l2(ycols, ref) <= S8_GATE
    ordered = oracle.linear_s8_fp32_ordered(q_ref, sc_ref, ws, ss)
    split = s8_splits_k(tl, xbits.shape[0], W)
    if not split:
        assert np.array_equal(ycols.view(np.uint32), ordered.view(np.uint32))
    # the same contraction on the pre-quantised activations, in both layouts
    y2 = tl.linear_s8_q(q, sc, W)
    torch.cuda.synchronize()
    y2 = y2.cpu().numpy()
    y2cols = y2 if rows is None else y2[:, rows]
    assert np.array_equal(y2cols.view(np.uint32), ordered.view(np.uint32))
    if split:
        # both are held to the gate against the exact oracle above and below;
        # two results within it of the same value differ by at most twice it
        assert rel_l2(y, y2) <= 2 * S8_GATE
        y = y2  # the unsplit result, for the layout comparison below
    if q_ref.shape[1] % 64 == 0:
        qo, sco = tl.quant_act_s8(x_dev, layout="operand_order")
        torch.cuda.synchronize()
        assert np.array_equal(qo.cpu().numpy(), operand_order(q_ref))
        assert np.array_equal(sco.cpu().numpy().view(np.uint32), sc_ref.view(np.uint32))
        y3 = tl.linear_s8_q(qo, sco, W, layout="operand_order")
        torch.cuda.synchronize()
        assert np.array_equal(y3.cpu().numpy().view(np.uint32), y.view(np.uint32))


# ---------------------------------------------------------- small shape


@pytest.fixture(scope="module")
def small(tl, torch):
    wts = ts.weights(ts.SMALL)
    W = tl.TernaryWeights.from_host(wts.w, wts.s)
    return wts, W


@pytest.mark.parametrize("T", [1, 4])
@pytest.mark.parametrize("rung", RUNGS + ("auto",))
def test_small_case_every_rung(tl, torch, small, T, rung):
    wts, W = small
    xbits = ts.activations(wts, T)
    y = run(tl, torch, to_dev_bf16(torch, xbits), W, rung)
    effective = rung if rung != "auto" else tl.resolve_rung(T)
    if effective == "s8":
        check_s8(tl, torch, xbits, to_dev_bf16(torch, xbits), W, wts.w, wts.s, y)
    else:
        ref = oracle.linear_bf16(xbits, wts.w, wts.s)
        assert rel_l2(y, ref) <= BF16_GATE
        assert rel_l2(y, ref) <= 1e-6  # fp32 accumulation of exact products


def test_small_case_s8_accumulators_bit_exact(tl, torch, small):
    wts, W = small
    xbits = ts.activations(wts, 4)
    q_ref, _ = oracle.quant_s8(xbits)
    expect = oracle.s8_acc(q_ref, wts.w, 64)
    for layout, qh in (("row_major", q_ref), ("operand_order", operand_order(q_ref))):
        acc = tl.debug_s8_acc(torch.from_numpy(np.ascontiguousarray(qh)).cuda(), W, layout=layout)
        torch.cuda.synchronize()
        assert np.array_equal(acc.cpu().numpy(), expect), layout


# ------------------------------------------------ wide-layer limb plans


@pytest.mark.parametrize("ns,k", [(1024, 512), (1100, 512), (2176, 512), (1024, 16384)])
def test_wide_limb_plans_exact(tl, torch, ns, k):
    """Layers of 1024 strips or more run the gemv (T = 1) and the resident
    limb kernel (T = 2..6) in workgroups of NS / 136 waves, 4 to 12, one strip
    per wave: 7, 8 and 12 waves here, with a ragged last workgroup at 1100 and
    2176 strips. With K = 16384 the limbs and scales outgrow the LDS: the
    gemv falls back to the bf16 kernel, T = 2..4 take the fused limb kernel
    (the resident limbs would need 128-165 KB) and T = 5..8 the tile kernel. Integer activations and power-of-two scales make every product
    and sum exact in fp32, so each T must match the oracle bit for bit, rows
    of every workgroup included."""
    n, G = 16 * ns, 128
    rng = np.random.default_rng(ns)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.pow2_scales(n, k, G, seed=ns)
    W = tl.TernaryWeights.from_host(w, s)
    for T in range(1, 9):
        print("wide plan", ns, "strips, K", k, "T", T, flush=True)
        xbits = ts.integer_activations(k, T, seed=ns + T)
        ref = oracle.linear_bf16(xbits, w, s)
        assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
        y = run(tl, torch, to_dev_bf16(torch, xbits), W, "auto")
        assert tl.last_rung() == ("gemv" if T == 1 else "small_t")
        assert np.array_equal(y.astype(np.float64), ref), T


# ------------------------------------------------ exact (integer) inputs


@pytest.mark.parametrize("n,k,G", [(64, 512, 128), (128, 256, 64), (48, 1280, 128)])
@pytest.mark.parametrize("T", [1, 3, 8, 13, 16, 21])
def test_integer_inputs_bit_exact(tl, torch, n, k, G, T):
    rng = np.random.default_rng(n + k + T)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.pow2_scales(n, k, G, seed=n * 7 + T)
    xbits = ts.integer_activations(k, T, seed=k + T)
    W = tl.TernaryWeights.from_host(w, s)
    ref = oracle.linear_bf16(xbits, w, s)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)  # exact in fp32
    x_dev = to_dev_bf16(torch, xbits)
    for rung in ("gemv", "small_t", "small_t_tiled"):
        if not rung_ok(rung, T):
            continue
        y = run(tl, torch, x_dev, W, rung)
        assert np.array_equal(y.astype(np.float64), ref), rung


@pytest.mark.parametrize("rung", RUNGS)
def test_single_nonzero_weight(tl, torch, rung):
    n, k, G, T = 64, 768, 128, 5
    w = np.zeros((n, k), np.int8)
    w[37, 517] = -1
    rng = np.random.default_rng(1)
    s = ts.draw_scales(rng, n, k, G)
    xbits = ts.f32_to_bf16_bits(rng.standard_normal((T, k)).astype(np.float32))
    W = tl.TernaryWeights.from_host(w, s)
    x_dev = to_dev_bf16(torch, xbits)
    y = run(tl, torch, x_dev, W, rung)
    expect = np.zeros((T, n), np.float32)
    if rung == "s8":
        q, sc = oracle.quant_s8(xbits)
        expect[:, 37] = oracle.linear_s8(q, sc, w[37:38], s[37:38])[:, 0]
    else:
        sv = ts.f16_bits_to_f32(s[37, 517 // G])
        expect[:, 37] = -(sv * ts.bf16_bits_to_f32(xbits[:, 517]))
    assert np.array_equal(y.view(np.uint32), expect.view(np.uint32))


# ------------------------------------------------------------ edge cases


@pytest.mark.parametrize("G", [64, 128])
@pytest.mark.parametrize("T", [1, 2, 5, 13, 16, 17, 64, 65])
def test_minimal_shape_every_rung(tl, torch, G, T):
    """The smallest layer the boundary accepts, N = 16 (one strip) by K = 256
    (one k-tile), on every rung that takes T: integer activations and
    power-of-two scales, so the bf16 rungs match the oracle bit for bit and
    the s8 rung is checked as everywhere else."""
    n, k = 16, 256
    rng = np.random.default_rng(10 * T + G)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.pow2_scales(n, k, G, seed=T + G)
    xbits = ts.integer_activations(k, T, seed=T)
    W = tl.TernaryWeights.from_host(w, s)
    x_dev = to_dev_bf16(torch, xbits)
    ref = oracle.linear_bf16(xbits, w, s)
    assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    for rung in RUNGS + ("auto",):
        if not rung_ok(rung, T):
            continue
        print("minimal shape G", G, "T", T, "rung", rung, flush=True)
        y = run(tl, torch, x_dev, W, rung)
        effective = rung if rung != "auto" else tl.resolve_rung(T)
        if effective == "s8":
            check_s8(tl, torch, xbits, x_dev, W, w, s, y)
        else:
            assert np.array_equal(y.astype(np.float64), ref), rung


@pytest.mark.parametrize("T", [1, 4, 17])
def test_longest_k_every_rung(tl, torch, T):
    """The longest K the boundary accepts (2^20, 4096 k-tiles) on one strip:
    the gemv's bf16 fallback, the narrow-layer kernel's widest K split, the
    two-pass quantisation (K above 32768) and the s8 K split."""
    n, k, G = 16, 1 << 20, 128
    rng = np.random.default_rng(77 + T)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.draw_scales(rng, n, k, G)
    xbits = ts.f32_to_bf16_bits(rng.standard_normal((T, k)).astype(np.float32))
    W = tl.TernaryWeights.from_host(w, s)
    x_dev = to_dev_bf16(torch, xbits)
    ref = oracle.linear_bf16(xbits, w, s)
    for rung in RUNGS + ("auto",):
        if not rung_ok(rung, T):
            continue
        print("longest K, T", T, "rung", rung, flush=True)
        y = run(tl, torch, x_dev, W, rung)
        effective = rung if rung != "auto" else tl.resolve_rung(T)
        if effective == "s8":
            check_s8(tl, torch, xbits, x_dev, W, w, s, y)
        else:
            assert rel_l2(y, ref) <= BF16_GATE, rung
            assert rel_l2(y, ref) <= 1e-5, rung  # fp32 sums of exact products over 2^20 terms




@pytest.fixture(scope="module")
def mid(tl, torch):
    shape = ts.Shape("mid_1024x256", 1024, 256, 128, 0.4, True, 301)
    wts = ts.weights(shape)
    return wts, tl.TernaryWeights.from_host(wts.w, wts.s)


@pytest.mark.parametrize("T", [1, 2, 7, 9, 15, 16, 17, 31, 33, 63, 65, 100, 129])
def test_ragged_token_counts(tl, torch, mid, T):
    wts, W = mid
    xbits = ts.activations(wts, T)
    x_dev = to_dev_bf16(torch, xbits)
    ref = oracle.linear_bf16(xbits, wts.w, wts.s)
    for rung in ("auto",) + RUNGS:
        if not rung_ok(rung, T):
            continue
        y = run(tl, torch, x_dev, W, rung)
        eff = rung if rung != "auto" else tl.resolve_rung(T)
        if eff == "s8":
            check_s8(tl, torch, xbits, x_dev, W, wts.w, wts.s, y)
        else:
            assert rel_l2(y, ref) <= BF16_GATE, rung


def test_zero_activation_rows(tl, torch, mid):
    wts, W = mid
    xbits = ts.activations(wts, 40)
    xbits[[0, 5, 39]] = 0
    xbits[7] = 0x8000  # -0.0
    x_dev = to_dev_bf16(torch, xbits)
    for rung in ("small_t_tiled", "s8"):
        y = run(tl, torch, x_dev, W, rung)
        assert np.all(y[[0, 5, 7, 39]] == 0)
    q, sc = tl.quant_act_s8(x_dev)
    assert np.all(sc.cpu().numpy()[[0, 5, 7, 39]] == 0)
    assert np.all(q.cpu().numpy()[[0, 5, 7, 39]] == 0)
    check_s8(tl, torch, xbits, x_dev, W, wts.w, wts.s, tl.linear(x_dev, W, rung="s8").cpu().numpy())


def test_output_guard_bands_and_determinism(tl, torch, mid):
    wts, W = mid
    T, N = 12, W.n
    xbits = ts.activations(wts, T)
    x_dev = to_dev_bf16(torch, xbits)
    for rung in RUNGS:
        buf = torch.full((T * N + 64,), float("nan"), device="cuda")
        y = buf[:T * N].view(T, N)
        tl.linear(x_dev, W, rung=rung, y=y)
        y2 = tl.linear(x_dev, W, rung=rung)
        torch.cuda.synchronize()
        assert torch.isnan(buf[T * N:]).all(), rung
        assert not torch.isnan(y).any(), rung
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32)), rung


def test_batch_invariance(tl, torch, mid):
    """A token's output does not depend on the other rows of its batch:
    bitwise when the other rows change (same T, same kernel). For s8 also
    across batch sizes (per-token quantisation, fixed group order in every
    tile shape). small_t_tiled runs different kernels at T = 1 and T = 24
    (the per-wave kernel splits K over waves, the prefill kernel does not),
    so across batch sizes it is held to the fp32-accumulation bound only."""
    wts, W = mid
    xbits = ts.activations(wts, 24)
    other = ts.activations(wts, 24, salt=5)
    keep = [0, 11, 23]
    mixed = other.copy()
    mixed[keep] = xbits[keep]
    x_dev, m_dev = to_dev_bf16(torch, xbits), to_dev_bf16(torch, mixed)
    for rung in ("small_t_tiled", "s8"):
        y = tl.linear(x_dev, W, rung=rung).cpu()
        ym = tl.linear(m_dev, W, rung=rung).cpu()
        assert torch.equal(ym[keep].view(torch.int32), y[keep].view(torch.int32)), rung
        for t in keep:
            yt = tl.linear(x_dev[t:t + 1].contiguous(), W, rung=rung).cpu()
            if rung == "s8":
                assert torch.equal(yt[0].view(torch.int32), y[t].view(torch.int32)), (rung, t)
            else:
                assert rel_l2(yt[0].numpy(), y[t].numpy()) <= 1e-6, (rung, t)


def test_stacked_matrices_concatenate(tl, torch):
    """The packed layout is strip-major, so matrices stacked along N (fused
    q|k|v, gate|up) are their code and scale buffers concatenated; on exact
    inputs every rung gives each part's outputs bit for bit."""
    k, G = 768, 128
    rng = np.random.default_rng(71)
    parts = [(ts.draw_weights(rng, n, k, 0.4), ts.pow2_scales(n, k, G, seed=n)) for n in (48, 96, 32)]
    Ws = [tl.TernaryWeights.from_host(w, s) for w, s in parts]
    F = tl.TernaryWeights(torch.cat([W.codes for W in Ws]), torch.cat([W.scales for W in Ws]),
                          sum(W.n for W in Ws), k, G)
    for T in (1, 5, 23):
        x_dev = to_dev_bf16(torch, ts.integer_activations(k, T, seed=T + 70))
        for rung in RUNGS:
            if not rung_ok(rung, T):
                continue
            yf = tl.linear(x_dev, F, rung=rung).cpu().numpy()
            ys = np.concatenate([tl.linear(x_dev, W, rung=rung).cpu().numpy() for W in Ws], axis=1)
            assert np.array_equal(yf.view(np.uint32), ys.view(np.uint32)), (rung, T)


# ------------------------------------------------------ full layer shapes


@pytest.fixture(scope="module")
def big(tl, torch):
    cache = {}

    def get(shape):
        if shape.name not in cache:
            wts = ts.weights(shape)
            cache[shape.name] = (wts, tl.TernaryWeights.from_host(wts.w, wts.s))
        return cache[shape.name]

    return get


def sample_rows(N, seed, n=64):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(N, n, replace=False), [0, 15, 16, N - 1]]))
    return rows


@pytest.mark.parametrize("shape", [ts.GATE_UP, ts.DOWN])
def test_decode_T1_full_rows(tl, torch, big, shape):
    """Decode at T=1 on the 27B-class shapes: every output checked."""
    wts, W = big(shape)
    xbits = ts.activations(wts, 1)
    x_dev = to_dev_bf16(torch, xbits)
    ref = oracle.linear_bf16(xbits, wts.w, wts.s)
    for rung in ("auto", "gemv", "small_t"):
        y = run(tl, torch, x_dev, W, rung)
        assert rel_l2(y, ref) <= BF16_GATE, rung
        assert rel_l2(y, ref) <= 1e-6, rung


@pytest.mark.parametrize("shape", [ts.GATE_UP, ts.DOWN, ts.OUT_PROJ])
@pytest.mark.parametrize("T", [2, 4, 8, 12, 16])
def test_small_T_batches_sampled(tl, torch, big, shape, T):
    wts, W = big(shape)
    xbits = ts.activations(wts, T)
    x_dev = to_dev_bf16(torch, xbits)
    rows = sample_rows(W.n, T)
    ref = oracle.linear_bf16(xbits, wts.w[rows], wts.s[rows])
    for rung in ("auto", "small_t", "small_t_tiled"):
        y = run(tl, torch, x_dev, W, rung)
        assert rel_l2(y[:, rows], ref) <= BF16_GATE, rung


@pytest.mark.parametrize("shape,T", [(ts.DOWN, 3), (ts.DOWN, 8), (ts.DOWN, 16), (ts.OUT_PROJ, 16)],
                         ids=["down-3", "down-8", "down-16", "o_proj-16"])
def test_narrow_layers_full_shape(tl, torch, big, shape, T):
    """The narrow-layer kernel where the dispatcher picks it, at the layers'
    full size (240 workgroups, K in 6 parts): exact bf16 products summed in
    fp32, so within 1e-6 of the fp64 oracle on sampled rows; and, on integer
    activations with power-of-two scales (every partial sum exact), equal to
    the oracle bit for bit on the same rows."""
    wts, W = big(shape)
    assert tl.plan_kernels(T, W.n, W.k, W.group) == ["smallt_narrow"]
    xbits = ts.activations(wts, T)
    rows = sample_rows(W.n, T + 101)
    y = run(tl, torch, to_dev_bf16(torch, xbits), W, "auto")
    assert rel_l2(y[:, rows], oracle.linear_bf16(xbits, wts.w[rows], wts.s[rows])) <= 1e-6
    sp = ts.pow2_scales(W.n, W.k, W.group, seed=T)
    Wi = tl.TernaryWeights.from_host(wts.w, sp)
    xi = ts.integer_activations(W.k, T, seed=T + 3)
    yi = run(tl, torch, to_dev_bf16(torch, xi), Wi, "auto")
    refi = oracle.linear_bf16(xi, wts.w[rows], sp[rows]).astype(np.float32)
    assert np.array_equal(np.ascontiguousarray(yi[:, rows]).view(np.uint32), refi.view(np.uint32))


@pytest.mark.parametrize("shape", [ts.GATE_UP, ts.DOWN])
@pytest.mark.parametrize("T", [17, 36, 508, 2048])
def test_prefill_bf16_sampled(tl, torch, big, shape, T):
    """The bf16 prefill path (small_t_tiled above one 16-token tile, where
    T >= 17 goes with the s8 rung switched off): exact bf16 x {-1,0,+1}
    products summed in fp32, so well inside the 2e-3 gate."""
    wts, W = big(shape)
    xbits = ts.activations(wts, T)
    x_dev = to_dev_bf16(torch, xbits)
    rows = sample_rows(W.n, T + 7)
    y = run(tl, torch, x_dev, W, "small_t_tiled")
    ref = oracle.linear_bf16(xbits, wts.w[rows], wts.s[rows])
    assert rel_l2(y[:, rows], ref) <= BF16_GATE
    assert rel_l2(y[:, rows], ref) <= 1e-6


@pytest.mark.parametrize("shape", [ts.GATE_UP, ts.DOWN])
@pytest.mark.parametrize("T", [17, 36, 508, 2048])
def test_prefill_s8_sampled(tl, torch, big, shape, T):
    wts, W = big(shape)
    xbits = ts.activations(wts, T)
    x_dev = to_dev_bf16(torch, xbits)
    rows = sample_rows(W.n, T)
    y = run(tl, torch, x_dev, W, "auto")
    assert tl.resolve_rung(T) == "s8"
    check_s8(tl, torch, xbits, x_dev, W, wts.w, wts.s, y, rows=rows)
    if T <= 36 or T == 508:
        q_ref, _ = oracle.quant_s8(xbits)
        expect = oracle.s8_acc(q_ref, wts.w[rows], 128)
        layouts = (("operand_order", operand_order(q_ref)),)
        if T <= 36:
            layouts += (("row_major", q_ref),)
        for layout, qh in layouts:
            acc = tl.debug_s8_acc(torch.from_numpy(np.ascontiguousarray(qh)).cuda(), W, layout=layout)
            torch.cuda.synchronize()
            acc = acc.cpu().numpy()
            assert np.array_equal(acc[:, rows], expect), layout
            del acc


# ------------------------------------------------ launch-shape variants

_TUNE_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle, tern_synth as ts, ternary_weight_linear_amd as tl
shape = ts.Shape("tune_4096x96", 4096, 96, int(sys.argv[2]), 0.4, True, 401)
wts = ts.weights(shape)
W = tl.TernaryWeights.from_host(wts.w, wts.s)
worst = 0.0
seen = set()
for T in (1, 5, 16, 23):
    xb = ts.activations(wts, T)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    ref = oracle.linear_bf16(xb, wts.w, wts.s)
    for rung in ("gemv", "small_t", "small_t_tiled"):
        if rung == "small_t" and T > 16:
            continue
        y = tl.linear(x, W, rung=rung).cpu().numpy().astype(np.float64)
        ks = tl.last_kernels()
        assert ks == tl.plan_kernels(T, W.n, W.k, W.group, rung), (T, rung, ks)
        seen.update(ks)
        err = np.linalg.norm(y - ref) / np.linalg.norm(ref)
        worst = max(worst, err)
print("KERNELS", ",".join(sorted(seen)))
print("WORST", worst)
"""


@pytest.mark.parametrize("strips,waves,G", [(1, 1, 128), (2, 1, 64), (4, 1, 128), (4, 3, 64),
                                            (1, 16, 128), (2, 8, 128)])
def test_launch_shapes_keep_parity(strips, waves, G):
    """Every (strips per wave, waves per block) launch shape the tuning knobs
    can select for the per-wave bf16 kernel (one-token rows at T = 1 with
    TERN_TUNE_GEMV=bf16, 16-token tiles above), including multi-chunk
    k-ranges (16 k-tiles on one wave) and partial strip blocks (6 strips with
    4 per block), stays within the gate."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TERN_TUNE_STRIPS=str(strips), TERN_TUNE_WAVES=str(waves),
               TERN_TUNE_GEMV="bf16")
    r = subprocess.run([sys.executable, "-c", _TUNE_CHILD, root, str(G)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    worst = float(r.stdout.split("WORST")[1])
    assert worst <= 1e-6, worst
    # the per-wave kernel ran under the forced shape: one-token rows (the
    # gemv's bf16 kernel) and 16-token tiles
    seen = set(r.stdout.split("KERNELS")[1].split()[0].split(","))
    assert {"gemv_bf16", "smallt_wave"} <= seen, seen


@pytest.mark.parametrize("strips,waves,depth,kparts", [(1, 4, 2, 1), (1, 4, 8, 1), (2, 3, 4, 2),
                                                    (4, 2, 2, 4), (1, 8, 4, 3)])
def test_tile_kernel_shapes_keep_parity(strips, waves, depth, kparts):
    """The activation-tiled small-T kernel forced for T <= 16 (above that
    small_t_tiled runs the prefill kernel): 8- and 16-row activation tiles,
    code/activation rings of 2, 4 and 8 k-tiles, K split over 1..4
    workgroups (16 k-tiles), partial strip blocks and waves without strips."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TERN_TUNE_SMALLT="tile", TERN_TUNE_STRIPS=str(strips),
               TERN_TUNE_WAVES=str(waves), TERN_TUNE_DEPTH=str(depth), TERN_TUNE_KPARTS=str(kparts))
    r = subprocess.run([sys.executable, "-c", _TUNE_CHILD, root, "128"], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    worst = float(r.stdout.split("WORST")[1])
    assert worst <= 1e-6, worst
    seen = set(r.stdout.split("KERNELS")[1].split()[0].split(","))
    assert "smallt_tile" in seen and ("smallt_tile_reduce" in seen) == (kparts > 1), seen


_NARROW_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle, tern_synth as ts, ternary_weight_linear_amd as tl
G = int(sys.argv[2])
worst, bad, seen = 0.0, [], set()
# 6 strips over K = 4096 (16 k-tiles) and 25 strips over K = 2816 (11
# k-tiles): partial strip blocks, waves without a strip, K parts of 1..16
# k-tiles
for n, k in ((96, 4096), (400, 2816)):
    rng = np.random.default_rng(n + k + G)
    w = ts.draw_weights(rng, n, k, 0.4)
    shape = ts.Shape(f"narrow_{k}x{n}", k, n, G, 0.4, True, n + k)
    wts = ts.weights(shape)
    W = tl.TernaryWeights.from_host(wts.w, wts.s)
    sp = ts.pow2_scales(n, k, G, seed=n)
    Wi = tl.TernaryWeights.from_host(w, sp)
    for T in (1, 2, 3, 4, 5, 8, 9, 13, 16):
        rung = "gemv" if T == 1 else "small_t"
        ws = torch.zeros((max(1, tl.workspace_bytes(T, n, k, G, rung)),), dtype=torch.uint8, device="cuda")
        # two calls on one workspace with fresh activations: the second finds
        # the arrival counters the first left
        for salt in (0, 1):
            xb = ts.activations(wts, T, salt=salt)
            x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
            y = tl.linear(x, W, rung=rung, workspace=ws).cpu().numpy().astype(np.float64)
            ks = tl.last_kernels()
            assert ks == tl.plan_kernels(T, n, k, G, rung) == ["smallt_narrow"], (T, ks)
            seen.update(ks)
            ref = oracle.linear_bf16(xb, wts.w, wts.s)
            worst = max(worst, np.linalg.norm(y - ref) / np.linalg.norm(ref))
        # integer activations and power-of-two scales: every partial sum is
        # exact, so y must equal the oracle bit for bit
        xi = ts.integer_activations(k, T, seed=T)
        x = torch.from_numpy(xi.view(np.int16)).cuda().view(torch.bfloat16)
        yi = tl.linear(x, Wi, rung=rung, workspace=ws).cpu().numpy()
        refi = oracle.linear_bf16(xi, w, sp).astype(np.float32)
        if not np.array_equal(yi.view(np.uint32), refi.view(np.uint32)):
            bad.append((n, k, T))
        # the counters are zero again after the calls
        if ws.numel() >= 4096:
            assert int(ws[:4096].view(torch.int32).abs().sum()) == 0, (n, k, T)
print("KERNELS", ",".join(sorted(seen)))
print("BAD", bad)
print("WORST", worst)
"""


@pytest.mark.parametrize("waves,kparts,depth,G", [(8, 0, 8, 128), (8, 1, 8, 64), (8, 3, 4, 128),
                                                  (16, 5, 8, 64), (8, 16, 0, 128), (16, 0, 4, 128),
                                                  (8, 1, 0, 128)])
def test_narrow_kernel_shapes_keep_parity(waves, kparts, depth, G):
    """The narrow-layer kernel forced (TERN_TUNE_SMALLT=narrow, and
    TERN_TUNE_GEMV=narrow for T = 1) at T = 1..16 with 4-, 8- and 16-row
    activation tiles, 8- and 16-wave workgroups and K split over 1 to 11
    workgroups (register rings of 4, 8, 12 and 16 k-tiles, requested 4 ahead
    of the one in use, the default, or all up front with TERN_TUNE_DEPTH=8):
    within the gate
    of the oracle on random activations, bit-exact on integer ones, two
    calls per workspace (fresh activations each), and the workspace's
    arrival counters zero after every call."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TERN_TUNE_SMALLT="narrow", TERN_TUNE_GEMV="narrow",
               TERN_TUNE_WAVES=str(waves), TERN_TUNE_KPARTS=str(kparts), TERN_TUNE_DEPTH=str(depth))
    r = subprocess.run([sys.executable, "-c", _NARROW_CHILD, root, str(G)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split("BAD")[1].split("\n")[0].strip() == "[]", r.stdout
    worst = float(r.stdout.split("WORST")[1])
    assert worst <= 1e-6, worst
    assert r.stdout.split("KERNELS")[1].split()[0] == "smallt_narrow", r.stdout


def test_narrow_kernel_graph_replays(tl, torch):
    """The narrow-layer kernel (default above 12 tokens on a short K) captured
    in a graph of four calls on one workspace, replayed three times with the
    program's own work and synchronisations between the replays: every replay
    equals the eager results bit for bit, so the arrival counters start each
    replay at zero (the calls leave them zero) and no call sees another's
    partials."""
    n, k, G = 1024, 4096, 128
    shape = ts.Shape("narrow_graph_4096x1024", k, n, G, 0.4, True, 77)
    wts = ts.weights(shape)
    W = tl.TernaryWeights.from_host(wts.w, wts.s)
    Ts = (16, 13, 16, 14)
    assert all(tl.plan_kernels(T, n, k, G) == ["smallt_narrow"] for T in Ts)
    xs = [to_dev_bf16(torch, ts.activations(wts, T, salt=i)) for i, T in enumerate(Ts)]
    ws = torch.zeros((max(tl.workspace_bytes(T, n, k, G) for T in Ts),), dtype=torch.uint8, device="cuda")
    ys = [torch.empty((T, n), dtype=torch.float32, device="cuda") for T in Ts]
    eager = []
    for x, y in zip(xs, ys):
        tl.linear(x, W, y=y, workspace=ws)
        eager.append(y.clone())
    torch.cuda.synchronize()
    for i, (T, e) in enumerate(zip(Ts, eager)):
        ref = oracle.linear_bf16(ts.activations(wts, T, salt=i), wts.w, wts.s)
        assert rel_l2(e.cpu().numpy(), ref) <= 1e-6
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, y in zip(xs, ys):
                tl.linear(x, W, y=y, workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert torch.equal(y.view(torch.int32), e.view(torch.int32)), rep
        # eager work between the replays, on the same workspace
        tl.linear(xs[0], W, y=ys[0], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(ys[0].view(torch.int32), eager[0].view(torch.int32))
    assert int(ws[:4096].view(torch.int32).abs().sum()) == 0


_S8_SPLIT_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle, tern_synth as ts, ternary_weight_linear_amd as tl
n, k, G = 96, 2560, int(sys.argv[2])
rng = np.random.default_rng(k + G)
w = ts.draw_weights(rng, n, k, 0.4)
s = ts.pow2_scales(n, k, G, seed=11)
W = tl.TernaryWeights.from_host(w, s)
bad = []
for T in (17, 40, 100):
    xb = ts.integer_activations(k, T, seed=T)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    q, sc = oracle.quant_s8(xb)
    ref = oracle.linear_s8(q, sc, w, s)
    y = tl.linear(x, W, rung="s8").cpu().numpy()
    ks = tl.last_kernels()
    assert ks == tl.plan_kernels(T, n, k, G, "s8") == ["quant_s8", "s8_mma", "s8_reduce"], ks
    if not np.array_equal(y.view(np.uint32), ref.view(np.uint32)):
        bad.append(T)
print("BAD", bad)
"""


@pytest.mark.parametrize("kparts,depth,G", [(3, 4, 128), (4, 4, 64), (10, 4, 128), (2, 2, 128)])
def test_s8_k_split_exact(kparts, depth, G):
    """The s8 rung with K split over workgroups (fp32 partials added by a
    second kernel) and the 4-deep pipeline, on integer activations and
    power-of-two scales, where every fp32 sum is exact whatever its order: y
    must equal the oracle bit for bit. 10 k-tiles over 2..10 parts give
    parts shorter than the pipeline and tails of every length."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TERN_TUNE_KPARTS=str(kparts), TERN_TUNE_DEPTH=str(depth))
    r = subprocess.run([sys.executable, "-c", _S8_SPLIT_CHILD, root, str(G)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split("BAD")[1].strip() == "[]", r.stdout


_LIMBTILE_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle, tern_synth as ts, ternary_weight_linear_amd as tl
n, k, G = 96, 2560, int(sys.argv[2])
rng = np.random.default_rng(k + G + 1)
w = ts.draw_weights(rng, n, k, 0.4)
s = ts.pow2_scales(n, k, G, seed=13)
W = tl.TernaryWeights.from_host(w, s)
bad = []
seen = set()
for T in (2, 3, 4, 5, 7, 8):
    xb = ts.integer_activations(k, T, seed=T + 30)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    ref = oracle.linear_bf16(xb, w, s)
    for rung in ("small_t", "small_t_tiled"):
        tl.probe_reset()
        y = tl.linear(x, W, rung=rung).cpu().numpy().astype(np.float64)
        ks = tl.last_kernels()
        assert ks == tl.plan_kernels(T, n, k, G, rung), (T, rung, ks)
        seen.update((T, kn) for kn in ks)
        if not np.array_equal(y, ref):
            bad.append((T, rung))
print("KERNELS", sorted(seen))
print("BAD", bad)
"""


@pytest.mark.parametrize("kernel,strips,waves,depth,G", [
    ("limb", 1, 4, 2, 128), ("limb", 2, 3, 4, 64), ("limb", 1, 8, 4, 128), ("limb", 2, 4, 2, 128),
    ("limb2", 1, 4, 2, 128), ("limb2", 2, 3, 4, 64),
    ("resident", 1, 4, 4, 128), ("resident", 2, 4, 2, 64)])
def test_small_t_limb_path_exact(kernel, strips, waves, depth, G):
    """The small_t limb path (int8 limbs of the activations, int8 MFMA)
    forced for T = 2..8, one and two row blocks, on integer activations and
    power-of-two scales, where the limbs and every fp32 sum are exact: y must
    equal the oracle bit for bit. "limb": up to 4 tokens the loader wave makes
    the limbs, above that a prep kernel does; "limb2": the prep kernel at
    every T. Partial strip blocks (6 strips) and waves without strips
    included."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TERN_TUNE_SMALLT=kernel, TERN_TUNE_STRIPS=str(strips),
               TERN_TUNE_WAVES=str(waves), TERN_TUNE_DEPTH=str(depth))
    r = subprocess.run([sys.executable, "-c", _LIMBTILE_CHILD, root, str(G)], env=env,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.split("BAD")[1].strip() == "[]", r.stdout
    import ast
    seen = ast.literal_eval(r.stdout.split("KERNELS")[1].split("BAD")[0].strip())
    want = {"limb": lambda T: "smallt_limb_fused" if T <= 4 else "smallt_limb_tile",
            "limb2": lambda T: "smallt_limb_tile",
            "resident": lambda T: "smallt_resident"}[kernel]
    for T in (2, 3, 4, 5, 7, 8):
        assert (T, want(T)) in seen, (T, seen)


# ------------------------------------- activation dynamic range (bf16 rungs)


def _range_case(name, T, k, rng):
    if name == "outliers":
        x = rng.standard_normal((T, k)).astype(np.float32)
        x[:, rng.choice(k, 20, replace=False)] *= 1000.0
        x[:, rng.choice(k, 40, replace=False)] *= 1e-5
    elif name == "subnormal":
        # magnitudes around the bf16 subnormal range (2^-133 .. 2^-120)
        x = (rng.standard_normal((T, k)) * 2.0 ** -126).astype(np.float32)
    elif name == "wide":
        # log-uniform over 16 decades, random signs
        x = (10.0 ** rng.uniform(-8, 8, (T, k)) * rng.choice([-1, 1], (T, k))).astype(np.float32)
    elif name == "huge":
        x = (rng.standard_normal((T, k)) * 1e30).astype(np.float32)
    else:
        raise ValueError(name)
    xb = ts.f32_to_bf16_bits(x)
    xb[0, :] = 0  # an all-zero token row
    return xb


@pytest.mark.parametrize("case", ["outliers", "subnormal", "wide", "huge"])
def test_bf16_rungs_activation_range(tl, torch, case):
    """Per-element bound on every bf16-activation rung for activation rows
    with extreme ranges. Products w*x are exact and sums are fp32, so the
    error of each output is a bounded number of fp32 roundings of
    sum_k |s w x| (at most 2^-16 of it here, K = 2048). The gemv kernel
    carries each activation as a 22-bit fixed-point number relative to the
    largest magnitude M of its 256-wide k-tile, which rounds it by at most
    2^-22 * M; that adds sum over k-tiles of 2^-22 * M * sum_{k in tile} |s w|."""
    n, k, G, T = 256, 2048, 128, 3
    rng = np.random.default_rng(["outliers", "subnormal", "wide", "huge"].index(case) + 77)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.draw_scales(rng, n, k, G)
    xb = _range_case(case, T, k, rng)
    W = tl.TernaryWeights.from_host(w, s)
    x_dev = to_dev_bf16(torch, xb)
    ref = oracle.linear_bf16(xb, w, s)
    xf = ts.bf16_bits_to_f32(xb).astype(np.float64)
    sw = np.abs(w.astype(np.float64) * np.repeat(ts.f16_bits_to_f32(s).astype(np.float64), G, axis=1))
    absdot = np.abs(xf) @ sw.T                                   # [T, n]
    tmax = np.abs(xf).reshape(T, k // 256, 256).max(axis=2)     # [T, k-tiles]
    swt = sw.reshape(n, k // 256, 256).sum(axis=2)               # [n, k-tiles]
    bound = 2.0 ** -16 * absdot + 2.0 ** -22 * (tmax @ swt.T)
    for rung in ("gemv", "small_t", "small_t_tiled"):
        y = run(tl, torch, x_dev, W, rung).astype(np.float64)
        assert np.all(np.isfinite(y)), rung
        assert np.all(y[0] == 0), rung
        err = np.abs(y - ref)
        assert np.all(err <= bound), (rung, float((err / np.maximum(bound, 1e-300)).max()))


_LIMB_RANGE_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle, tern_synth as ts, ternary_weight_linear_amd as tl
from tests.test_gpu_parity import _range_case
n, k, G = 96, 2048, 128
worst = 0.0
seen = set()
for ci, case in enumerate(["outliers", "subnormal", "wide", "huge"]):
    rng = np.random.default_rng(ci + 177)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.draw_scales(rng, n, k, G)
    W = tl.TernaryWeights.from_host(w, s)
    for T in (3, 4, 6):
        xb = _range_case(case, T, k, rng)
        ref = oracle.linear_bf16(xb, w, s)
        xf = ts.bf16_bits_to_f32(xb).astype(np.float64)
        sw = np.abs(w.astype(np.float64) * np.repeat(ts.f16_bits_to_f32(s).astype(np.float64), G, axis=1))
        tmax = np.abs(xf).reshape(T, k // 256, 256).max(axis=2)
        swt = sw.reshape(n, k // 256, 256).sum(axis=2)
        bound = 2.0 ** -16 * (np.abs(xf) @ sw.T) + 2.0 ** -22 * (tmax @ swt.T)
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        y = tl.linear(x, W, rung="small_t").cpu().numpy().astype(np.float64)
        seen.update((T, kn) for kn in tl.last_kernels())
        assert np.all(np.isfinite(y)) and np.all(y[0] == 0), (case, T)
        worst = max(worst, float((np.abs(y - ref) / np.maximum(bound, 1e-300)).max()))
print("KERNELS", sorted(seen))
print("WORST", worst)
"""


@pytest.mark.parametrize("kernel", ["limb", "limb2", "resident"])
def test_limb_path_activation_range(kernel):
    """The activation-range bound of test_bf16_rungs_activation_range on the
    small_t limb path (forced): limbs made by the loader wave (T <= 4) or by
    the prep kernel, rows spanning 2^-40..2^40, subnormals, huge values and an
    all-zero token."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, TERN_TUNE_SMALLT=kernel)
    r = subprocess.run([sys.executable, "-c", _LIMB_RANGE_CHILD, root], env=env, capture_output=True,
                       text=True, timeout=240, cwd=root)
    assert r.returncode == 0, r.stderr[-2000:]
    assert float(r.stdout.split("WORST")[1]) <= 1.0, r.stdout
    import ast
    seen = ast.literal_eval(r.stdout.split("KERNELS")[1].split("WORST")[0].strip())
    want = {"limb": {3: "smallt_limb_fused", 4: "smallt_limb_fused", 6: "smallt_limb_tile"},
            "limb2": {3: "smallt_limb_tile", 4: "smallt_limb_tile", 6: "smallt_limb_tile"},
            "resident": {3: "smallt_resident", 4: "smallt_resident", 6: "smallt_resident"}}[kernel]
    for T, kn in want.items():
        assert (T, kn) in seen, (T, seen)


# ------------------------------------- rotated quantisation (1024-wide blocks)


def _rot_inputs(T, K, seed):
    rng = np.random.default_rng(seed)
    xf = rng.standard_normal((T, K)).astype(np.float32)
    xf[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20.0  # fixed outlier channels
    xf[0] = 0.0                 # all-zero token
    if T > 2:
        xf[2] *= 1e-38          # subnormal range
    if T > 3:
        xf[3] *= 1e30           # large, block sums still finite
    return ts.f32_to_bf16_bits(xf)


@pytest.mark.parametrize("K", [1024, 2048, 5120, 17408, 32768])
@pytest.mark.parametrize("layout", ["row_major", "operand_order"])
def test_quant_rot_bit_exact(tl, torch, K, layout):
    """The fused rotate-and-quantise kernel reproduces the oracle's codes and
    scales bit for bit: 1, 2, 5, 17 and 32 blocks per token (1 to 8 blocks
    per wave, ragged over the 4 waves), a zero token, a token in the
    subnormal range, a large one."""
    T = 7
    x = _rot_inputs(T, K, 900 + K // 1024)
    q_ref, s_ref = oracle.quant_s8_rot(x)
    q, sc = tl.quant_act_s8_rot(to_dev_bf16(torch, x), layout=layout)
    torch.cuda.synchronize()
    want = q_ref if layout == "row_major" else operand_order(q_ref)
    assert np.array_equal(q.cpu().numpy(), want)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("shape", [ts.GATE_UP, ts.DOWN])
def test_quant_rot_full_prefill_exact(tl, torch, shape):
    """At the prefill size (T = 2048 tokens of the layer's K, the launch
    configuration the benchmark times) every code and scale is compared."""
    T, K = 2048, shape.k
    x = _rot_inputs(T, K, 77 + K)
    q_ref, s_ref = oracle.quant_s8_rot(x)
    q, sc = tl.quant_act_s8_rot(to_dev_bf16(torch, x), layout="operand_order")
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), operand_order(q_ref))
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_quant_rot_feeds_the_s8_contraction(tl, torch):
    """Rotated codes through the s8 contraction: y within the s8 gate of the
    oracle's exactly rounded s8 output on the same codes."""
    rng = np.random.default_rng(31)
    N, K, G, T = 256, 2048, 128, 40
    w = ts.draw_weights(rng, N, K, 0.4)
    s = ts.draw_scales(rng, N, K, G)
    x = _rot_inputs(T, K, 32)
    q_ref, s_ref = oracle.quant_s8_rot(x)
    y_ref = oracle.linear_s8(q_ref, s_ref, w, s)
    W = tl.TernaryWeights.from_host(w, s)
    q, sc = tl.quant_act_s8_rot(to_dev_bf16(torch, x), layout="operand_order")
    y = tl.linear_s8_q(q, sc, W, layout="operand_order")
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy(), y_ref) <= S8_GATE


def test_quant_rot_rejects_bad_shapes(tl, torch):
    x = torch.zeros((2, 1536), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tl.TernError):
        tl.quant_act_s8_rot(x)
    x = torch.zeros((2, 65536), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tl.TernError):
        tl.quant_act_s8_rot(x)


def _boundary_tokens(T, K, seed):
    """bf16 tokens whose quotients v / scale lie on or near half-integers:
    even tokens have an absmax of 127 * 2^e (scale 2^e exactly, every value
    (k + 1/2) 2^e an exact tie), odd ones a random absmax; the other values
    are the bf16 roundings of (k + 1/2) * scale moved by -2..2 bf16 steps."""
    rng = np.random.default_rng(seed)
    x = np.empty((T, K), np.uint16)
    for t in range(T):
        e = int(rng.integers(-20, 20))
        am = 127.0 * 2.0 ** e if t % 2 == 0 else rng.uniform(0.5, 4.0) * 2.0 ** e
        amb = ts.f32_to_bf16_bits(np.asarray([am], np.float32))[0]
        amf = ts.bf16_bits_to_f32(np.asarray([amb]))[0]
        sc = amf / np.float32(127.0)
        k = rng.integers(-127, 127, K).astype(np.float64)
        v = ts.f32_to_bf16_bits(((k + 0.5) * np.float64(sc)).astype(np.float32))
        v = (v.astype(np.int32) + rng.integers(-2, 3, K) * (t % 2)).astype(np.uint16)
        big = np.abs(ts.bf16_bits_to_f32(v)) > amf
        v[big] = amb
        v[int(rng.integers(0, K))] = amb
        x[t] = v
    return x


@pytest.mark.parametrize("K", [5120, 17408, 65536])
@pytest.mark.parametrize("layout", ["row_major", "operand_order"])
def test_quant_codes_at_rounding_boundaries(tl, torch, K, layout):
    """Quotients on and near half-integers, where a code computed through the
    reciprocal of the scale could differ from the oracle's rounding of the
    IEEE quotient: codes and scales bit-exact at 256 tokens (the launch shapes
    of long batches: 256 threads per token below K = 16384, 512 from there)
    and at 16 (1024 threads per token up to K = 32768)."""
    x = _boundary_tokens(256, K, 5 + K)
    scale = oracle.quant_s8(x)[1].astype(np.float64)
    quot = ts.bf16_bits_to_f32(x).astype(np.float64) / scale[:, None]
    off = np.abs(quot - np.floor(quot) - 0.5)
    assert (off == 0).sum() > 1000 and ((off > 0) & (off < 2.0 ** -15)).sum() > 100
    for T in (256, 16):
        q_ref, s_ref = oracle.quant_s8(x[:T])
        q, sc = tl.quant_act_s8(to_dev_bf16(torch, x[:T]), layout=layout)
        torch.cuda.synchronize()
        want = q_ref if layout == "row_major" else operand_order(q_ref)
        assert np.array_equal(q.cpu().numpy(), want)
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


# ------------------------------------------- environment arms on the GPU

_ARM_CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle, tern_synth as ts, ternary_weight_linear_amd as tl
shape = ts.Shape("arm_768x2048", 768, 2048, 128, 0.4, True, 611)
wts = ts.weights(shape)
W = tl.TernaryWeights.from_host(wts.w, wts.s)
out = []
for T in (1, 5, 12, 20):
    xb = ts.activations(wts, T)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    rung = tl.resolve_rung(T)
    tl.probe_reset()
    y = tl.linear(x, W).cpu().numpy()
    snap = tl.probe_snapshot()
    assert snap[rung] == 1 and sum(snap.values()) == 1, (T, snap)
    ks = tl.last_kernels()
    assert ks == tl.plan_kernels(T, W.n, W.k, W.group), (T, ks)
    kp = {k: v for k, v in tl.kernel_probe_snapshot().items() if v}
    assert kp == {k: 1 for k in ks}, (T, kp)
    if rung == "s8":
        q, sc = oracle.quant_s8(xb)
        err = np.linalg.norm(y - oracle.linear_s8(q, sc, wts.w, wts.s)) / np.linalg.norm(
            oracle.linear_s8(q, sc, wts.w, wts.s).astype(np.float64))
        ok = err <= 1e-6
    else:
        ref = oracle.linear_bf16(xb, wts.w, wts.s)
        ok = np.linalg.norm(y - ref) / np.linalg.norm(ref) <= 2e-3
    out.append(f"{T}:{rung}:{'+'.join(ks)}:{'ok' if ok else 'BAD'}")
print("ARMS", " ".join(out))
"""


@pytest.mark.parametrize("env,expect", [
    ({}, "gemv small_t small_t_tiled s8"),
    ({"TERN_RUNG": "gemv"}, "gemv gemv gemv gemv"),
    ({"TERN_RUNG": "small_t"}, None),  # T = 20 is beyond one 16-token tile: an error, tested below
    ({"TERN_RUNG": "small_t_tiled"}, "small_t_tiled small_t_tiled small_t_tiled small_t_tiled"),
    ({"TERN_RUNG": "s8"}, "s8 s8 s8 s8"),
    ({"TERN_S8": "0"}, "gemv small_t small_t_tiled small_t_tiled"),
    ({"TERN_SMALL_T_TILED_MAX": "10"}, "gemv small_t s8 s8"),
    ({"TERN_SMALL_T_MAX": "16"}, "gemv small_t small_t s8")])
def test_env_arms_run_on_the_gpu(env, expect):
    """One binary, every rung forced by the environment in a process of its
    own: the auto-dispatched calls run the forced rung (rung probe), the
    kernels the dry run names (kernel probe), and stay within their gates
    ("NINFER ternary perf-tuning" notes, section 3: arms toggled by env)."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _ARM_CHILD, root], env=dict(os.environ, **env),
                       capture_output=True, text=True, timeout=240)
    if expect is None:
        assert r.returncode != 0 and "TERN_ERR_RUNG" in r.stderr, r.stderr[-2000:]
        return
    assert r.returncode == 0, r.stderr[-2000:]
    arms = r.stdout.split("ARMS")[1].split()
    assert [a.split(":")[1] for a in arms] == expect.split(), arms
    assert all(a.endswith(":ok") for a in arms), arms
    if env.get("TERN_S8") == "0":
        assert arms[3].split(":")[2] == "b16_prefill", arms


@pytest.mark.parametrize("n,k,T", [(16384, 10752, 4), (16384, 13824, 5), (16384, 7680, 6)])
def test_resident_limbs_with_g64_on_wide_layers(tl, torch, n, k, T):
    """Wide layers with a long K and G = 64, where the resident limb kernel's
    scales take twice the LDS they take at G = 128: the dispatcher sizes the
    plan with the call's group size, so the call runs (no launch error) and,
    on integer activations with power-of-two scales, matches the oracle bit
    for bit on sampled rows of every workgroup."""
    G = 64
    rng = np.random.default_rng(n + k + T)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.pow2_scales(n, k, G, seed=k)
    W = tl.TernaryWeights.from_host(w, s)
    xbits = ts.integer_activations(k, T, seed=k + T)
    print("resident G=64", n, k, T, tl.plan_kernels(T, n, k, G), flush=True)
    y = run(tl, torch, to_dev_bf16(torch, xbits), W, "auto")
    rows = sample_rows(n, k, n=256)
    ref = oracle.linear_bf16(xbits, w[rows], s[rows])
    assert np.array_equal(y[:, rows].astype(np.float64), ref)


@pytest.fixture(scope="module")
def qkv(tl, torch):
    """The fused q|k|v matrix (three 5120 -> 5120 projections stacked along
    N: 5120 -> 15360) as the bench's fused stack times it, from the stack's
    layer-0 seeds."""
    parts = [ts.weights(ts.stack_shape(0, p)) for p in range(3)]
    w = np.concatenate([p.w for p in parts])
    s = np.concatenate([p.s for p in parts])
    return parts[0], w, s, tl.TernaryWeights.from_host(w, s)


def test_fused_qkv_decode_every_output(tl, torch, qkv):
    wq, w, s, W = qkv
    xbits = ts.activations(wq, 1)
    y = run(tl, torch, to_dev_bf16(torch, xbits), W, "auto")
    ref = oracle.linear_bf16(xbits, w, s)
    assert rel_l2(y, ref) <= 1e-6


@pytest.mark.parametrize("rung", ["s8", "small_t_tiled"])
def test_fused_qkv_prefill_chunk_sampled(tl, torch, qkv, rung):
    """A 1024-token prefill chunk on the fused q|k|v matrix, s8 and the bf16
    prefill, on sampled rows."""
    wq, w, s, W = qkv
    T = 1024
    xbits = ts.activations(wq, T)
    x_dev = to_dev_bf16(torch, xbits)
    rows = sample_rows(W.n, 1024 + len(rung))
    y = run(tl, torch, x_dev, W, rung)
    if rung == "s8":
        check_s8(tl, torch, xbits, x_dev, W, w, s, y, rows=rows)
    else:
        ref = oracle.linear_bf16(xbits, w[rows], s[rows])
        assert rel_l2(y[:, rows], ref) <= 1e-6


# ------------------------------------------------------ base-3 layout t5


@pytest.mark.parametrize("n,k,G", [(64, 1024, 128), (128, 2048, 64), (16 * 1100, 1024, 128),
                                   (16 * 2176, 5120, 128), (5120, 17408, 128)])
def test_t5_gemv_exact(tl, torch, n, k, G):
    """The gemv on base-3 weights: integer activations and power-of-two
    scales make every step exact, so y must equal the oracle bit for bit;
    narrow (K split over waves) and wide plans, a ragged last workgroup,
    both group sizes. Rows sampled on the two large shapes."""
    rng = np.random.default_rng(n + k + G)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.pow2_scales(n, k, G, seed=n + 3)
    W = tl.TernaryWeights.from_host(w, s, layout="t5")
    xbits = ts.integer_activations(k, 1, seed=k + 9)
    print("t5 gemv", n, k, G, flush=True)
    y = run(tl, torch, to_dev_bf16(torch, xbits), W, "auto")
    assert tl.last_kernels() == ["gemv_t5"]
    rows = np.arange(n) if n * k <= 64 * 2**20 else sample_rows(n, n, n=256)
    ref = oracle.linear_bf16(xbits, w[rows], s[rows])
    assert np.array_equal(y[:, rows].astype(np.float64), ref)


@pytest.mark.parametrize("shape", [ts.GATE_UP, ts.DOWN])
def test_t5_gemv_decode_full_rows(tl, torch, big, shape):
    """Decode at T = 1 from t5 weights on the 27B-class shapes: every output
    within the gate (and within 1e-6 of the fp64 oracle, as the 2-bit gemv)."""
    wts, _ = big(shape)
    W = tl.TernaryWeights.from_host(wts.w, wts.s, layout="t5")
    xbits = ts.activations(wts, 1)
    y = run(tl, torch, to_dev_bf16(torch, xbits), W, "gemv")
    ref = oracle.linear_bf16(xbits, wts.w, wts.s)
    assert rel_l2(y, ref) <= 1e-6
    del W


@pytest.mark.parametrize("case", ["outliers", "subnormal", "wide", "huge"])
def test_t5_gemv_activation_range(tl, torch, case):
    """The per-element bound of test_bf16_rungs_activation_range for the t5
    gemv (the same 22-bit fixed point per k-tile)."""
    n, k, G, T = 256, 2048, 128, 1
    rng = np.random.default_rng(["outliers", "subnormal", "wide", "huge"].index(case) + 91)
    w = ts.draw_weights(rng, n, k, 0.4)
    s = ts.draw_scales(rng, n, k, G)
    xb = _range_case(case, 2, k, rng)[1:2].copy()
    W = tl.TernaryWeights.from_host(w, s, layout="t5")
    ref = oracle.linear_bf16(xb, w, s)
    xf = ts.bf16_bits_to_f32(xb).astype(np.float64)
    sw = np.abs(w.astype(np.float64) * np.repeat(ts.f16_bits_to_f32(s).astype(np.float64), G, axis=1))
    tmax = np.abs(xf).reshape(T, k // 256, 256).max(axis=2)
    swt = sw.reshape(n, k // 256, 256).sum(axis=2)
    bound = 2.0 ** -16 * (np.abs(xf) @ sw.T) + 2.0 ** -22 * (tmax @ swt.T)
    y = run(tl, torch, to_dev_bf16(torch, xb), W, "gemv").astype(np.float64)
    assert np.all(np.isfinite(y))
    assert np.all(np.abs(y - ref) <= bound), float((np.abs(y - ref) / np.maximum(bound, 1e-300)).max())
    # an all-zero row gives zeros
    z = run(tl, torch, to_dev_bf16(torch, np.zeros((1, k), np.uint16)), W, "gemv")
    assert np.all(z == 0)


def test_binding_rejects_mismatched_buffers(tl, torch, small):
    """The library takes raw pointers; the binding checks every buffer's
    shape and device before a call, so none is read or written past its end."""
    wts, W = small
    x = to_dev_bf16(torch, ts.activations(wts, 4))
    with pytest.raises(ValueError):
        tl.linear(x, W, y=torch.empty((3, W.n), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        tl.linear(x, W, y=torch.empty((4, W.n - 16), dtype=torch.float32, device="cuda"))
    with pytest.raises((ValueError, TypeError)):
        tl.linear(x, W, workspace=torch.zeros((1 << 20,), dtype=torch.uint8))  # host memory
    with pytest.raises(ValueError):
        tl.quant_act_s8(x, q=torch.empty((4, W.k - 64), dtype=torch.int8, device="cuda"))
    with pytest.raises(ValueError):
        tl.quant_act_s8(x, scale=torch.empty((3,), dtype=torch.float32, device="cuda"))
    q, sc = tl.quant_act_s8(x)
    with pytest.raises(ValueError):
        tl.linear_s8_q(q, sc[:3], W)
    with pytest.raises(ValueError):
        tl.debug_s8_acc(q, W, acc=torch.empty((4, W.n, 1), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
