"""The persistent decode chain (tern_linear_chain) on the GPU: every
projection's y bit for bit equal to tern_linear's gemv rung on the same
inputs, with independent inputs, with a real dependency chain (each x the
bf16-rounded y of the projection before, as computed by sequential
tern_linear calls), on three layers of the 64-layer stack with the stack's
dependency structure, and a forced give-up of the bounded wait."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tern_synth as ts

pytestmark = pytest.mark.gpu


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


def dev_bf16(torch, xbits):
    return torch.from_numpy(xbits.view(np.int16)).cuda().view(torch.bfloat16)


def test_chain_independent_items_match_gemv(tl, torch):
    shapes = [ts.Shape("c0", 256, 128, 128, 0.4, True, 901), ts.Shape("c1", 1024, 4096, 128, 0.4, True, 902),
              ts.OUT_PROJ, ts.Shape("c3", 2048, 16 * 1100, 128, 0.4, True, 904), ts.DOWN]
    items, refs = [], []
    for sh in shapes:
        w = ts.weights(sh)
        W = tl.TernaryWeights.from_host(w.w, w.s)
        x = dev_bf16(torch, ts.activations(w, 1))
        y = torch.full((1, sh.n), float("nan"), device="cuda")
        items.append((W, x, y, None, -1))
        refs.append(tl.linear(x, W))
    ch = tl.Chain(items)
    tl.probe_reset()
    ch.run()
    torch.cuda.synchronize()
    assert tl.last_kernels() == ["chain"] and not ch.failed()
    for (W, x, y, _, _), ref in zip(items, refs):
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), W.n


def test_chain_dependent_projections(tl, torch):
    """x of item i is item i-1's y rounded to bf16 inside the kernel: o
    (5120 -> 5120), gate (5120 -> 17408), down (17408 -> 5120), o again."""
    shapes = [ts.stack_shape(0, 3), ts.stack_shape(0, 4), ts.stack_shape(0, 6), ts.stack_shape(1, 3)]
    ws = [ts.weights(sh) for sh in shapes]
    Ws = [tl.TernaryWeights.from_host(w.w, w.s) for w in ws]
    x0 = dev_bf16(torch, ts.activations(ws[0], 1))
    ys = [torch.empty((1, W.n), device="cuda") for W in Ws]
    ybs = [torch.empty((1, W.n), dtype=torch.bfloat16, device="cuda") for W in Ws]
    items = [(Ws[0], x0, ys[0], ybs[0], -1)] + [(Ws[i], ybs[i - 1], ys[i], ybs[i], i - 1) for i in range(1, 4)]
    ch = tl.Chain(items)
    for rep in range(3):  # counters left zeroed: every launch waits correctly
        for y in ys:
            y.fill_(float("nan"))
        ch.run()
        torch.cuda.synchronize()
        assert not ch.failed(), rep
        x = x0
        for i, W in enumerate(Ws):
            ref = tl.linear(x, W)
            assert torch.equal(ys[i].view(torch.int32), ref.view(torch.int32)), (rep, i)
            assert torch.equal(ybs[i].view(torch.int16), ref.to(torch.bfloat16).view(torch.int16)), (rep, i)
            x = ref.to(torch.bfloat16)
    # the first stage against the oracle as well
    ref = oracle.linear_bf16(ts.activations(ws[0], 1), ws[0].w, ws[0].s)
    err = np.linalg.norm(ys[0].cpu().numpy() - ref) / np.linalg.norm(ref)
    assert err <= 1e-6


def stack_items(tl, torch, layers):
    """The 7 projections of each layer with the stack's dependencies (q, k, v
    after the previous layer's down; o after v; gate and up after o; down
    after up); every projection its own synthetic x, as the stack is run."""
    items, info = [], []
    for li in layers:
        base = len(items)
        for p in range(7):
            sh = ts.stack_shape(li, p)
            w = ts.weights(sh)
            W = tl.TernaryWeights.from_host(w.w, w.s)
            xb = ts.activations(w, 1)
            x = dev_bf16(torch, xb)
            y = torch.full((1, sh.n), float("nan"), device="cuda")
            after = {0: base - 1, 1: base - 1, 2: base - 1, 3: base + 2, 4: base + 3, 5: base + 3, 6: base + 5}[p]
            items.append((W, x, y, None, after))
            info.append((w, xb))
    return items, info


def test_chain_three_stack_layers(tl, torch):
    items, info = stack_items(tl, torch, (0, 31, 63))
    ch = tl.Chain(items)
    ch.run()
    torch.cuda.synchronize()
    assert not ch.failed()
    for (W, x, y, _, _), (w, xb) in zip(items, info):
        ref = tl.linear(x, W)
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), W.n
        rows = np.random.default_rng(W.n).choice(W.n, 64, replace=False)
        r = oracle.linear_bf16(xb, w.w[rows], w.s[rows])
        got = y.cpu().numpy()[:, rows]
        assert np.linalg.norm(got - r) / np.linalg.norm(r) <= 1e-6


def test_chain_wait_gives_up_and_exits(tl, torch):
    """A one-poll spin limit on a wait whose producer takes microseconds: the
    waiting workgroups give up, set the flag and skip the rest; the kernel
    exits, the counters are left zeroed, and the next run with a normal limit
    is correct."""
    sh0 = ts.Shape("g0", 17408, 16, 128, 0.4, True, 911)    # one unit: one workgroup works, all others wait
    sh1 = ts.Shape("g1", 1024, 2048, 128, 0.4, True, 912)
    w0, w1 = ts.weights(sh0), ts.weights(sh1)
    W0, W1 = tl.TernaryWeights.from_host(w0.w, w0.s), tl.TernaryWeights.from_host(w1.w, w1.s)
    x0, x1 = dev_bf16(torch, ts.activations(w0, 1)), dev_bf16(torch, ts.activations(w1, 1))
    y0, y1 = torch.empty((1, 16), device="cuda"), torch.empty((1, 2048), device="cuda")
    ch = tl.Chain([(W0, x0, y0, None, -1), (W1, x1, y1, None, 0)])
    ch.run(spin_limit=1)
    torch.cuda.synchronize()
    assert ch.failed()
    assert int(ch.counters.abs().sum().item()) == 0
    ch.error_flag.zero_()
    ch.run()
    torch.cuda.synchronize()
    assert not ch.failed()
    assert torch.equal(y1.view(torch.int32), tl.linear(x1, W1).view(torch.int32))


def test_chain_fresh_inputs_each_launch(tl, torch):
    """Chained projections with two items in one stage (both reading the
    first item's output, like k and v beside q) and a third reading one of
    them; x0 changes before every launch, so a read of an earlier launch's
    (stale) values would show: every stage bit-identical to tern_linear on
    that launch's inputs."""
    shapes = [ts.stack_shape(2, 3), ts.stack_shape(2, 0), ts.stack_shape(2, 4), ts.stack_shape(2, 6)]
    ws = [ts.weights(sh) for sh in shapes]
    Ws = [tl.TernaryWeights.from_host(w.w, w.s) for w in ws]
    x0 = torch.empty((1, Ws[0].k), dtype=torch.bfloat16, device="cuda")
    ys = [torch.empty((1, W.n), device="cuda") for W in Ws]
    ybs = [torch.empty((1, W.n), dtype=torch.bfloat16, device="cuda") for W in Ws]
    srcs = [x0, ybs[0], ybs[0], ybs[2]]
    afters = [-1, 0, 0, 2]
    ch = tl.Chain([(Ws[i], srcs[i], ys[i], ybs[i], afters[i]) for i in range(4)])
    for rep in range(4):
        x0.copy_(dev_bf16(torch, ts.activations(ws[0], 1, salt=rep + 7)))
        ch.run()
        torch.cuda.synchronize()
        assert not ch.failed(), rep
        refs = []
        for i, W in enumerate(Ws):
            src = x0 if i == 0 else refs[afters[i]].to(torch.bfloat16)
            refs.append(tl.linear(src, W))
            assert torch.equal(ys[i].view(torch.int32), refs[i].view(torch.int32)), (rep, i)
