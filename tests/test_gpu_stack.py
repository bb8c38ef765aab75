"""The 64-layer linear stack: q, k, v, o (5120 -> 5120), gate and up
(5120 -> 17408) and down (17408 -> 5120) per layer, per-layer seeds, run as a
T = 1 decode pass and as a 2048-token prefill in chunks of 1024 tokens.

Three layers (first, middle, last) are checked, all seven projections each:
the decode call on every output (gemv rung), the prefill chunks (s8 rung) on
sampled output rows, which the oracle computes exactly row by row.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tern_synth as ts

pytestmark = pytest.mark.gpu

LAYERS = (0, 31, 63)


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
    return np.linalg.norm(y - ref) / np.linalg.norm(ref)


@pytest.mark.parametrize("layer", LAYERS)
@pytest.mark.parametrize("proj", range(len(ts.STACK_PROJ)))
def test_stack_layer(tl, torch, layer, proj):
    shape = ts.stack_shape(layer, proj)
    wts = ts.weights(shape)
    W = tl.TernaryWeights.from_host(wts.w, wts.s)
    # decode, T = 1: every output
    x1 = ts.activations(wts, 1)
    y1 = tl.linear(torch.from_numpy(x1.view(np.int16)).cuda().view(torch.bfloat16), W)
    torch.cuda.synchronize()
    assert tl.last_rung() == "gemv"
    ref1 = oracle.linear_bf16(x1, wts.w, wts.s)
    err = rel_l2(y1.cpu().numpy(), ref1)
    assert err <= 2e-3 and err <= 1e-6, err
    # prefill: 2048 tokens in two chunks of 1024 (s8 rung), sampled rows
    xp = ts.activations(wts, 2048)
    rng = np.random.default_rng([shape.seed, 9])
    rows = np.unique(np.concatenate([rng.choice(shape.n, 48, replace=False), [0, shape.n - 1]]))
    for c in range(2):
        xc = np.ascontiguousarray(xp[1024 * c:1024 * (c + 1)])
        yc = tl.linear(torch.from_numpy(xc.view(np.int16)).cuda().view(torch.bfloat16), W)
        torch.cuda.synchronize()
        assert tl.last_rung() == "s8"
        q, sc = oracle.quant_s8(xc)
        yr = yc.cpu().numpy()[:, rows]
        ref = oracle.linear_s8(q, sc, wts.w[rows], wts.s[rows])
        assert rel_l2(yr, ref) <= 1e-6
        ordered = oracle.linear_s8_fp32_ordered(q, sc, wts.w[rows], wts.s[rows])
        assert np.array_equal(yr.view(np.uint32), ordered.view(np.uint32))
