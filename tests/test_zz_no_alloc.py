"""tern_linear_noalloc: the entry point for callers that cannot allocate,
with its workspace in the library's static device scratch. Called through the
raw C ABI and held bit for bit to tern_linear with a caller workspace (the
same kernels), on two calls in a row per case, the second with a smaller
input (the scratch keeps the first call's contents)."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

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


def _noalloc(tl, torch, x, W, y, rung):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return tl.lib().tern_linear_noalloc(x.data_ptr(), x.shape[0], W.ref(), y.data_ptr(),
                                        tl.RUNG_ID[rung], stream)


# (layer, rung, first T, second T): the rungs and kernels that use a
# workspace -- s8 with and without a K split, the narrow-layer kernel's K-split
# partials and the arrival counters in the scratch's header -- and one that
# uses none.
CASES = [
    (ts.OUT_PROJ, "s8", 508, 40),         # unsplit, then split K (partials)
    (ts.DOWN, "small_t_tiled", 12, 9),    # narrow-layer kernel, K split over workgroups
    (ts.GATE_UP, "s8", 2048, 17),         # 10.5 MB of codes in the scratch, then a short prefill
    (ts.SMALL, "auto", 20, 1),            # s8, then the gemv (no workspace)
]


@pytest.mark.parametrize("shape,rung,t1,t2", CASES, ids=[f"{c[0].name}-{c[1]}" for c in CASES])
def test_noalloc_matches_tern_linear(tl, torch, shape, rung, t1, t2):
    wts = ts.weights(shape)
    W = tl.TernaryWeights.from_host(wts.w, wts.s)
    for T in (t1, t2):
        print("noalloc", shape.name, rung, "T", T, flush=True)
        xb = ts.activations(wts, T)
        x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        y = torch.full((T, W.n), float("nan"), dtype=torch.float32, device="cuda")
        assert _noalloc(tl, torch, x, W, y, rung) == 0, tl.lib().tern_last_error()
        kernels = tl.last_kernels()
        y_ref = tl.linear(x, W, rung=rung)
        torch.cuda.synchronize()
        assert kernels == tl.last_kernels() == tl.plan_kernels(T, W.n, W.k, W.group, rung)
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), (shape.name, rung, T)


def test_noalloc_rejects_calls_beyond_the_scratch(tl, torch):
    """The s8 rung at T = 4096 on K = 17408 needs 71 MB of workspace, more than
    the 64 MiB scratch: refused before any launch."""
    n, k, T = 5120, 17408, 4096
    assert tl.workspace_bytes(T, n, k, 128, "s8") > tl.NOALLOC_SCRATCH_BYTES
    W = tl._Weights(0x100000, 0x200000, n, k, 128, tl.LAYOUT_V1)
    tl.probe_reset()
    st = tl.lib().tern_linear_noalloc(0x400000, T, ctypes.byref(W), 0x300000, tl.RUNG_ID["s8"], None)
    assert tl.STATUS[st] == "TERN_ERR_WORKSPACE"
    assert "static scratch" in tl.lib().tern_last_error().decode()
    assert all(v == 0 for v in tl.kernel_probe_snapshot().values())
