"""Python binding of ``libtern.so``, the MI355X ternary-weight linear layer.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels (gfx950). PyTorch provides device memory and the current stream.
The binding fails loudly if the library has not been built; there is no CPU
fallback.

Entry points mirror the C ABI in ``include/tern.h``:

* ``pack`` / ``unpack``        -- offline relayout to packed layout v1 (host)
* ``TernaryWeights``           -- packed codes + scales resident on the GPU
* ``quant_act_s8``             -- per-token int8 activation quantisation
* ``quant_act_s8_rot``         -- the same after a blockwise (1024) Hadamard rotation
* ``linear``                   -- ``y = ternary_linear(x)`` with rung dispatch
* ``linear_s8_q``              -- the s8 contraction on pre-quantised activations
* ``debug_s8_acc``             -- the s8 rung's int32 group accumulators
* ``probe_snapshot`` / ``probe_reset`` / ``last_rung`` / ``resolve_rung``
* ``kernel_probe_snapshot`` / ``last_kernels`` -- which kernels ran

Streams: every device call enqueues on ``stream`` (default: the current
stream). Tensors the binding allocates for such a call (outputs, workspace)
are recorded on that stream when it is not the current one, so the caching
allocator does not hand their memory to other work before the call's kernels
are done with it.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtern.so")

RUNGS = ("auto", "gemv", "small_t", "small_t_tiled", "s8")
RUNG_ID = {name: i for i, name in enumerate(RUNGS)}
LAYOUT_V1 = 0x54524E31
LAYOUT_T5 = 0x54524E35
LAYOUTS = {"v1": LAYOUT_V1, "t5": LAYOUT_T5}

STATUS = {0: "TERN_OK", 1: "TERN_ERR_NULL", 2: "TERN_ERR_SHAPE", 3: "TERN_ERR_ALIGN",
          4: "TERN_ERR_VALUE", 5: "TERN_ERR_RUNG", 6: "TERN_ERR_WORKSPACE", 7: "TERN_ERR_CONFIG",
          8: "TERN_ERR_HIP", 9: "TERN_ERR_LAYOUT"}

# Kernel ids of the kernel probe, in the order of tern_kernel in tern.h.
KERNELS = ("quant_s8", "quant_s8_row", "quant_s8_rot", "gemv_limb", "gemv_bf16",
           "smallt_resident", "smallt_limb_fused", "smallt_limb_prep", "smallt_limb_tile",
           "smallt_wave", "smallt_tile", "smallt_tile_reduce", "b16_prefill", "s8_mma",
           "s8_reduce", "s8_row", "s8_acc_export", "stream_read", "gemv_t5", "chain",
           "smallt_narrow")

# Symbols declared in include/tern.h (checked by the host tests).
EXPORTS = ("tern_packed_code_bytes", "tern_scale_count", "tern_pack", "tern_unpack",
           "tern_quant_act_s8", "tern_quant_act_s8_rot", "tern_workspace_bytes", "tern_linear", "tern_linear_s8_q",
           "tern_debug_s8_acc", "tern_stream_read",
           "tern_probe_snapshot", "tern_probe_reset", "tern_last_rung", "tern_resolve_rung",
           "tern_rung_name", "tern_last_error", "tern_abi_version",
           "tern_kernel_probe_snapshot", "tern_last_kernels", "tern_kernel_name",
           "tern_plan_kernels", "tern_linear_noalloc", "tern_packed_code_bytes_t5", "tern_pack_t5",
           "tern_unpack_t5", "tern_chain_table_bytes", "tern_chain_counter_bytes", "tern_chain_build",
           "tern_linear_chain")


class TernError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class _Weights(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("n", ctypes.c_int32),
                ("k", ctypes.c_int32), ("group", ctypes.c_int32), ("layout", ctypes.c_uint32)]


class _ChainItem(ctypes.Structure):
    _fields_ = [("W", _Weights), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("y_bf16", ctypes.c_void_p), ("after", ctypes.c_int32)]


class _ChainPlan(ctypes.Structure):
    _fields_ = [("count", ctypes.c_int32), ("group", ctypes.c_int32), ("workgroups", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("waits", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libtern.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m ternary_weight_linear_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    p, i, sz, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_int
    sig = {
        "tern_packed_code_bytes": (sz, [i, i]),
        "tern_scale_count": (sz, [i, i, i]),
        "tern_pack": (st, [p, p, i, i, i, p, p]),
        "tern_unpack": (st, [p, p, i, i, i, p, p]),
        "tern_quant_act_s8": (st, [p, i, i, p, p, i, p]),
        "tern_quant_act_s8_rot": (st, [p, i, i, p, p, i, p]),
        "tern_workspace_bytes": (sz, [i, i, i, i, i]),
        "tern_linear": (st, [p, i, ctypes.POINTER(_Weights), p, i, p, sz, p]),
        "tern_linear_s8_q": (st, [p, p, i, ctypes.POINTER(_Weights), p, i, p]),
        "tern_debug_s8_acc": (st, [p, i, ctypes.POINTER(_Weights), p, i, p]),
        "tern_stream_read": (st, [p, sz, i, i, p, p]),
        "tern_probe_snapshot": (None, [p]),
        "tern_probe_reset": (None, []),
        "tern_last_rung": (i, []),
        "tern_resolve_rung": (i, [i, i]),
        "tern_rung_name": (ctypes.c_char_p, [i]),
        "tern_last_error": (ctypes.c_char_p, []),
        "tern_abi_version": (i, []),
        "tern_kernel_probe_snapshot": (None, [p]),
        "tern_last_kernels": (ctypes.c_uint64, []),
        "tern_kernel_name": (ctypes.c_char_p, [i]),
        "tern_plan_kernels": (ctypes.c_uint64, [i, i, i, i, ctypes.c_uint32, i]),
        "tern_packed_code_bytes_t5": (sz, [i, i]),
        "tern_pack_t5": (st, [p, p, i, i, i, p, p]),
        "tern_unpack_t5": (st, [p, p, i, i, i, p, p]),
        "tern_linear_noalloc": (st, [p, i, ctypes.POINTER(_Weights), p, i, p]),
        "tern_chain_table_bytes": (sz, [ctypes.POINTER(_ChainItem), i]),
        "tern_chain_counter_bytes": (sz, [i]),
        "tern_chain_build": (st, [ctypes.POINTER(_ChainItem), i, p, sz, ctypes.POINTER(_ChainPlan)]),
        "tern_linear_chain": (st, [ctypes.POINTER(_ChainPlan), p, p, sz, p, i, p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise TernError(status, lib().tern_last_error().decode())


def _rung(r) -> int:
    if isinstance(r, str):
        if r not in RUNG_ID:
            raise ValueError(f"unknown rung {r!r}; expected one of {RUNGS}")
        return RUNG_ID[r]
    return int(r)


# ------------------------------------------------------------------- host


def pack(w: np.ndarray, scales: np.ndarray, layout: str = "v1"):
    """Relayout int8 weights [N, K] and fp16 scales [N, K/G] (uint16 bits or
    float16) to packed layout v1 (2 bits per weight) or t5 (base-3, five per
    byte). Returns (codes uint8, scales uint16 [N*K/G])."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    scales = np.ascontiguousarray(scales)
    if scales.dtype == np.float16:
        scales = scales.view(np.uint16)
    if scales.dtype != np.uint16:
        raise TypeError("scales must be float16 or uint16 bit patterns")
    n, k = w.shape
    if scales.ndim != 2 or scales.shape[0] != n or scales.shape[1] == 0 or k % scales.shape[1]:
        raise ValueError(f"scales shape {scales.shape} does not match w {w.shape}")
    group = k // scales.shape[1]
    t5 = {"v1": False, "t5": True}[layout]
    nbytes = (lib().tern_packed_code_bytes_t5 if t5 else lib().tern_packed_code_bytes)(n, k)
    codes = np.empty(max(nbytes, 1), np.uint8)
    sp = np.empty(scales.size, np.uint16)
    _check((lib().tern_pack_t5 if t5 else lib().tern_pack)(
        w.ctypes.data, scales.ctypes.data, n, k, group, codes.ctypes.data, sp.ctypes.data))
    return codes[:nbytes], sp


def unpack(codes: np.ndarray, scales_packed, n: int, k: int, group: int, layout: str = "v1"):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    fn = {"v1": lib().tern_unpack, "t5": lib().tern_unpack_t5}[layout]
    w = np.empty((n, k), np.int8)
    if scales_packed is None:
        _check(fn(codes.ctypes.data, None, n, k, group, w.ctypes.data, None))
        return w, None
    sp = np.ascontiguousarray(scales_packed, dtype=np.uint16)
    s = np.empty((n, k // group), np.uint16)
    _check(fn(codes.ctypes.data, sp.ctypes.data, n, k, group, w.ctypes.data, s.ctypes.data))
    return w, s


def workspace_bytes(T: int, n: int, k: int, group: int, rung="auto") -> int:
    v = lib().tern_workspace_bytes(T, n, k, group, _rung(rung))
    if v == ctypes.c_size_t(-1).value:
        raise TernError(5, lib().tern_last_error().decode())
    return v


def resolve_rung(T: int, rung="auto") -> str:
    r = lib().tern_resolve_rung(T, _rung(rung))
    if r < 0:
        raise TernError(-r, lib().tern_last_error().decode())
    return RUNGS[r]


def probe_snapshot() -> dict:
    arr = (ctypes.c_uint64 * len(RUNGS))()
    lib().tern_probe_snapshot(arr)
    return {RUNGS[i]: int(arr[i]) for i in range(1, len(RUNGS))}


def probe_reset() -> None:
    lib().tern_probe_reset()


def last_rung() -> str:
    return RUNGS[lib().tern_last_rung()]


def kernel_probe_snapshot() -> dict:
    """Launches per kernel (name -> count) since the last probe_reset()."""
    arr = (ctypes.c_uint64 * len(KERNELS))()
    lib().tern_kernel_probe_snapshot(arr)
    return {KERNELS[i]: int(arr[i]) for i in range(len(KERNELS))}


def _names(mask: int) -> list:
    return [KERNELS[i] for i in range(len(KERNELS)) if mask >> i & 1]


def last_kernels() -> list:
    """Names of the kernels the last successful call on this thread launched."""
    return _names(lib().tern_last_kernels())


def plan_kernels(T: int, n: int, k: int, group: int, rung="auto", layout="v1") -> list:
    """Names of the kernels linear() would launch for this call on weights of
    `layout` ("v1" or "t5"): a host-only dry run of the dispatcher."""
    m = lib().tern_plan_kernels(T, n, k, group, LAYOUTS[layout], _rung(rung))
    if m == 0:
        raise TernError(5, lib().tern_last_error().decode())
    return _names(m)


# ----------------------------------------------------------------- device


def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _side_stream(stream):
    """The torch stream object of `stream` when it is not the current stream
    (None when the call runs on the current stream)."""
    if stream is None:
        return None
    torch = _torch()
    s = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return None
    return s


def _on(stream):
    """Context for the binding's own allocations: the launch stream when it is
    not the current one, so that the caching allocator ties each block to the
    stream that uses it and a zero fill runs before the launch on that stream
    (an allocation on the current stream could be handed out again, or still
    be filling, while the launch stream reads it)."""
    s = _side_stream(stream)
    return contextlib.nullcontext() if s is None else _torch().cuda.stream(s)


def _dev(t, dtype, name, shape=None, device=None):
    """Checks a device tensor argument: HIP, dtype, contiguous, and (when
    given) its exact shape and device. The library takes raw pointers, so a
    buffer smaller than the call needs would be read or written past its end."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t


class TernaryWeights:
    """Packed ternary weights resident on the GPU (layout "v1" or "t5")."""

    def __init__(self, codes, scales, n: int, k: int, group: int, layout: str = "v1"):
        torch = _torch()
        self.codes = _dev(codes, torch.uint8, "codes")
        self.scales = _dev(scales, torch.int16, "scales")
        self.n, self.k, self.group = int(n), int(k), int(group)
        self.layout = layout
        self._struct = _Weights(self.codes.data_ptr(), self.scales.data_ptr(), self.n, self.k,
                                self.group, LAYOUTS[layout])

    @classmethod
    def from_host(cls, w: np.ndarray, scales: np.ndarray, device="cuda", layout: str = "v1"):
        torch = _torch()
        codes, sp = pack(w, scales, layout)
        n, k = w.shape
        group = k // scales.shape[1]
        return cls(torch.from_numpy(codes).to(device), torch.from_numpy(sp.view(np.int16)).to(device),
                   n, k, group, layout)

    @property
    def nbytes(self) -> int:
        return self.codes.numel() + 2 * self.scales.numel()

    def ref(self):
        return ctypes.byref(self._struct)


Q_LAYOUTS = {"row_major": 0, "operand_order": 1}


def quant_act_s8(x, q=None, scale=None, stream=None, layout="row_major"):
    """Per-token int8 quantisation of bf16 activations x [T, K] (device).
    layout: "row_major" or "operand_order" (the s8 contraction's byte order)."""
    torch = _torch()
    _dev(x, torch.bfloat16, "x")
    T, K = x.shape
    with _on(stream):
        if q is None:
            q = torch.empty((T, K), dtype=torch.int8, device=x.device)
        if scale is None:
            scale = torch.empty((T,), dtype=torch.float32, device=x.device)
    _dev(q, torch.int8, "q", (T, K), x.device)
    _dev(scale, torch.float32, "scale", (T,), x.device)
    _check(lib().tern_quant_act_s8(x.data_ptr(), T, K, q.data_ptr(), scale.data_ptr(),
                                   Q_LAYOUTS[layout], _stream(stream)))
    return q, scale


def quant_act_s8_rot(x, q=None, scale=None, stream=None, layout="row_major"):
    """Rotated per-token int8 quantisation: each 1024-wide block of x [T, K]
    (bf16, device) rotated by the orthonormal Hadamard matrix, then quantised
    as quant_act_s8 does. K a multiple of 1024, at most 32768."""
    torch = _torch()
    _dev(x, torch.bfloat16, "x")
    T, K = x.shape
    with _on(stream):
        if q is None:
            q = torch.empty((T, K), dtype=torch.int8, device=x.device)
        if scale is None:
            scale = torch.empty((T,), dtype=torch.float32, device=x.device)
    _dev(q, torch.int8, "q", (T, K), x.device)
    _dev(scale, torch.float32, "scale", (T,), x.device)
    _check(lib().tern_quant_act_s8_rot(x.data_ptr(), T, K, q.data_ptr(), scale.data_ptr(),
                                       Q_LAYOUTS[layout], _stream(stream)))
    return q, scale


def stream_read(buf, nbytes=None, depth=8, waves_per_cu=8, sink=None, stream=None):
    """One launch of the streaming-read ceiling kernel over the first `nbytes`
    bytes of the device tensor `buf` (default: all of it; a multiple of 1024).
    `sink` is a device int32/uint32 tensor of at least one element."""
    torch = _torch()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    total = buf.numel() * buf.element_size()
    nbytes = total if nbytes is None else int(nbytes)
    if nbytes > total:
        raise ValueError(f"nbytes={nbytes} exceeds the buffer's {total} bytes")
    if sink is None:
        with _on(stream):
            sink = torch.zeros((1,), dtype=torch.int32, device=buf.device)
    if not sink.is_cuda or sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must be a device tensor of at least 4 bytes")
    _check(lib().tern_stream_read(buf.data_ptr(), nbytes, depth, waves_per_cu, sink.data_ptr(),
                                  _stream(stream)))
    return sink


def linear(x, W: TernaryWeights, rung="auto", y=None, workspace=None, stream=None):
    """y [T, N] float32 = ternary_linear(x [T, K] bf16) on the GPU."""
    torch = _torch()
    _dev(x, torch.bfloat16, "x")
    T, K = x.shape
    if K != W.k:
        raise ValueError(f"x has K={K}, weights have K={W.k}")
    if y is None:
        with _on(stream):
            y = torch.empty((T, W.n), dtype=torch.float32, device=x.device)
    if W.codes.device != x.device:
        raise ValueError(f"x is on {x.device}, the weights on {W.codes.device}")
    _dev(y, torch.float32, "y", (T, W.n), x.device)
    r = _rung(rung)
    need = lib().tern_workspace_bytes(T, W.n, W.k, W.group, r)
    if need == ctypes.c_size_t(-1).value:
        raise TernError(5, lib().tern_last_error().decode())
    if workspace is None and need > 0:
        # zeroed: the workspace header holds arrival counters that start at zero
        with _on(stream):
            workspace = torch.zeros((need,), dtype=torch.uint8, device=x.device)
    if workspace is not None and (not workspace.is_cuda or workspace.device != x.device
                                  or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on the device of x")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().tern_linear(x.data_ptr(), T, W.ref(), y.data_ptr(), r, ws_ptr, ws_bytes,
                             _stream(stream)))
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20


def linear_noalloc(x, W: TernaryWeights, y, rung="auto", stream=None):
    """y = ternary_linear(x) into the caller's y with no workspace and no
    allocation (tern_linear_noalloc: the library's static device scratch of
    NOALLOC_SCRATCH_BYTES per GPU; calls that overlap on one GPU race)."""
    torch = _torch()
    _dev(x, torch.bfloat16, "x")
    T, K = x.shape
    if K != W.k:
        raise ValueError(f"x {tuple(x.shape)} does not match the weights' K={W.k}")
    _dev(y, torch.float32, "y", (T, W.n), x.device)
    _check(lib().tern_linear_noalloc(x.data_ptr(), T, W.ref(), y.data_ptr(), _rung(rung),
                                     _stream(stream)))
    return y


def linear_s8_q(q, scale, W: TernaryWeights, y=None, stream=None, layout="row_major"):
    """s8 contraction on pre-quantised activations (q int8 [T, K] in `layout`,
    scale float32 [T])."""
    torch = _torch()
    _dev(q, torch.int8, "q")
    T, K = q.shape
    if K != W.k:
        raise ValueError(f"q has K={K}, weights have K={W.k}")
    _dev(scale, torch.float32, "scale", (T,), q.device)
    if y is None:
        with _on(stream):
            y = torch.empty((T, W.n), dtype=torch.float32, device=q.device)
    _dev(y, torch.float32, "y", (T, W.n), q.device)
    _check(lib().tern_linear_s8_q(q.data_ptr(), scale.data_ptr(), T, W.ref(), y.data_ptr(),
                                  Q_LAYOUTS[layout], _stream(stream)))
    return y


def debug_s8_acc(q, W: TernaryWeights, acc=None, stream=None, layout="row_major"):
    """int32 [T, N, K/G] group accumulators of the s8 contraction on q in
    `layout` (each layout runs its own kernel)."""
    torch = _torch()
    _dev(q, torch.int8, "q")
    T = q.shape[0]
    if acc is None:
        with _on(stream):
            acc = torch.empty((T, W.n, W.k // W.group), dtype=torch.int32, device=q.device)
    if q.shape[1] != W.k:
        raise ValueError(f"q has K={q.shape[1]}, weights have K={W.k}")
    _dev(acc, torch.int32, "acc", (T, W.n, W.k // W.group), q.device)
    _check(lib().tern_debug_s8_acc(q.data_ptr(), T, W.ref(), acc.data_ptr(), Q_LAYOUTS[layout],
                                   _stream(stream)))
    return acc


class Chain:
    """A chain of T = 1 projections run by one persistent launch
    (tern_linear_chain). items: (W, x, y, y_bf16 or None, after) tuples of
    device tensors (x bf16 [1, K] or [K], y float32 [1, N], y_bf16 bf16 [1, N]);
    after = -1 or the index j of an earlier item: x is read once items 0..j are
    done. The table is built once; run() enqueues the whole chain."""

    def __init__(self, items, device="cuda"):
        torch = _torch()
        self._keep = []
        arr = (_ChainItem * len(items))()
        for i, (W, x, y, yb, after) in enumerate(items):
            _dev(x, torch.bfloat16, "x")
            _dev(y, torch.float32, "y")
            if x.numel() != W.k or y.numel() != W.n:
                raise ValueError(f"chain item {i}: x has {x.numel()} elements and y {y.numel()}, "
                                 f"the weights take {W.k} and give {W.n}")
            if yb is not None:
                _dev(yb, torch.bfloat16, "y_bf16")
                if yb.numel() != W.n:
                    raise ValueError(f"chain item {i}: y_bf16 has {yb.numel()} elements, not {W.n}")
            arr[i].W = W._struct
            arr[i].x = x.data_ptr()
            arr[i].y = y.data_ptr()
            arr[i].y_bf16 = yb.data_ptr() if yb is not None else None
            arr[i].after = int(after)
            self._keep += [W, x, y, yb]
        n = len(items)
        self.count = n
        tb = lib().tern_chain_table_bytes(arr, n)
        if tb == 0:
            raise TernError(2, lib().tern_last_error().decode())
        self.table = torch.empty((tb,), dtype=torch.uint8, device=device)
        cb = lib().tern_chain_counter_bytes(n)
        self.counters = torch.zeros((cb // 4,), dtype=torch.int32, device=device)
        self.error_flag = torch.zeros((1,), dtype=torch.int32, device=device)
        self.plan = _ChainPlan()
        torch.cuda.synchronize()
        _check(lib().tern_chain_build(arr, n, self.table.data_ptr(), self.table.numel(),
                                      ctypes.byref(self.plan)))

    def run(self, spin_limit: int = 1 << 20, stream=None):
        _check(lib().tern_linear_chain(ctypes.byref(self.plan), self.table.data_ptr(),
                                       self.counters.data_ptr(), self.counters.numel() * 4,
                                       self.error_flag.data_ptr(), int(spin_limit), _stream(stream)))

    def failed(self) -> bool:
        """True if a wait gave up (synchronises on the flag)."""
        return bool(self.error_flag.item())
