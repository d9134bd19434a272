"""MI355X (gfx950) quantized Mixture-of-Experts FFN layer.

A thin ctypes binding over ``libqmoe.so`` (C ABI declared in
``include/qmoe.h``).  This module only marshals arguments: it checks torch
tensors' device, dtype, contiguity and shape against the sizes it passes, and
hands raw device pointers plus the current HIP stream to the library.  Every
step of the layer runs in the library's HIP kernels; there is no fallback.
PyTorch provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqmoe.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE = -3
ERR_HIP = -4
DTYPE_F16 = 1
DTYPE_BF16 = 2
ACT_SWIGLU = 0
ACT_GEGLU = 1
DECODE_MAX_ROUTES = 80
STAGE_ROUTE, STAGE_GROUP, STAGE_FC1, STAGE_FC2, STAGE_COMBINE = range(5)
RAW_SINGLE_BASE = 0
RAW_MULTI_BASE = 1

EXPORTED = ("qmoe_last_error", "qmoe_route", "qmoe_router", "qmoe_worklist_capacity", "qmoe_group",
            "qmoe_workspace_size", "qmoe_forward", "qmoe_forward_ex", "qmoe_forward_noalloc",
            "qmoe_shared_workspace_size", "qmoe_forward_shared", "qmoe_dequantize",
            "qmoe_raw_codes",
            "qmoe_timer_start", "qmoe_timer_stop")


class QMoEError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


class _Proj(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("zero_points", ctypes.c_void_p), ("bits", ctypes.c_int32)]


class _LayerOpts(ctypes.Structure):
    _fields_ = [("fc1_bias", ctypes.c_void_p), ("fc2_bias", ctypes.c_void_p),
                ("fc3", ctypes.POINTER(_Proj)), ("fc3_bias", ctypes.c_void_p),
                ("router_weights", ctypes.c_void_p), ("swiglu_fusion", ctypes.c_int32),
                ("activation_alpha", ctypes.c_float), ("activation_beta", ctypes.c_float),
                ("swiglu_limit", ctypes.c_float)]


SWIGLU_SEPARATE, SWIGLU_INTERLEAVED, SWIGLU_HALVES = 0, 1, 2


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libqmoe.so and declare its signatures (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() or "
                           "python quantized_mixture_experts_route_amd/build.py")
    lib = ctypes.CDLL(path)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sz = ctypes.c_size_t
    lib.qmoe_last_error.restype = ctypes.c_char_p
    lib.qmoe_last_error.argtypes = []
    lib.qmoe_route.argtypes = [P, i64, i32, i32, i32, P, P, P]
    lib.qmoe_router.argtypes = [P, P, i64, i32, i32, i32, i32, i32, P, P, P, P]
    lib.qmoe_worklist_capacity.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.qmoe_worklist_capacity.restype = i64
    lib.qmoe_group.argtypes = [P, i64, i32, i32, i32, i32, i32, P, P, P, i64, P, P]
    lib.qmoe_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.qmoe_workspace_size.restype = sz
    lib.qmoe_forward.argtypes = [P, P, i64, i32, i32, i32, ctypes.POINTER(_Proj),
                                 ctypes.POINTER(_Proj), f32, i32, i32, i32, i32, i32, P, P, P, P,
                                 sz, P]
    lib.qmoe_forward_ex.argtypes = [P, P, i64, i32, i32, i32, ctypes.POINTER(_Proj),
                                    ctypes.POINTER(_Proj), f32, i32, i32, i32, i32, i32, P, P, P,
                                    ctypes.POINTER(_LayerOpts), P, sz, P]
    lib.qmoe_forward_noalloc.argtypes = [P, P, i64, i32, i32, i32, ctypes.POINTER(_Proj),
                                         ctypes.POINTER(_Proj), f32, i32, i32, i32, i32, i32, P,
                                         P, P, P]
    lib.qmoe_shared_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    lib.qmoe_shared_workspace_size.restype = sz
    lib.qmoe_forward_shared.argtypes = [P, P, i64, i32, i32, i32, ctypes.POINTER(_Proj),
                                        ctypes.POINTER(_Proj), i32, ctypes.POINTER(_Proj),
                                        ctypes.POINTER(_Proj), P, f32, i32, i32, i32, i32, i32,
                                        P, P, P, P, sz, P]
    lib.qmoe_dequantize.argtypes = [ctypes.POINTER(_Proj), i32, i32, i32, i32, f32, i32, P, P, P]
    lib.qmoe_raw_codes.argtypes = [ctypes.POINTER(_Proj), i32, i32, i32, i32, i32, P, P]
    lib.qmoe_timer_start.argtypes = [i32]
    lib.qmoe_timer_stop.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    for name in ("qmoe_route", "qmoe_router", "qmoe_group", "qmoe_forward", "qmoe_forward_ex",
                 "qmoe_forward_noalloc",
                 "qmoe_forward_shared",
                 "qmoe_dequantize", "qmoe_raw_codes",
                 "qmoe_timer_start", "qmoe_timer_stop"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().qmoe_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise QMoEError(rc, last_error())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float16:
        return DTYPE_F16
    if dt == torch.bfloat16:
        return DTYPE_BF16
    raise ValueError(f"activation dtype must be float16 or bfloat16, got {dt}")


def zp_row_bytes(n_blocks: int, bits: int) -> int:
    return n_blocks if bits == 3 else -(-n_blocks // (8 // bits))


@dataclass
class Projection:
    """One quantized projection of all experts (device tensors).

    codes: uint8 [E, N, K*bits/8]; scales: fp16/bf16 [E, N, K/block_size];
    zero_points: None or uint8 [E, N, zp_row_bytes(K/block_size, bits)]."""
    codes: torch.Tensor
    scales: torch.Tensor
    zero_points: Optional[torch.Tensor]
    bits: int

    def _struct(self, E, N, K, block_size, name) -> _Proj:
        _dev(self.codes, f"{name}.codes", torch.uint8, (E, N, K * self.bits // 8))
        _dev(self.scales, f"{name}.scales", (torch.float16, torch.bfloat16),
             (E, N, K // block_size))
        if self.zero_points is not None:
            _dev(self.zero_points, f"{name}.zero_points", torch.uint8,
                 (E, N, zp_row_bytes(K // block_size, self.bits)))
        return _Proj(_ptr(self.codes), _ptr(self.scales), _ptr(self.zero_points), int(self.bits))


def route(logits: torch.Tensor, top_k: int, normalize: int = 1, stream=None):
    """Top-k expert ids (int32 [T, k]) and weights (float32 [T, k]) on the device."""
    _dev(logits, "logits", torch.float32)
    T, E = logits.shape
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check(load_library().qmoe_route(_ptr(logits), T, E, top_k, normalize, _ptr(ids), _ptr(w),
                                     _stream(stream)))
    return ids, w


def router(hidden: torch.Tensor, gate_weight: torch.Tensor, top_k: int, normalize: int = 1,
           want_logits: bool = True, stream=None):
    """Router projection + top-k in one launch: (logits float32 [T, E] or None,
    ids int32 [T, k], weights float32 [T, k]); gate_weight is [E, H] in hidden's dtype."""
    dt = dtype_code(hidden.dtype)
    _dev(hidden, "hidden")
    T, H = hidden.shape
    E = gate_weight.shape[0]
    _dev(gate_weight, "gate_weight", hidden.dtype, (E, H))
    dev = hidden.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None
    ids = torch.empty((T, top_k), dtype=torch.int32, device=dev)
    w = torch.empty((T, top_k), dtype=torch.float32, device=dev)
    _check(load_library().qmoe_router(_ptr(hidden), _ptr(gate_weight), T, H, E, dt, top_k,
                                      normalize, _ptr(logits), _ptr(ids), _ptr(w),
                                      _stream(stream)))
    return logits, ids, w


def worklist_capacity(T, top_k, E, m_tile, n_tile, N) -> int:
    return int(load_library().qmoe_worklist_capacity(T, top_k, E, m_tile, n_tile, N))


def group(topk_ids: torch.Tensor, E: int, m_tile: int, n_tile: int, N: int, stream=None,
          capacity: Optional[int] = None):
    """Expert offsets [E+1], sorted route ids [R], work-list [cap, 3], item count [1] (device)."""
    _dev(topk_ids, "topk_ids", torch.int32)
    T, top_k = topk_ids.shape if topk_ids.dim() == 2 else (topk_ids.numel(), 1)
    R = T * top_k
    cap = worklist_capacity(T, top_k, E, m_tile, n_tile, N) if capacity is None else capacity
    dev = topk_ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_routes = torch.full((max(R, 1),), -1, dtype=torch.int32, device=dev)
    worklist = torch.zeros((max(cap, 1), 3), dtype=torch.int32, device=dev)
    n_items = torch.zeros(1, dtype=torch.int32, device=dev)
    _check(load_library().qmoe_group(_ptr(topk_ids), T, top_k, E, m_tile, n_tile, N,
                                     _ptr(offsets), _ptr(sorted_routes), _ptr(worklist), cap,
                                     _ptr(n_items), _stream(stream)))
    return offsets, sorted_routes[:R], worklist, n_items


def workspace_size(T, H, I, E, top_k, dtype) -> int:
    return int(load_library().qmoe_workspace_size(T, H, I, E, top_k, dtype))


def alloc_workspace(T, H, I, E, top_k, dtype, device="cuda") -> torch.Tensor:
    n = workspace_size(T, H, I, E, top_k, dtype)
    if n == 0:
        raise ValueError("invalid sizes for the workspace")
    return torch.empty(n, dtype=torch.uint8, device=device)  # torch blocks are 512-byte aligned


def forward(hidden: torch.Tensor, logits: torch.Tensor, fc1: Projection, fc2: Projection, *,
            top_k: int, block_size: int, normalize: int = 1, activation: int = ACT_SWIGLU,
            zero_point_offset: float = math.nan, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, return_routing: bool = False,
            stream=None, fc1_bias: Optional[torch.Tensor] = None,
            fc2_bias: Optional[torch.Tensor] = None, fc3: Optional[Projection] = None,
            fc3_bias: Optional[torch.Tensor] = None,
            router_weights: Optional[torch.Tensor] = None,
            swiglu_fusion: int = SWIGLU_INTERLEAVED, activation_alpha: float = 1.0,
            activation_beta: float = 0.0, swiglu_limit: float = math.inf):
    """The QMoE layer: out [T, H] in hidden's dtype (plus routing if asked).

    The keyword options after ``stream`` are the operator's optional inputs and
    attributes (qmoe_forward_ex): expert biases (float32), a separate up
    projection fc3 with swiglu_fusion = SWIGLU_SEPARATE, the gate/up halves
    layout SWIGLU_HALVES, router_weights (float32 [T, E]) and the SwiGLU
    parameters."""
    dt = dtype_code(hidden.dtype)
    _dev(hidden, "hidden")
    T, H = hidden.shape
    _dev(logits, "logits", torch.float32)
    if logits.shape[0] != T:
        raise ValueError("logits rows must equal hidden rows")
    E = logits.shape[1]
    for name, proj in (("fc1", fc1), ("fc2", fc2)):
        # the library reads scales as the layer's dtype; another dtype's bits would be misread
        if proj.scales.dtype != hidden.dtype:
            raise ValueError(f"{name}.scales has dtype {proj.scales.dtype}, expected {hidden.dtype}")
    I = fc2.codes.shape[2] * 8 // fc2.bits
    n1 = I if swiglu_fusion == SWIGLU_SEPARATE else 2 * I
    p1 = fc1._struct(E, n1, H, block_size, "fc1")
    p2 = fc2._struct(E, H, I, block_size, "fc2")
    if out is None:
        out = torch.empty_like(hidden)
    _dev(out, "out", hidden.dtype, (T, H))
    if workspace is None:
        workspace = alloc_workspace(T, H, I, E, top_k, dt, hidden.device)
    _dev(workspace, "workspace", torch.uint8)
    ids = w = None
    if return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=hidden.device)
        w = torch.empty((T, top_k), dtype=torch.float32, device=hidden.device)
    p3 = None
    if fc3 is not None:
        if fc3.scales.dtype != hidden.dtype:
            raise ValueError(f"fc3.scales has dtype {fc3.scales.dtype}, expected {hidden.dtype}")
        p3 = fc3._struct(E, I, H, block_size, "fc3")
    for name, b, shape in (("fc1_bias", fc1_bias, (E, n1)), ("fc2_bias", fc2_bias, (E, H)),
                           ("fc3_bias", fc3_bias, (E, I)), ("router_weights", router_weights, (T, E))):
        if b is not None:
            _dev(b, name, torch.float32, shape)
    opts = _LayerOpts(_ptr(fc1_bias), _ptr(fc2_bias), ctypes.pointer(p3) if p3 is not None else None,
                      _ptr(fc3_bias), _ptr(router_weights), int(swiglu_fusion),
                      float(activation_alpha), float(activation_beta), float(swiglu_limit))
    _check(load_library().qmoe_forward_ex(
        _ptr(hidden), _ptr(logits), T, H, I, E, ctypes.byref(p1), ctypes.byref(p2),
        float(zero_point_offset), block_size, top_k, normalize, activation, dt, _ptr(out),
        _ptr(ids), _ptr(w), ctypes.byref(opts), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return (out, ids, w) if return_routing else out


def forward_shared(hidden: torch.Tensor, logits: torch.Tensor, fc1: Projection, fc2: Projection,
                   shared_fc1: Projection, shared_fc2: Projection, shared_gate: torch.Tensor, *,
                   top_k: int, block_size: int, normalize: int = 1, activation: int = ACT_SWIGLU,
                   zero_point_offset: float = math.nan, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, return_routing: bool = False,
                   stream=None):
    """The layer with a shared expert: routed output + sigmoid(x . shared_gate) * shared FFN."""
    dt = dtype_code(hidden.dtype)
    _dev(hidden, "hidden")
    T, H = hidden.shape
    _dev(logits, "logits", torch.float32)
    E = logits.shape[1]
    for name, proj in (("fc1", fc1), ("fc2", fc2), ("shared_fc1", shared_fc1),
                       ("shared_fc2", shared_fc2)):
        if proj.scales.dtype != hidden.dtype:
            raise ValueError(f"{name}.scales has dtype {proj.scales.dtype}, expected {hidden.dtype}")
    I = fc2.codes.shape[2] * 8 // fc2.bits
    Is = shared_fc2.codes.shape[2] * 8 // shared_fc2.bits
    p1 = fc1._struct(E, 2 * I, H, block_size, "fc1")
    p2 = fc2._struct(E, H, I, block_size, "fc2")
    s1 = shared_fc1._struct(1, 2 * Is, H, block_size, "shared_fc1")
    s2 = shared_fc2._struct(1, H, Is, block_size, "shared_fc2")
    _dev(shared_gate, "shared_gate", hidden.dtype, (H,))
    if out is None:
        out = torch.empty_like(hidden)
    _dev(out, "out", hidden.dtype, (T, H))
    if workspace is None:
        n = int(load_library().qmoe_shared_workspace_size(T, H, I, E, top_k, Is, dt))
        if n == 0:
            raise ValueError("invalid sizes for the shared-expert workspace")
        workspace = torch.empty(n, dtype=torch.uint8, device=hidden.device)
    _dev(workspace, "workspace", torch.uint8)
    ids = w = None
    if return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=hidden.device)
        w = torch.empty((T, top_k), dtype=torch.float32, device=hidden.device)
    _check(load_library().qmoe_forward_shared(
        _ptr(hidden), _ptr(logits), T, H, I, E, ctypes.byref(p1), ctypes.byref(p2), Is,
        ctypes.byref(s1), ctypes.byref(s2), _ptr(shared_gate), float(zero_point_offset),
        block_size, top_k, normalize, activation, dt, _ptr(out), _ptr(ids), _ptr(w),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return (out, ids, w) if return_routing else out


NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_noalloc(hidden: torch.Tensor, logits: torch.Tensor, fc1: Projection,
                    fc2: Projection, *, top_k: int, block_size: int, normalize: int = 1,
                    activation: int = ACT_SWIGLU, zero_point_offset: float = math.nan,
                    out: torch.Tensor, return_routing: bool = False, stream=None):
    """The QMoE layer through qmoe_forward_noalloc: the library's fixed scratch
    array serves as workspace and the call allocates nothing on the device
    (``out`` and, with return_routing, the routing outputs are the caller's)."""
    dt = dtype_code(hidden.dtype)
    _dev(hidden, "hidden")
    T, H = hidden.shape
    _dev(logits, "logits", torch.float32)
    if logits.shape[0] != T:
        raise ValueError("logits rows must equal hidden rows")
    E = logits.shape[1]
    for name, proj in (("fc1", fc1), ("fc2", fc2)):
        if proj.scales.dtype != hidden.dtype:
            raise ValueError(f"{name}.scales has dtype {proj.scales.dtype}, expected {hidden.dtype}")
    I = fc2.codes.shape[2] * 8 // fc2.bits
    p1 = fc1._struct(E, 2 * I, H, block_size, "fc1")
    p2 = fc2._struct(E, H, I, block_size, "fc2")
    _dev(out, "out", hidden.dtype, (T, H))
    ids = w = None
    if return_routing:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=hidden.device)
        w = torch.empty((T, top_k), dtype=torch.float32, device=hidden.device)
    _check(load_library().qmoe_forward_noalloc(
        _ptr(hidden), _ptr(logits), T, H, I, E, ctypes.byref(p1), ctypes.byref(p2),
        float(zero_point_offset), block_size, top_k, normalize, activation, dt, _ptr(out),
        _ptr(ids), _ptr(w), _stream(stream)))
    return (out, ids, w) if return_routing else out


def dequantize(proj: Projection, E: int, N: int, K: int, block_size: int, dtype: torch.dtype,
               zero_point_offset: float = math.nan, want_codes: bool = True, stream=None):
    """Unpacked codes (int32 [E, N, K] or None) and dequantized weights (dtype [E, N, K])."""
    if proj.scales.dtype != dtype:
        raise ValueError(f"scales have dtype {proj.scales.dtype}, expected {dtype}")
    p = proj._struct(E, N, K, block_size, "projection")
    dev = proj.codes.device
    w = torch.empty((E, N, K), dtype=dtype, device=dev)
    q = torch.empty((E, N, K), dtype=torch.int32, device=dev) if want_codes else None
    _check(load_library().qmoe_dequantize(ctypes.byref(p), E, N, K, block_size,
                                          float(zero_point_offset), dtype_code(dtype), _ptr(q),
                                          _ptr(w), _stream(stream)))
    return q, w


def raw_codes(proj: Projection, E: int, N: int, K: int, block_size: int, dtype: torch.dtype,
              variant: int = RAW_SINGLE_BASE, stream=None):
    """int32 [E, N, K]: the codes the decode kernels' raw-code MFMA operands carry."""
    p = proj._struct(E, N, K, block_size, "projection")
    q = torch.empty((E, N, K), dtype=torch.int32, device=proj.codes.device)
    _check(load_library().qmoe_raw_codes(ctypes.byref(p), E, N, K, dtype_code(dtype), variant,
                                         _ptr(q), _stream(stream)))
    return q


def timer_start(stage: int):
    _check(load_library().qmoe_timer_start(stage))


def timer_stop():
    """(summed milliseconds, number of launches timed) since timer_start."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check(load_library().qmoe_timer_stop(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
