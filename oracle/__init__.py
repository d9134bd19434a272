"""CPU oracle of the QMoE layer (double precision) -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports or calls
it and shares no code with it.  The arithmetic lives in ``qmoe_oracle.c``;
this module only builds that file with gcc and marshals numpy arrays through
ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qmoe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_F16 = 1
DTYPE_BF16 = 2


def build() -> str:
    """Compile qmoe_oracle.c into liboracle.so (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_widen.argtypes = [P, i64, i32, P]
    lib.oracle_route_key.argtypes = [ctypes.c_float]
    lib.oracle_route_key.restype = i32
    lib.oracle_route.argtypes = [P, P, i64, i32, i32, i32, P, P]
    lib.oracle_dequant.argtypes = [P, P, P, i64, i32, i32, i32, f64, i32, P, P]
    lib.oracle_forward.argtypes = [P, P, i64, i32, i32, i32,
                                   P, P, P, i32, P, P, P, i32,
                                   f64, i32, i32, i32, i32, i32, P, i64,
                                   ctypes.POINTER(_Opts), P]
    lib.oracle_group.argtypes = [P, i64, i32, i32, i32, i32, P, P, P, i64, P]
    lib.oracle_router_logits.argtypes = [P, P, i64, i32, i32, i32, P]
    lib.oracle_gated.argtypes = [f64, f64, i32, f64, f64, f64]
    lib.oracle_gated.restype = f64
    lib.oracle_shared_expert.argtypes = [P, i64, i32, i32, P, P, P, i32, P, P, P, i32,
                                         f64, i32, i32, i32, P, P, i64, P]
    _lib = lib
    return lib


class _Opts(ctypes.Structure):
    """Mirror of oracle_opts in qmoe_oracle.c."""
    _fields_ = [("fc1_bias", ctypes.c_void_p), ("fc2_bias", ctypes.c_void_p),
                ("fc3_codes", ctypes.c_void_p), ("fc3_scales", ctypes.c_void_p),
                ("fc3_zp", ctypes.c_void_p), ("fc3_bits", ctypes.c_int32),
                ("fc3_bias", ctypes.c_void_p), ("router_weights", ctypes.c_void_p),
                ("swiglu_fusion", ctypes.c_int32), ("alpha", ctypes.c_double),
                ("beta", ctypes.c_double), ("limit", ctypes.c_double)]


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """fp16/bf16 bit patterns -> float64."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    _load().oracle_widen(_ptr(bits), bits.size, dtype, _ptr(out))
    return out


def gated(gate: float, up: float, activation: int, alpha: float = 1.0, beta: float = 0.0,
          limit: float = float("inf")) -> float:
    """The gated activation of one (gate, up) pair, with the SwiGLU parameters."""
    return float(_load().oracle_gated(gate, up, activation, alpha, beta, limit))


def route_key(x: float) -> int:
    return int(_load().oracle_route_key(float(np.float32(x))))


def router_logits(hidden: np.ndarray, weight: np.ndarray, dtype: int) -> np.ndarray:
    """Router logits (float64 [T, E]) = hidden [T, H] @ weight[E, H]^T, both fp16/bf16 bit patterns."""
    hidden = _c(hidden, np.uint16)
    weight = _c(weight, np.uint16)
    T, H = hidden.shape
    E = weight.shape[0]
    assert weight.shape[1] == H
    out = np.empty((T, E), dtype=np.float64)
    _load().oracle_router_logits(_ptr(hidden), _ptr(weight), T, H, E, dtype, _ptr(out))
    return out


def route(logits: np.ndarray, top_k: int, normalize: int, router_weights=None):
    """Top-k expert ids (int32 [T, k]) and routing weights (float64 [T, k]); with
    router_weights (float32 [T, E]) the weights come from it instead of the logits."""
    logits = _c(logits, np.float32)
    rw = _c(router_weights, np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), dtype=np.int32)
    w = np.empty((T, top_k), dtype=np.float64)
    _load().oracle_route(_ptr(logits), _ptr(rw), T, E, top_k, normalize, _ptr(ids), _ptr(w))
    return ids, w


def dequant(codes, scales, zero_points, K, bits, block_size, zpo, dtype, want_codes=True,
            want_weights=True):
    """Unpacked codes (int32 [..., K]) and exact dequantized weights (float64 [..., K])."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    zero_points = _c(zero_points, np.uint8)
    lead = codes.shape[:-1]
    rows = int(np.prod(lead)) if lead else 1
    q = np.empty(lead + (K,), dtype=np.int32) if want_codes else None
    w = np.empty(lead + (K,), dtype=np.float64) if want_weights else None
    _load().oracle_dequant(_ptr(codes), _ptr(scales), _ptr(zero_points), rows, K, bits,
                           block_size, float(zpo), dtype, _ptr(q), _ptr(w))
    return q, w


def group(ids, E, m_tile, n_tile, N, capacity=None):
    """Offsets [E+1], stable expert-sorted route ids [n_valid], work-list [n_items, 3]."""
    ids = _c(ids, np.int32).reshape(-1)
    R = ids.size
    if capacity is None:
        n_tiles = -(-N // n_tile)
        capacity = (-(-R // m_tile) + min(E, R)) * n_tiles
    offsets = np.empty(E + 1, dtype=np.int32)
    sorted_routes = np.full(max(R, 1), -1, dtype=np.int32)
    worklist = np.zeros((max(capacity, 1), 3), dtype=np.int32)
    n_items = np.zeros(1, dtype=np.int64)
    _load().oracle_group(_ptr(ids), R, E, m_tile, n_tile, N, _ptr(offsets), _ptr(sorted_routes),
                         _ptr(worklist), capacity, _ptr(n_items))
    n = int(n_items[0])
    return offsets, sorted_routes[:offsets[E]], worklist[:min(n, capacity)], n


def forward(inp: dict, spec: dict, tokens=None) -> np.ndarray:
    """Layer output in float64 for the given token indices (all tokens by default)."""
    T, H, I, E = spec["T"], spec["H"], spec["I"], spec["E"]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = _c(tokens, np.int64)
    out = np.empty((tokens.size, H), dtype=np.float64)
    arrs = dict(hidden=_c(inp["hidden"], np.uint16), logits=_c(inp["logits"], np.float32),
                c1=_c(inp["fc1_codes"], np.uint8), s1=_c(inp["fc1_scales"], np.uint16),
                z1=_c(inp["fc1_zp"], np.uint8), c2=_c(inp["fc2_codes"], np.uint8),
                s2=_c(inp["fc2_scales"], np.uint16), z2=_c(inp["fc2_zp"], np.uint8),
                b1=_c(inp.get("fc1_bias"), np.float32), b2=_c(inp.get("fc2_bias"), np.float32),
                c3=_c(inp.get("fc3_codes"), np.uint8), s3=_c(inp.get("fc3_scales"), np.uint16),
                z3=_c(inp.get("fc3_zp"), np.uint8), b3=_c(inp.get("fc3_bias"), np.float32),
                rw=_c(inp.get("router_weights"), np.float32))
    opts = _Opts(_ptr(arrs["b1"]), _ptr(arrs["b2"]), _ptr(arrs["c3"]), _ptr(arrs["s3"]),
                 _ptr(arrs["z3"]), int(spec.get("fc3_bits", spec["fc1_bits"])), _ptr(arrs["b3"]),
                 _ptr(arrs["rw"]), int(spec.get("swiglu_fusion", 1)),
                 float(spec.get("alpha", 1.0)), float(spec.get("beta", 0.0)),
                 float(spec.get("limit", float("inf"))))
    _load().oracle_forward(
        _ptr(arrs["hidden"]), _ptr(arrs["logits"]), T, H, I, E,
        _ptr(arrs["c1"]), _ptr(arrs["s1"]), _ptr(arrs["z1"]), spec["fc1_bits"],
        _ptr(arrs["c2"]), _ptr(arrs["s2"]), _ptr(arrs["z2"]), spec["fc2_bits"],
        float(spec["zpo"]), spec["block_size"], spec["k"], spec["normalize"], spec["act"],
        spec["dtype"], _ptr(tokens), tokens.size, ctypes.byref(opts), _ptr(out))
    return out


def shared_expert(inp: dict, shared: dict, spec: dict, tokens=None) -> np.ndarray:
    """The shared expert's gated contribution (float64 [n_tokens, H]) for the given tokens:
    sigmoid(x . gate) * shared_fc2(act(shared_fc1(x)))."""
    T, H = spec["T"], spec["H"]
    Is = shared["I"]
    if tokens is None:
        tokens = np.arange(T, dtype=np.int64)
    tokens = _c(tokens, np.int64)
    out = np.empty((tokens.size, H), dtype=np.float64)
    a = dict(hidden=_c(inp["hidden"], np.uint16), c1=_c(shared["fc1_codes"], np.uint8),
             s1=_c(shared["fc1_scales"], np.uint16), z1=_c(shared["fc1_zp"], np.uint8),
             c2=_c(shared["fc2_codes"], np.uint8), s2=_c(shared["fc2_scales"], np.uint16),
             z2=_c(shared["fc2_zp"], np.uint8), g=_c(shared["gate"], np.uint16))
    _load().oracle_shared_expert(
        _ptr(a["hidden"]), T, H, Is, _ptr(a["c1"]), _ptr(a["s1"]), _ptr(a["z1"]), spec["fc1_bits"],
        _ptr(a["c2"]), _ptr(a["s2"]), _ptr(a["z2"]), spec["fc2_bits"], float(spec["zpo"]),
        spec["block_size"], spec["act"], spec["dtype"], _ptr(a["g"]), _ptr(tokens), tokens.size,
        _ptr(out))
    return out
