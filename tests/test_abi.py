"""The C ABI without a GPU: the library loads, exports every entry point that
include/qmoe.h declares, sizes its workspace, and rejects every invalid
argument before touching the device (these calls never reach a launch)."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

import quantized_mixture_experts_route_amd as qm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")

FAKE = 1 << 20  # a 256-byte aligned non-NULL address; never dereferenced on these paths


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(qmoe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_bound_entry_points():
    assert set(_declared()) == set(qm.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = qm.load_library()
    for name in _declared():
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (QMOE_[A-Z0-9_]+) \(?(-?\d+)\)?", text))
    assert int(consts["QMOE_OK"]) == qm.OK
    assert int(consts["QMOE_ERR_INVALID_ARG"]) == qm.ERR_INVALID_ARG
    assert int(consts["QMOE_ERR_UNSUPPORTED"]) == qm.ERR_UNSUPPORTED
    assert int(consts["QMOE_ERR_WORKSPACE"]) == qm.ERR_WORKSPACE
    assert int(consts["QMOE_ERR_HIP"]) == qm.ERR_HIP
    assert int(consts["QMOE_DTYPE_F16"]) == qm.DTYPE_F16
    assert int(consts["QMOE_DTYPE_BF16"]) == qm.DTYPE_BF16
    assert int(consts["QMOE_ACT_SWIGLU"]) == qm.ACT_SWIGLU
    assert int(consts["QMOE_ACT_GEGLU"]) == qm.ACT_GEGLU
    assert int(consts["QMOE_DECODE_MAX_ROUTES"]) == qm.DECODE_MAX_ROUTES


def test_worklist_capacity_formula():
    # (ceil(R/m_tile) + min(E, R)) * ceil(N/n_tile)
    assert qm.worklist_capacity(512, 2, 8, 128, 128, 2048) == (8 + 8) * 16
    assert qm.worklist_capacity(6, 10, 512, 16, 32, 768) == (4 + 60) * 24
    assert qm.worklist_capacity(0, 2, 8, 16, 16, 16) == 0
    assert qm.worklist_capacity(-1, 2, 8, 16, 16, 16) == -1


def test_workspace_size_monotone_and_invalid():
    a = qm.workspace_size(8, 2048, 2048, 8, 2, 1)
    b = qm.workspace_size(512, 2048, 2048, 8, 2, 1)
    assert 0 < a < b
    assert a % 256 == 0 and b % 256 == 0
    # fp32 [R, H] plus dtype [R, I] intermediates dominate
    assert b >= 1024 * 2048 * 4 + 1024 * 2048 * 2
    assert qm.workspace_size(8, 2048, 2048, 8, 2, 3) == 0
    assert qm.workspace_size(8, 0, 2048, 8, 2, 1) == 0
    assert qm.workspace_size(1 << 40, 2048, 2048, 8, 2, 1) == 0
    # inputs are addressed with 32-bit element offsets: T*H and T*top_k*I stay below 2^32
    assert qm.workspace_size((1 << 20) - 1, 4096, 1024, 8, 2, 1) > 0
    assert qm.workspace_size(1 << 20, 4096, 1024, 8, 2, 1) == 0
    assert qm.workspace_size(1 << 19, 1024, 4096, 8, 2, 1) == 0


def _proj(bits=4, codes=FAKE, scales=FAKE, zp=None):
    return qm._Proj(codes, scales, zp, bits)


def _fwd(lib, **kw):
    args = dict(hidden=FAKE, logits=FAKE, T=4, H=256, I=256, E=8, fc1=_proj(), fc2=_proj(),
                zpo=math.nan, bs=32, k=2, normalize=1, act=0, dtype=1, out=FAKE, ids=None,
                w=None, ws=FAKE, ws_bytes=1 << 30)
    args.update(kw)
    fc1 = ctypes.byref(args["fc1"]) if args["fc1"] is not None else None
    fc2 = ctypes.byref(args["fc2"]) if args["fc2"] is not None else None
    return lib.qmoe_forward(args["hidden"], args["logits"], args["T"], args["H"], args["I"],
                            args["E"], fc1, fc2, args["zpo"], args["bs"], args["k"],
                            args["normalize"], args["act"], args["dtype"], args["out"],
                            args["ids"], args["w"], args["ws"], args["ws_bytes"], None)


INVALID_FORWARD = [
    (dict(T=-1), qm.ERR_INVALID_ARG),
    (dict(H=0), qm.ERR_INVALID_ARG),
    (dict(E=0), qm.ERR_INVALID_ARG),
    (dict(E=1025), qm.ERR_INVALID_ARG),
    (dict(k=0), qm.ERR_INVALID_ARG),
    (dict(k=9), qm.ERR_INVALID_ARG),
    (dict(normalize=2), qm.ERR_INVALID_ARG),
    (dict(act=2), qm.ERR_INVALID_ARG),
    (dict(dtype=0), qm.ERR_INVALID_ARG),
    (dict(bs=24), qm.ERR_INVALID_ARG),
    (dict(bs=8), qm.ERR_INVALID_ARG),
    (dict(H=272, bs=32), qm.ERR_INVALID_ARG),
    (dict(H=160, bs=32), qm.ERR_UNSUPPORTED),
    (dict(I=96, bs=32), qm.ERR_UNSUPPORTED),
    (dict(fc1=_proj(bits=5)), qm.ERR_INVALID_ARG),
    (dict(fc2=_proj(bits=6)), qm.ERR_INVALID_ARG),
    (dict(fc2=_proj(bits=5)), qm.ERR_INVALID_ARG),
    (dict(fc1=None), qm.ERR_INVALID_ARG),
    (dict(fc1=_proj(codes=None)), qm.ERR_INVALID_ARG),
    (dict(fc2=_proj(scales=None)), qm.ERR_INVALID_ARG),
    (dict(fc1=_proj(codes=FAKE + 8)), qm.ERR_INVALID_ARG),
    (dict(zpo=math.inf), qm.ERR_INVALID_ARG),
    (dict(hidden=None), qm.ERR_INVALID_ARG),
    (dict(out=FAKE + 2), qm.ERR_INVALID_ARG),
    (dict(ws=None), qm.ERR_INVALID_ARG),
    (dict(ws=FAKE + 64), qm.ERR_INVALID_ARG),
    (dict(ws_bytes=1000), qm.ERR_WORKSPACE),
    (dict(T=1 << 31), qm.ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,code", INVALID_FORWARD)
def test_forward_rejects_before_launch(kw, code):
    lib = qm.load_library()
    rc = _fwd(lib, **kw)
    assert rc == code, (kw, rc, qm.last_error())
    assert qm.last_error().startswith("qmoe: ")


def _opts(**kw):
    o = qm._LayerOpts(None, None, None, None, None, qm.SWIGLU_INTERLEAVED, 1.0, 0.0, math.inf)
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def test_forward_ex_option_validation():
    lib = qm.load_library()
    p = _proj()
    p3 = _proj(bits=2)

    def call(opts, act=0):
        return lib.qmoe_forward_ex(FAKE, FAKE, 4, 256, 256, 8, ctypes.byref(p), ctypes.byref(p),
                                   math.nan, 32, 2, 1, act, 1, FAKE, None, None, ctypes.byref(opts),
                                   FAKE, 1 << 30, None)

    assert call(_opts(swiglu_fusion=3)) == qm.ERR_INVALID_ARG
    assert call(_opts(swiglu_fusion=2), act=1) == qm.ERR_INVALID_ARG  # halves only with SwiGLU
    assert call(_opts(swiglu_fusion=0)) == qm.ERR_INVALID_ARG          # fc3 missing
    assert call(_opts(fc3=ctypes.pointer(p))) == qm.ERR_INVALID_ARG    # fc3 without fusion 0
    assert call(_opts(swiglu_fusion=0, fc3=ctypes.pointer(p3))) == qm.ERR_UNSUPPORTED  # width
    assert call(_opts(fc3_bias=FAKE)) == qm.ERR_INVALID_ARG            # fc3_bias without fc3
    assert call(_opts(fc1_bias=FAKE + 2)) == qm.ERR_INVALID_ARG        # alignment
    assert call(_opts(router_weights=FAKE + 1)) == qm.ERR_INVALID_ARG
    # T = 0 with every option set is a no-op
    opts = _opts(swiglu_fusion=0, fc3=ctypes.pointer(p), fc1_bias=FAKE, fc2_bias=FAKE,
                 fc3_bias=FAKE, router_weights=FAKE, activation_alpha=1.7, swiglu_limit=7.0)
    assert lib.qmoe_forward_ex(None, None, 0, 256, 256, 8, ctypes.byref(p), ctypes.byref(p),
                               math.nan, 32, 2, 1, 0, 1, None, None, None, ctypes.byref(opts),
                               None, 0, None) == qm.OK


def test_forward_zero_tokens_is_a_noop():
    lib = qm.load_library()
    # T = 0: every pointer of the token side may be NULL and nothing is launched
    assert _fwd(lib, T=0, hidden=None, logits=None, out=None, ws=None, ws_bytes=0) == qm.OK
    assert qm.last_error() == ""


def test_route_validation():
    lib = qm.load_library()
    assert lib.qmoe_route(FAKE, 4, 0, 1, 1, FAKE, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_route(FAKE, 4, 8, 9, 1, FAKE, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_route(FAKE, 4, 8, 2, 3, FAKE, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_route(None, 4, 8, 2, 1, FAKE, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_route(FAKE + 1, 4, 8, 2, 1, FAKE, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_route(None, 0, 8, 2, 1, None, None, None) == qm.OK


def test_group_validation():
    lib = qm.load_library()
    cap = qm.worklist_capacity(8, 2, 8, 16, 32, 64)
    args = [FAKE, 8, 2, 8, 16, 32, 64, FAKE, FAKE, FAKE, cap, FAKE, None]
    bad = list(args)
    bad[10] = cap - 1
    assert lib.qmoe_group(*bad) == qm.ERR_WORKSPACE
    bad = list(args)
    bad[3] = 2000
    assert lib.qmoe_group(*bad) == qm.ERR_INVALID_ARG
    bad = list(args)
    bad[4] = 0
    assert lib.qmoe_group(*bad) == qm.ERR_INVALID_ARG
    bad = list(args)
    bad[7] = None
    assert lib.qmoe_group(*bad) == qm.ERR_INVALID_ARG


def test_dequantize_validation():
    lib = qm.load_library()
    p = _proj(bits=3)
    assert lib.qmoe_dequantize(ctypes.byref(p), 1, 1, 48, 16, math.nan, 1, None, FAKE, None) \
        == qm.ERR_UNSUPPORTED
    assert lib.qmoe_dequantize(ctypes.byref(p), 1, 1, 64, 48, math.nan, 1, None, FAKE, None) \
        == qm.ERR_INVALID_ARG
    assert lib.qmoe_dequantize(ctypes.byref(p), 1, 1, 64, 32, math.nan, 1, None, None, None) \
        == qm.ERR_INVALID_ARG
    assert lib.qmoe_dequantize(None, 1, 1, 64, 32, math.nan, 1, None, FAKE, None) \
        == qm.ERR_INVALID_ARG


def test_raw_codes_validation():
    lib = qm.load_library()
    p = _proj(bits=3)
    # 3-bit codes have no multi-base variant; K must be a multiple of 32
    assert lib.qmoe_raw_codes(ctypes.byref(p), 1, 1, 64, 1, qm.RAW_MULTI_BASE, FAKE, None) \
        == qm.ERR_UNSUPPORTED
    assert lib.qmoe_raw_codes(ctypes.byref(p), 1, 1, 48, 1, qm.RAW_SINGLE_BASE, FAKE, None) \
        == qm.ERR_UNSUPPORTED
    assert lib.qmoe_raw_codes(ctypes.byref(p), 1, 1, 64, 1, 2, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_raw_codes(ctypes.byref(p), 1, 1, 64, 3, 0, FAKE, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_raw_codes(ctypes.byref(p), 1, 1, 64, 1, 0, None, None) == qm.ERR_INVALID_ARG
    assert lib.qmoe_raw_codes(None, 1, 1, 64, 1, 0, FAKE, None) == qm.ERR_INVALID_ARG


def test_router_validation():
    lib = qm.load_library()
    args = [FAKE, FAKE, 4, 256, 8, 1, 2, 1, None, FAKE, FAKE, None]

    def call(**kw):
        a = list(args)
        names = ["hidden", "gate", "T", "H", "E", "dtype", "k", "norm", "logits", "ids", "w", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.qmoe_router(*a)

    assert call(H=240) == qm.ERR_UNSUPPORTED       # not a multiple of 32
    assert call(E=0) == qm.ERR_INVALID_ARG
    assert call(E=1025) == qm.ERR_INVALID_ARG
    assert call(k=9) == qm.ERR_INVALID_ARG
    assert call(dtype=3) == qm.ERR_INVALID_ARG
    assert call(norm=2) == qm.ERR_INVALID_ARG
    assert call(hidden=None) == qm.ERR_INVALID_ARG
    assert call(gate=FAKE + 8) == qm.ERR_INVALID_ARG  # 16-byte alignment
    assert call(T=0, hidden=None) == qm.OK           # nothing to do


def test_shared_validation():
    lib = qm.load_library()
    p = _proj()
    n = lib.qmoe_shared_workspace_size(8, 256, 256, 8, 2, 128, 1)
    assert n > qm.workspace_size(8, 256, 256, 8, 2, 1)
    assert lib.qmoe_shared_workspace_size(8, 256, 256, 8, 2, 0, 1) == 0

    def call(I_shared=128, gate=FAKE, bs=32, ws=FAKE, ws_bytes=1 << 30, sp=p):
        return lib.qmoe_forward_shared(FAKE, FAKE, 8, 256, 256, 8, ctypes.byref(p), ctypes.byref(p),
                                       I_shared, ctypes.byref(sp), ctypes.byref(sp), gate,
                                       math.nan, bs, 2, 1, 0, 1, FAKE, None, None, ws, ws_bytes, None)

    assert call(I_shared=0) == qm.ERR_INVALID_ARG
    assert call(gate=None) == qm.ERR_INVALID_ARG
    assert call(bs=0) == qm.ERR_INVALID_ARG
    assert call(I_shared=96) == qm.ERR_UNSUPPORTED       # not a multiple of 128
    assert call(ws_bytes=n - 1) == qm.ERR_WORKSPACE
    assert call(sp=_proj(bits=5)) == qm.ERR_INVALID_ARG


def test_timer_validation():
    lib = qm.load_library()
    assert lib.qmoe_timer_start(7) == qm.ERR_INVALID_ARG


def test_workspace_holds_fc2_k_parts():
    # prefill layers whose fc2 work-list fills the last round of a 256-unit
    # grid poorly get room for fc2 K parts: y2 float32 [S, R, H] with S up to 4
    R, H, I = 4096 * 2, 4096, 14336
    big = qm.workspace_size(4096, H, I, 8, 2, 2)
    assert big >= 2 * R * H * 4 + R * I * 2
    # K = I = 384 holds no two equal parts of whole 128-input super-steps:
    # one y2 slice
    R2, H2, I2 = 65536 * 2, 512, 384
    one = qm.workspace_size(65536, H2, I2, 8, 2, 1)
    assert R2 * H2 * 4 + R2 * I2 * 2 <= one < 2 * R2 * H2 * 4 + R2 * I2 * 2
    # decode layers never split
    dec = qm.workspace_size(8, 2048, 2048, 8, 2, 1)
    assert dec < 2 * 16 * 2048 * 4 + 16 * 2048 * 2 + 65536
