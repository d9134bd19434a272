"""GPU parity of the operator options (qmoe_forward_ex) against the oracle:
expert biases, the gate/up layouts (halves, separate fc3), router_weights
aggregation, SwiGLU alpha/beta/limit, and 1- and 8-bit codes, on the decode
path (T*top_k <= 80) and the prefill tiles; routing ids bit-exact, weights to
float32 rounding, layer outputs within 1e-2 * max|ref| + 1e-3."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
import qmoe_synth as synth
import quantized_mixture_experts_route_amd as qm
from tests import _device as dv

pytestmark = pytest.mark.gpu

U = 2.0 ** -24

OPTIONS = {
    "bias": dict(bias=True),
    "halves": dict(swiglu_fusion=2),
    "fc3": dict(swiglu_fusion=0, bias=True),
    "rw_norm": dict(router_weights=True),
    "rw_plain": dict(router_weights=True, normalize=0),
    "swiglu_params": dict(alpha=1.702, beta=0.5, limit=0.75),
    "int8": dict(fc1_bits=8, fc2_bits=8),
    "int1": dict(fc1_bits=1, fc2_bits=1),
    "mixed_8_2": dict(fc1_bits=8, fc2_bits=2, bias=True),
    "everything": dict(swiglu_fusion=0, bias=True, router_weights=True, alpha=1.5, beta=0.25,
                       limit=1.0, fc1_bits=4, fc2_bits=8),
}


def _spec(name, T, dtype, zp, bs=64, I=384):
    o = dict(OPTIONS[name])
    zpo = {"sym": math.nan, "zpo": 1.5, "u8": math.nan}[zp]
    # 8-bit codes span 16x the int4 range: scales 16x smaller keep the fp16
    # activations in range, as a real int8 quantisation would
    wide = 8 in (o.get("fc1_bits"), o.get("fc2_bits"))
    return synth.custom(T=T, H=256, I=I, E=6, k=2, block_size=bs, dtype=dtype, act=0,
                        zp_mode=zp, zpo=zpo, zp_range=(0, 1) if "int1" in name else (0, 3),
                        scale_range=(0.0003, 0.00125) if wide else (0.005, 0.02),
                        name=f"opt_{name}_T{T}", **{k: v for k, v in o.items() if k != "normalize"},
                        **({"normalize": o["normalize"]} if "normalize" in o else {}))


def _check(spec, seed, tokens=None):
    inp = synth.make_inputs(spec, seed)
    dev = dv.to_device(inp, spec)
    kw = dv.option_kwargs(inp, spec)
    out, ids, w = qm.forward(dev["hidden"], dev["logits"], dev["fc1"], dev["fc2"], top_k=spec["k"],
                             block_size=spec["block_size"], normalize=spec["normalize"],
                             activation=spec["act"], zero_point_offset=spec["zpo"],
                             return_routing=True, **kw)
    torch.cuda.synchronize()
    ids_ref, w_ref = oracle.route(inp["logits"], spec["k"], spec["normalize"], inp.get("router_weights"))
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=(spec["k"] + 6) * U, atol=1e-30)
    ref = oracle.forward(inp, spec, tokens)
    got = dv.as_f64(out)
    if tokens is not None:
        got = got[tokens]
    err = float(np.abs(got - ref).max())
    tol = dv.tolerance(ref)
    print(f"  {spec['name']}: max|err|={err:.3e} tol={tol:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("name", list(OPTIONS))
@pytest.mark.parametrize("T,dtype,zp", [(5, 1, "zpo"), (37, 2, "u8"), (90, 1, "sym"), (300, 2, "zpo")])
def test_options_layer(name, T, dtype, zp):
    # T = 5 and 37 decode (plan + m-tile kernels), 90 and 300 the prefill tiles
    _check(_spec(name, T, dtype, zp), 900 + T + len(name))


@pytest.mark.parametrize("name", ["halves", "fc3", "bias"])
def test_options_large_prefill_tile(name):
    # 4096 routes against I = 8192: the 128-row prefill tile with its staged scales
    spec = _spec(name, 2048, 2, "sym", bs=128, I=8192)
    spec["E"] = 4
    tokens = np.unique(np.concatenate([np.linspace(0, 2047, 40).astype(np.int64), [1, 2046]]))
    _check(spec, 77, tokens=tokens)


@pytest.mark.parametrize("bits", [1, 8])
@pytest.mark.parametrize("dtype", [1, 2])
@pytest.mark.parametrize("mode", ["sym", "zpo", "u8"])
def test_dequant_wide_and_narrow_codes_bit_exact(bits, dtype, mode):
    rng = np.random.default_rng(bits * 7 + dtype + len(mode))
    E, N, K, bs = 2, 24, 256, 32
    codes = rng.integers(0, 256, size=(E, N, K * bits // 8), dtype=np.uint8)
    s32 = rng.uniform(0.005, 0.02, size=(E, N, K // bs)).astype(np.float32)
    scales = synth._to_dtype_bits(s32, dtype)
    zp, zpo = None, math.nan
    if mode == "u8":
        zp = synth._draw_zero_points(rng, E, N, K // bs, bits, 0, (1 << bits) - 1)
    elif mode == "zpo":
        zpo = 0.5 if bits == 1 else 127.5
    proj = qm.Projection(torch.from_numpy(codes).cuda(), dv.bits_tensor(scales, dtype),
                         None if zp is None else torch.from_numpy(zp).cuda(), bits)
    q, w = qm.dequantize(proj, E, N, K, bs, dv.torch_dtype(dtype), zpo)
    q_ref, w_ref = oracle.dequant(codes, scales, zp, K, bits, bs, zpo, dtype)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    got = w.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, dv.round_to_dtype_bits(w_ref, dtype))
