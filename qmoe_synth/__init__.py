"""Seeded synthetic inputs for the QMoE layer.

This module only draws random bytes in the shapes, dtypes and value ranges of
the workloads below; it holds none of the layer's arithmetic (no routing, no
unpacking, no dequantization, no matmul).  Both the GPU library's tests and the
CPU oracle consume exactly the arrays it returns.

Every array is a plain numpy array:

* ``logits``      float32 ``[T, E]``
* ``hidden``      uint16 ``[T, H]`` -- raw fp16 or bf16 bit patterns
* ``fcX_codes``   uint8 ``[E, N, K*bits/8]`` -- packed codes, uniform bytes
  (uniform bytes give uniform codes for 2/4-bit packing, and uniform 24-bit
  groups for 3-bit packing)
* ``fcX_scales``  uint16 ``[E, N, K/block_size]`` -- fp16/bf16 bit patterns
* ``fcX_zp``      uint8 zero-point tensor or ``None``

fc1 has ``N = 2*I`` rows (gate/up interleaved) and ``K = H``; fc2 has
``N = H`` and ``K = I``.

The five named workloads are the QMoE layer shapes the pages discuss: the tiny
int4 layer, the H100-measured decode/prefill shape of the int2/int4 QMoE pull
request (hidden = inter = 2048, E = 8, top-2, block 128), the 512-expert
top-10 mixed int3/int2 decode of the INT3 pull request, and a large skewed
int4 prefill.
"""
from __future__ import annotations

import math

import numpy as np

DTYPE_F16 = 1
DTYPE_BF16 = 2
ACT_SWIGLU = 0
ACT_GEGLU = 1

WORKLOADS = {
    1: dict(name="tiny_int4_T16_H256_I512_E8_k2", T=16, H=256, I=512, E=8, k=2,
            normalize=1, act=ACT_SWIGLU, dtype=DTYPE_F16, fc1_bits=4, fc2_bits=4,
            block_size=32, zp_mode="sym", zpo=math.nan, scale_range=(0.005, 0.02),
            logit_sigma=1.0, logit_bias=None),
    2: dict(name="decode_int2_geglu_T8_H2048_I2048_E8_k2", T=8, H=2048, I=2048, E=8, k=2,
            normalize=1, act=ACT_GEGLU, dtype=DTYPE_F16, fc1_bits=2, fc2_bits=2,
            block_size=128, zp_mode="zpo", zpo=1.5, scale_range=(0.005, 0.02),
            logit_sigma=1.0, logit_bias=None),
    3: dict(name="prefill_int4_u8zp_T512_H2048_I2048_E8_k2", T=512, H=2048, I=2048, E=8, k=2,
            normalize=1, act=ACT_SWIGLU, dtype=DTYPE_F16, fc1_bits=4, fc2_bits=4,
            block_size=128, zp_mode="u8", zp_range=(6, 10), zpo=math.nan,
            scale_range=(0.005, 0.02), logit_sigma=1.0, logit_bias=None),
    4: dict(name="many_expert_int3_int2_T6_H2048_I768_E512_k10", T=6, H=2048, I=768, E=512,
            k=10, normalize=1, act=ACT_SWIGLU, dtype=DTYPE_BF16, fc1_bits=3, fc2_bits=2,
            block_size=32, zp_mode="sym", zpo=math.nan, scale_range=(0.005, 0.02),
            logit_sigma=2.0, logit_bias=None),
    5: dict(name="skewed_prefill_int4_T4096_H4096_I14336_E8_k2", T=4096, H=4096, I=14336, E=8,
            k=2, normalize=1, act=ACT_SWIGLU, dtype=DTYPE_BF16, fc1_bits=4, fc2_bits=4,
            block_size=128, zp_mode="sym", zpo=math.nan, scale_range=(0.002, 0.01),
            logit_sigma=1.0, logit_bias="linspace0to2"),
}


def workload(i: int, **overrides) -> dict:
    """A copy of named workload ``i`` (1..5) with optional field overrides."""
    spec = dict(WORKLOADS[i])
    spec.update(overrides)
    return spec


def custom(T, H, I, E, k, *, fc1_bits=4, fc2_bits=4, block_size=32, dtype=DTYPE_F16,
           act=ACT_SWIGLU, normalize=1, zp_mode="sym", zpo=math.nan, zp_range=None,
           scale_range=(0.005, 0.02), logit_sigma=1.0, logit_bias=None, name="custom", **options):
    """A workload spec for arbitrary (test) shapes.  Options: swiglu_fusion (0, 1, 2),
    fc3_bits, bias (bool), router_weights (bool), alpha, beta, limit."""
    spec = dict(name=name, T=T, H=H, I=I, E=E, k=k, normalize=normalize, act=act,
                dtype=dtype, fc1_bits=fc1_bits, fc2_bits=fc2_bits, block_size=block_size,
                zp_mode=zp_mode, zpo=zpo, zp_range=zp_range, scale_range=scale_range,
                logit_sigma=logit_sigma, logit_bias=logit_bias)
    spec.update(options)
    return spec


def _to_dtype_bits(x32: np.ndarray, dtype: int) -> np.ndarray:
    """Round float32 values to fp16/bf16 (round-to-nearest-even) and return the bit patterns."""
    if dtype == DTYPE_F16:
        return x32.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _zp_row_bytes(n_blocks: int, bits: int) -> int:
    """Bytes per row of a zero-point tensor: 2/4-bit values share bytes, 3-bit ones get a byte each."""
    return n_blocks if bits == 3 else -(-n_blocks // (8 // bits))


def _draw_zero_points(rng, E, N, n_blocks, bits, lo, hi) -> np.ndarray:
    """Zero-point bytes holding values drawn uniformly from the integers [lo, hi].

    For 2/4-bit widths the values of consecutive blocks fill each byte from the
    low bits up; for 3-bit one byte holds one value."""
    vals = rng.integers(lo, hi + 1, size=(E, N, n_blocks), dtype=np.int64)
    if bits == 3:
        return vals.astype(np.uint8)
    per = 8 // bits
    nbytes = _zp_row_bytes(n_blocks, bits)
    padded = np.zeros((E, N, nbytes * per), dtype=np.int64)
    padded[:, :, :n_blocks] = vals
    padded = padded.reshape(E, N, nbytes, per)
    out = np.zeros((E, N, nbytes), dtype=np.int64)
    for j in range(per):
        out |= padded[:, :, :, j] << (bits * j)
    return out.astype(np.uint8)


def _draw_logits(rng, spec) -> np.ndarray:
    T, E = spec["T"], spec["E"]
    logits = rng.standard_normal((T, E), dtype=np.float32) * np.float32(spec["logit_sigma"])
    if spec.get("logit_bias") == "linspace0to2":
        logits = logits + np.linspace(0.0, 2.0, E, dtype=np.float32)[None, :]
    return np.ascontiguousarray(logits, dtype=np.float32)


def make_logits(spec: dict, seed: int) -> np.ndarray:
    """Only the router logits of ``make_inputs(spec, seed)`` (they are drawn first)."""
    return _draw_logits(np.random.default_rng(seed), spec)


def make_inputs(spec: dict, seed: int) -> dict:
    """Draw one layer's inputs for ``spec`` with ``numpy.random.default_rng(seed)``.

    Draw order is fixed: logits, hidden, fc1 codes, fc1 scales, fc1 zero points,
    fc2 codes, fc2 scales, fc2 zero points.
    """
    rng = np.random.default_rng(seed)
    T, H, I, E, bs = spec["T"], spec["H"], spec["I"], spec["E"], spec["block_size"]
    dtype = spec["dtype"]

    logits = _draw_logits(rng, spec)

    hidden = _to_dtype_bits(rng.standard_normal((T, H), dtype=np.float32), dtype)

    out = dict(logits=logits, hidden=np.ascontiguousarray(hidden))
    lo_s, hi_s = spec["scale_range"]
    fusion = spec.get("swiglu_fusion", 1)
    n1 = I if fusion == 0 else 2 * I  # fc1 rows: gate only when a separate fc3 holds the up rows
    for name, N, K, bits in (("fc1", n1, H, spec["fc1_bits"]), ("fc2", H, I, spec["fc2_bits"])):
        row_bytes = K * bits // 8
        codes = rng.integers(0, 256, size=(E, N, row_bytes), dtype=np.uint8)
        n_blocks = K // bs
        s32 = rng.uniform(lo_s, hi_s, size=(E, N, n_blocks)).astype(np.float32)
        scales = _to_dtype_bits(s32, dtype)
        zp = None
        if spec.get("zp_mode") == "u8":
            lo_z, hi_z = spec["zp_range"]
            zp = _draw_zero_points(rng, E, N, n_blocks, bits, lo_z, hi_z)
        out[name + "_codes"] = codes
        out[name + "_scales"] = np.ascontiguousarray(scales)
        out[name + "_zp"] = zp
    # operator options, drawn after everything above so the base arrays keep their bytes
    if fusion == 0:  # the separate up projection fc3 [E, I, H]
        bits = spec.get("fc3_bits", spec["fc1_bits"])
        out["fc3_codes"] = rng.integers(0, 256, size=(E, I, H * bits // 8), dtype=np.uint8)
        s32 = rng.uniform(lo_s, hi_s, size=(E, I, H // bs)).astype(np.float32)
        out["fc3_scales"] = np.ascontiguousarray(_to_dtype_bits(s32, dtype))
        out["fc3_zp"] = None
        if spec.get("zp_mode") == "u8":
            lo_z, hi_z = spec["zp_range"]
            out["fc3_zp"] = _draw_zero_points(rng, E, I, H // bs, bits, lo_z, hi_z)
    if spec.get("bias"):  # float32 expert biases ~ N(0, 0.1^2)
        out["fc1_bias"] = (rng.standard_normal((E, n1), dtype=np.float32) * np.float32(0.1))
        out["fc2_bias"] = (rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.1))
        if fusion == 0:
            out["fc3_bias"] = (rng.standard_normal((E, I), dtype=np.float32) * np.float32(0.1))
    if spec.get("router_weights"):  # aggregation weights, uniform in [0, 1)
        out["router_weights"] = rng.random((T, E), dtype=np.float32)
    return out


def make_router_weights(E: int, H: int, dtype: int, seed: int) -> np.ndarray:
    """Router (gate) weight bit patterns [E, H]: N(0, 1/H) values rounded to the dtype,
    so that the logits of N(0, 1) hidden rows are about N(0, 1)."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / math.sqrt(H))
    return np.ascontiguousarray(_to_dtype_bits(w, dtype))


def make_hidden(T: int, H: int, dtype: int, seed: int) -> np.ndarray:
    """Hidden-state bit patterns [T, H]: N(0, 1) rounded to the dtype."""
    rng = np.random.default_rng(seed)
    return np.ascontiguousarray(_to_dtype_bits(rng.standard_normal((T, H), dtype=np.float32), dtype))


def make_shared_expert(spec: dict, I_shared: int, seed: int) -> dict:
    """One shared expert for ``spec``'s layer, in the experts' packed format
    (widths, block size, scale range and zero-point mode of ``spec``), plus
    its gate vector [H] drawn N(0, 1/H) and rounded to the dtype.  Keys:
    fc1_codes [1, 2*I_shared, H*b/8], fc1_scales, fc1_zp, fc2_codes
    [1, H, I_shared*b/8], fc2_scales, fc2_zp, gate [H], I."""
    sub = dict(spec, T=1, I=I_shared, E=1)
    drawn = make_inputs(sub, seed)
    rng = np.random.default_rng(seed + 1)
    H = spec["H"]
    gate = rng.standard_normal(H, dtype=np.float32) * np.float32(1.0 / math.sqrt(H))
    out = {k: v for k, v in drawn.items() if k.startswith("fc")}
    out["gate"] = np.ascontiguousarray(_to_dtype_bits(gate, spec["dtype"]))
    out["I"] = I_shared
    return out


def seed_for(i: int) -> int:
    """Default seed of named workload ``i``."""
    return 1000 + i
