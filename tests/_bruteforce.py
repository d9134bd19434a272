"""Independent brute-force definitions used to pin the CPU oracle.

Nothing here is shared with ``oracle/`` or with the GPU library.  Each routine
takes a different route to the same quantity than the oracle does:

* totalOrder of float32 values from the IEEE 754 predicate's definition (sign,
  NaN class, magnitude), not from integer bit tricks;
* code unpacking through ``numpy.unpackbits`` as a little-endian bit stream;
* the layer as dense dequantized tensors and numpy/torch float64 matmuls over
  *all* experts, combined with a one-hot routing matrix.
"""
from __future__ import annotations

import math
import struct

import numpy as np
import torch
import torch.nn.functional as F


def total_order_position(x: float) -> tuple:
    """Sort key realising IEEE 754 totalOrder on float32 values.

    Negative NaNs sit below -inf (larger payload lower), positive NaNs above
    +inf (larger payload higher), and -0 directly below +0."""
    bits = struct.unpack("<I", struct.pack("<f", x))[0]
    negative = bits >> 31
    exponent = (bits >> 23) & 0xFF
    fraction = bits & 0x7FFFFF
    if exponent == 0xFF and fraction != 0:
        return (-2, -fraction, 0) if negative else (2, fraction, 0)
    value = struct.unpack("<f", struct.pack("<I", bits))[0]
    return (0, value, 0 if negative else 1)


def route(logits: np.ndarray, k: int):
    """Expert ids chosen by a stable descending sort on totalOrder (ties keep the lower index)."""
    T, E = logits.shape
    ids = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        row = [float(v) for v in logits[t]]
        order = sorted(range(E), key=lambda e: total_order_position(row[e]), reverse=True)
        ids[t] = order[:k]
    return ids


def route_weights(logits: np.ndarray, ids: np.ndarray, normalize: int) -> np.ndarray:
    """Softmax weights of the selected experts (torch float64 softmax)."""
    lg = torch.from_numpy(logits.astype(np.float64))
    idx = torch.from_numpy(ids.astype(np.int64))
    if normalize:
        return torch.softmax(torch.gather(lg, 1, idx), dim=1).numpy()
    return torch.gather(torch.softmax(lg, dim=1), 1, idx).numpy()


def unpack_bitstream(packed: np.ndarray, bits: int, count: int) -> np.ndarray:
    """Read ``count`` unsigned ``bits``-wide fields from each row's little-endian bit stream."""
    stream = np.unpackbits(packed, axis=-1, bitorder="little")
    fields = stream[..., : count * bits].reshape(packed.shape[:-1] + (count, bits)).astype(np.int64)
    return (fields << np.arange(bits, dtype=np.int64)).sum(axis=-1)


def widen(bits: np.ndarray, dtype: int) -> np.ndarray:
    """fp16 (dtype 1) or bf16 (dtype 2) bit patterns to float64 via numpy / torch."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == 1:
        return bits.view(np.float16).astype(np.float64)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def dense_weights(codes, scales, zp, K, bits, block_size, zpo, dtype) -> np.ndarray:
    """Every expert's dequantized weights [E, N, K] in float64."""
    q = unpack_bitstream(codes, bits, K).astype(np.float64)
    n_blocks = K // block_size
    s = widen(scales, dtype)
    if zp is not None:
        if bits == 3:
            z = zp.astype(np.float64)
        else:
            z = unpack_bitstream(zp, bits, n_blocks).astype(np.float64)
    elif not math.isnan(zpo):
        z = np.full(s.shape, zpo)
    else:
        z = np.full(s.shape, float(2 ** (bits - 1)))
    z_full = np.repeat(z, block_size, axis=-1)
    s_full = np.repeat(s, block_size, axis=-1)
    return (q - z_full) * s_full


def gate_activation(g: np.ndarray, act: int) -> np.ndarray:
    t = torch.from_numpy(g)
    if act == 1:
        return F.gelu(t, approximate="tanh").numpy()
    return F.silu(t).numpy()


def layer(inp: dict, spec: dict) -> np.ndarray:
    """Whole-layer output [T, H] in float64: all experts computed densely, then mixed.

    Options (default SwiGLU/GeGLU parameters only): expert biases, the three
    gate/up layouts (swiglu_fusion 1 interleaved, 2 halves, 0 a separate fc3),
    and router_weights as the weights of the selected experts."""
    T, H, I, E, k = spec["T"], spec["H"], spec["I"], spec["E"], spec["k"]
    dt = spec["dtype"]
    fusion = spec.get("swiglu_fusion", 1)
    x = widen(inp["hidden"], dt)
    w1 = dense_weights(inp["fc1_codes"], inp["fc1_scales"], inp["fc1_zp"], H, spec["fc1_bits"],
                       spec["block_size"], spec["zpo"], dt)
    w2 = dense_weights(inp["fc2_codes"], inp["fc2_scales"], inp["fc2_zp"], I, spec["fc2_bits"],
                       spec["block_size"], spec["zpo"], dt)
    if fusion == 0:
        w3 = dense_weights(inp["fc3_codes"], inp["fc3_scales"], inp["fc3_zp"], H,
                           spec.get("fc3_bits", spec["fc1_bits"]), spec["block_size"], spec["zpo"], dt)
    ids = route(inp["logits"], k)
    rw = inp.get("router_weights")
    if rw is None:
        wts = route_weights(inp["logits"], ids, spec["normalize"])
    else:
        picked = np.take_along_axis(rw.astype(np.float64), ids.astype(np.int64), 1)
        den = picked.sum(axis=1, keepdims=True) if spec["normalize"] else np.ones((T, 1))
        wts = np.where(den == 0, 0.0, picked / np.where(den == 0, 1.0, den))
    mix = np.zeros((T, E))
    for t in range(T):
        for s in range(k):
            mix[t, ids[t, s]] += wts[t, s]
    b1, b2, b3 = inp.get("fc1_bias"), inp.get("fc2_bias"), inp.get("fc3_bias")
    out = np.zeros((T, H))
    for e in range(E):
        y1 = x @ w1[e].T + (0.0 if b1 is None else b1[e].astype(np.float64))
        if fusion == 1:
            g, u = y1[:, 0::2], y1[:, 1::2]
        elif fusion == 2:
            g, u = y1[:, :I], y1[:, I:]
        else:
            g, u = y1, x @ w3[e].T + (0.0 if b3 is None else b3[e].astype(np.float64))
        a = gate_activation(g, spec["act"]) * u
        y2 = a @ w2[e].T + (0.0 if b2 is None else b2[e].astype(np.float64))
        out += mix[:, e:e + 1] * y2
    return out


def group(ids: np.ndarray, E: int, m_tile: int, n_tile: int, N: int):
    """Offsets, stable expert-sorted routes and (expert, m, n) work-list by plain Python sorting."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    valid = [r for r in range(len(flat)) if 0 <= flat[r] < E]
    order = sorted(valid, key=lambda r: (flat[r], r))
    counts = [0] * E
    for r in valid:
        counts[flat[r]] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    items = []
    n_tiles = -(-N // n_tile)
    for e in range(E):
        for m in range(-(-counts[e] // m_tile)):
            for n in range(n_tiles):
                items.append((e, m, n))
    return (np.array(offsets, dtype=np.int32), np.array(order, dtype=np.int32),
            np.array(items, dtype=np.int32).reshape(-1, 3))
