"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: every expected value comes
from a golden fixture quoting the pages, a closed form, an invariant, a
library routine (numpy / torch), or the independent brute force in
``tests/_bruteforce.py``.
"""
from __future__ import annotations

import math
import os
import struct

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import qmoe_synth as synth
from tests import _bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    fields = {}
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, *rest = line.split()
            try:
                rows.append([float(head)] + [float(v) for v in rest])
            except ValueError:
                fields[head] = rest
    return fields, rows


def _pack_bitstream(values, bits):
    """Pack small unsigned ints into a little-endian bit stream (test-side encoder)."""
    stream = np.zeros(len(values) * bits, dtype=np.uint8)
    for i, v in enumerate(values):
        for b in range(bits):
            stream[i * bits + b] = (int(v) >> b) & 1
    pad = (-len(stream)) % 8
    stream = np.concatenate([stream, np.zeros(pad, dtype=np.uint8)])
    return np.packbits(stream, bitorder="little")


# ---------------------------------------------------------------- widening
def test_fp16_widening_matches_numpy_for_every_pattern():
    pats = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.widen(pats, 1)
    ref = pats.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_bf16_widening_matches_torch_for_every_pattern():
    pats = np.arange(1 << 16, dtype=np.uint16)
    got = oracle.widen(pats, 2)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


# ---------------------------------------------------------------- unpacking
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_unpack_matches_little_endian_bitstream(bits):
    rng = np.random.default_rng(7 + bits)
    K = 256
    codes = rng.integers(0, 256, size=(5, K * bits // 8), dtype=np.uint8)
    q, _ = oracle.dequant(codes, np.zeros((5, K // 32), np.uint16), None, K, bits, 32,
                          math.nan, 1, want_weights=False)
    assert np.array_equal(q, bf.unpack_bitstream(codes, bits, K))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_pack_unpack_round_trip(bits):
    rng = np.random.default_rng(11 + bits)
    K = 128
    vals = rng.integers(0, 1 << bits, size=K)
    packed = _pack_bitstream(vals, bits)[None, :]
    q, _ = oracle.dequant(packed, np.zeros((1, K // 16), np.uint16), None, K, bits, 16,
                          math.nan, 1, want_weights=False)
    assert np.array_equal(q[0], vals)


def test_int3_group_layout_is_24_bit_little_endian_word():
    # one 3-byte group holding codes 0..7 in order: word = sum j << 3j
    word = sum(j << (3 * j) for j in range(8))
    group = np.array([[word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF]], dtype=np.uint8)
    q, _ = oracle.dequant(group, np.zeros((1, 1), np.uint16), None, 8, 3, 8, math.nan, 1,
                          want_weights=False)
    assert list(q[0]) == list(range(8))


# ---------------------------------------------------------------- zero points
def test_fractional_zero_point_worked_example():
    fields, _ = _golden("fractional_zero_point_int2.txt")
    bits = int(fields["bits"][0])
    zpo = float(fields["zero_point_offset"][0])
    codes = [int(v) for v in fields["codes"]]
    expect = [float(v) for v in fields["dequant_over_scale"]]
    # 16 elements: the four codes repeated, one block of 16, scale 0.01 in fp16
    vals = codes * 4
    packed = _pack_bitstream(vals, bits)[None, :]
    scale = np.array([[np.float16(0.01)]], dtype=np.float16).view(np.uint16)
    q, w = oracle.dequant(packed, scale, None, 16, bits, 16, zpo, 1)
    s = float(np.float16(0.01))
    assert list(q[0, :4]) == codes
    assert np.array_equal(w[0, :4], np.array(expect) * s)


def test_symmetric_centres():
    _, rows = _golden("symmetric_centres.txt")
    for bits_f, centre in rows:
        bits = int(bits_f)
        vals = [int(centre)] * 8 + [0] * 8
        packed = _pack_bitstream(vals, bits)[None, :]
        scale = np.array([[np.float16(0.5)]], dtype=np.float16).view(np.uint16)
        _, w = oracle.dequant(packed, scale, None, 16, bits, 16, math.nan, 1)
        assert np.all(w[0, :8] == 0.0)
        assert np.all(w[0, 8:] == -centre * 0.5)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_uint8_zero_points_take_precedence_over_offset(bits):
    rng = np.random.default_rng(3)
    K, bs = 64, 16
    nb = K // bs
    codes = rng.integers(0, 256, size=(3, K * bits // 8), dtype=np.uint8)
    zvals = rng.integers(0, 1 << bits, size=(3, nb))
    if bits == 3:
        zp = zvals.astype(np.uint8)
    else:
        zp = np.stack([_pack_bitstream(r, bits) for r in zvals])
    scales = np.full((3, nb), np.float16(1.0), dtype=np.float16).view(np.uint16)
    q, w = oracle.dequant(codes, scales, zp, K, bits, bs, 1.5, 1)
    expect = q - np.repeat(zvals, bs, axis=1)
    assert np.array_equal(w, expect.astype(np.float64))


def test_dequant_matches_dense_bruteforce_all_modes():
    rng = np.random.default_rng(5)
    for bits in (1, 2, 3, 4, 8):
        for dtype in (1, 2):
            for mode in ("sym", "zpo", "u8"):
                K, bs, N = 128, 32, 6
                codes = rng.integers(0, 256, size=(2, N, K * bits // 8), dtype=np.uint8)
                s32 = rng.uniform(0.005, 0.02, size=(2, N, K // bs)).astype(np.float32)
                scales = synth._to_dtype_bits(s32, dtype)
                zp = None
                zpo = math.nan
                if mode == "u8":
                    zp = synth._draw_zero_points(rng, 2, N, K // bs, bits, 0, (1 << bits) - 1)
                elif mode == "zpo":
                    zpo = 1.5 if bits == 2 else 3.25
                _, w = oracle.dequant(codes, scales, zp, K, bits, bs, zpo, dtype)
                ref = bf.dense_weights(codes, scales, zp, K, bits, bs, zpo, dtype)
                assert np.array_equal(w, ref), (bits, dtype, mode)


# ---------------------------------------------------------------- activation parameters
def test_swiglu_defaults_are_silu_and_geglu_ignores_parameters():
    g = np.linspace(-9.0, 9.0, 37)
    u = np.linspace(2.0, -3.0, 37)
    silu = F.silu(torch.from_numpy(g)).numpy() * u
    gelu = F.gelu(torch.from_numpy(g), approximate="tanh").numpy() * u
    for i in range(g.size):
        assert math.isclose(oracle.gated(g[i], u[i], 0), silu[i], rel_tol=1e-14, abs_tol=1e-300)
        v = oracle.gated(g[i], u[i], 1, alpha=3.0, beta=0.5, limit=0.25)
        assert math.isclose(v, gelu[i], rel_tol=1e-14, abs_tol=1e-300)


def test_swiglu_alpha_beta_limit_properties():
    # [qmoe.rs, swiglu_value]: gate bounded above by the limit, linear part
    # clamped to [-limit, limit], value = g' * sigmoid(alpha g') * (u' + beta)
    L = 1.5
    for g in (-4.0, -0.5, 0.0, 0.7, 1.2):
        for u in (-1.0, 0.3, 1.4):
            # alpha = 2: g * sigmoid(2g) = silu(2g) / 2 (textbook routine), inside the limit
            want = F.silu(torch.tensor(2.0 * g, dtype=torch.float64)).item() / 2.0 * u
            assert math.isclose(oracle.gated(g, u, 0, alpha=2.0, limit=L), want, rel_tol=1e-14,
                                abs_tol=1e-300)
            # beta enters linearly: f(beta) - f(0) = beta * f(u = 1)
            d = oracle.gated(g, u, 0, beta=0.75, limit=L) - oracle.gated(g, u, 0, limit=L)
            assert math.isclose(d, 0.75 * oracle.gated(g, 1.0, 0, limit=L), rel_tol=1e-12,
                                abs_tol=1e-15)
    # above the limit the gate no longer matters; the linear part saturates at +-limit
    assert oracle.gated(7.0, 0.5, 0, limit=L) == oracle.gated(L, 0.5, 0, limit=L)
    assert oracle.gated(0.8, 9.0, 0, limit=L) == oracle.gated(0.8, L, 0, limit=L)
    assert oracle.gated(0.8, -9.0, 0, limit=L) == oracle.gated(0.8, -L, 0, limit=L)
    # a NaN linear part stays NaN; a NaN gate is bounded to the limit (fmin)
    assert math.isnan(oracle.gated(0.8, float("nan"), 0, limit=L))
    assert oracle.gated(float("nan"), 0.5, 0, limit=L) == oracle.gated(L, 0.5, 0, limit=L)


# ---------------------------------------------------------------- operator options
OPTION_CASES = [
    dict(bias=True),
    dict(swiglu_fusion=2),
    dict(swiglu_fusion=0),
    dict(swiglu_fusion=0, bias=True, fc3_bits=2),
    dict(router_weights=True),
    dict(router_weights=True, normalize=0),
    dict(fc1_bits=8, fc2_bits=1),
    dict(fc1_bits=1, fc2_bits=8, zp_mode="u8", zp_range=(0, 1)),
]


@pytest.mark.parametrize("case", range(len(OPTION_CASES)))
def test_layer_options_match_dense_bruteforce(case):
    opts = dict(OPTION_CASES[case])
    spec = synth.custom(T=9, H=64, I=32, E=5, k=2, block_size=16, act=case % 2,
                        dtype=1 + case % 2, **opts)
    if spec.get("zp_mode") == "u8" and spec.get("zp_range") is None:
        spec["zp_range"] = (0, 3)
    inp = synth.make_inputs(spec, 70 + case)
    got = oracle.forward(inp, spec)
    ref = bf.layer(inp, spec)
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_router_weights_select_by_logits_and_weigh_by_aggregation():
    rng = np.random.default_rng(12)
    logits = rng.standard_normal((30, 16)).astype(np.float32)
    rw = rng.random((30, 16), dtype=np.float32)
    rw[3, :] = 0.0  # all-zero aggregation: weights 0
    ids0, _ = oracle.route(logits, 4, 1)
    ids, w = oracle.route(logits, 4, 0, router_weights=rw)
    assert np.array_equal(ids, ids0)  # selection by the logits alone
    assert np.array_equal(w, np.take_along_axis(rw, ids.astype(np.int64), 1).astype(np.float64))
    ids, w = oracle.route(logits, 4, 1, router_weights=rw)
    assert np.array_equal(ids, ids0)
    ok = np.arange(30) != 3
    assert np.allclose(w[ok].sum(axis=1), 1.0, rtol=0, atol=1e-15)
    picked = np.take_along_axis(rw, ids.astype(np.int64), 1).astype(np.float64)
    assert np.allclose(w[ok] * picked[ok][:, :1], picked[ok] * w[ok][:, :1], rtol=1e-14, atol=0)
    assert np.all(w[3] == 0.0)


# ---------------------------------------------------------------- routing
def _adversarial_logits():
    nan_pos = struct.unpack("<f", struct.pack("<I", 0x7FC00001))[0]
    nan_pos_big = struct.unpack("<f", struct.pack("<I", 0x7FFFFFFF))[0]
    nan_neg = struct.unpack("<f", struct.pack("<I", 0xFFC00000))[0]
    nan_neg_big = struct.unpack("<f", struct.pack("<I", 0xFFFFFFFF))[0]
    inf = float("inf")
    rows = [
        [0.0, -0.0, 0.0, -0.0, 1.0, -1.0, 0.0, -0.0],
        [-0.0, -0.0, 0.0, -1e-45, 1e-45, -inf, inf, 0.0],
        [nan_pos, inf, nan_neg, -inf, 3.0, nan_pos_big, nan_neg_big, 2.0],
        [1.5] * 8,
        [-inf] * 8,
        [nan_neg, nan_neg_big, -inf, -3.4e38, -1.0, -1e-38, -0.0, nan_neg],
        [2.0, 2.0, 1.0, 2.0, 1.0, 3.0, 3.0, 1.0],
        [nan_pos, nan_pos, nan_pos_big, nan_pos_big, 0.0, 0.0, -0.0, -0.0],
    ]
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("k", [1, 2, 3, 5, 8])
def test_route_ids_match_ieee_total_order_bruteforce(k):
    rng = np.random.default_rng(k)
    logits = np.concatenate([_adversarial_logits(),
                             rng.standard_normal((40, 8)).astype(np.float32),
                             np.round(rng.standard_normal((40, 8)) * 2).astype(np.float32)])
    ids, _ = oracle.route(logits, k, 1)
    assert np.array_equal(ids, bf.route(logits, k))


def test_route_key_orders_like_total_order():
    rng = np.random.default_rng(9)
    vals = list(_adversarial_logits().reshape(-1)) + list(
        rng.standard_normal(200).astype(np.float32))
    for a in vals[:60]:
        for b in vals[::7]:
            ka, kb = oracle.route_key(a), oracle.route_key(b)
            pa, pb = bf.total_order_position(float(a)), bf.total_order_position(float(b))
            assert (ka < kb) == (pa < pb) and (ka == kb) == (pa == pb)


def test_route_all_equal_logits_picks_lowest_indices():
    logits = np.full((4, 16), 0.25, dtype=np.float32)
    for k in (1, 4, 16):
        ids, w = oracle.route(logits, k, 1)
        assert np.array_equal(ids, np.tile(np.arange(k), (4, 1)))
        assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-15)


def test_route_k_equals_e_is_a_permutation_and_softmax():
    rng = np.random.default_rng(21)
    logits = rng.standard_normal((30, 12)).astype(np.float32)
    ids, w = oracle.route(logits, 12, 0)
    assert all(sorted(r) == list(range(12)) for r in ids.tolist())
    ref = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    assert np.allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-14, atol=0)


@pytest.mark.parametrize("E,k", [(8, 2), (512, 10), (64, 7), (1000, 1)])
def test_route_weights_invariants(E, k):
    rng = np.random.default_rng(E + k)
    logits = (rng.standard_normal((25, E)) * 2).astype(np.float32)
    ids, w = oracle.route(logits, k, 1)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=4e-16 * k)
    # the best expert's numerator is exp(0) = 1, so w0 = 1 / sum
    assert np.all(np.diff(w, axis=1) <= 0)
    ref = bf.route_weights(logits, ids, 1)
    assert np.allclose(w, ref, rtol=1e-14, atol=0)
    ids_u, w_u = oracle.route(logits, k, 0)
    assert np.array_equal(ids_u, ids)
    assert np.allclose(w_u, bf.route_weights(logits, ids, 0), rtol=1e-13, atol=0)
    assert np.all(w_u.sum(axis=1) <= 1.0 + 1e-15)


def _f32_bits(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


def test_route_weights_on_non_finite_rows():
    # [qmoe.rs, qmoe_route]: the maximum is a running fmaxf over the row, so a
    # NaN logit never becomes m; the weights are plain IEEE arithmetic on
    # exp(l - m).  Expected values come from torch float64 softmax over the
    # selected finite logits, or are NaN where IEEE arithmetic makes them NaN.
    inf, nan_neg, nan_neg2 = float("inf"), _f32_bits(0xFFC00000), _f32_bits(0xFFFFFFFF)
    nan_pos = _f32_bits(0x7FC00001)
    finite_rows = np.array([
        [1.0, 0.5, nan_neg, 0.2, -inf, 0.1, nan_neg2, -0.3],   # -NaN, -inf unselected
        [nan_neg, -inf, -2.0, 3.0, -inf, 2.5, nan_neg, -1.0],
        [-inf, -inf, -inf, 0.0, -inf, -inf, -0.0, -inf],       # finite ones selected first
    ], dtype=np.float32)
    for k in (1, 2, 3):
        ids, w = oracle.route(finite_rows, k, 1)
        assert np.array_equal(ids, bf.route(finite_rows, k))
        sel = np.take_along_axis(finite_rows.astype(np.float64), ids.astype(np.int64), 1)
        assert not np.any(np.isnan(sel)) and np.all(np.isfinite(sel[:, 0]))
        ref = torch.softmax(torch.from_numpy(sel), dim=1).numpy()
        assert np.allclose(w, ref, rtol=1e-14, atol=0)
    # normalize = 0: the denominator sums exp(l - m) over every expert; -inf
    # terms are 0, and one NaN anywhere makes every weight of the row NaN
    no_nan = np.array([[1.0, -inf, 0.5, 0.25, -inf, -1.0, 2.0, 0.0]], dtype=np.float32)
    ids, w = oracle.route(no_nan, 3, 0)
    ref = torch.softmax(torch.from_numpy(no_nan.astype(np.float64)), dim=1).numpy()
    assert np.allclose(w, np.take_along_axis(ref, ids.astype(np.int64), 1), rtol=1e-14, atol=0)
    _, w = oracle.route(finite_rows[:2], 2, 0)
    assert np.all(np.isnan(w))
    # a selected +inf or +NaN: exp(inf - inf) and exp(NaN - m) are NaN, and
    # with normalize = 1 so is the denominator, hence every weight of the row
    bad = np.array([[0.5, inf, 1.0, -1.0], [nan_pos, 2.0, 1.0, 0.0], [-inf, -inf, -inf, -inf]],
                   dtype=np.float32)
    for normalize in (0, 1):
        ids, w = oracle.route(bad, 2, normalize)
        assert np.array_equal(ids, bf.route(bad, 2))
        assert np.all(np.isnan(w)), (normalize, w)


def test_route_top1_normalized_weight_is_exactly_one():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((50, 32)).astype(np.float32)
    _, w = oracle.route(logits, 1, 1)
    assert np.all(w == 1.0)


# ---------------------------------------------------------------- router projection
@pytest.mark.parametrize("dtype", [1, 2])
def test_router_logits_match_torch_float64_linear(dtype):
    # the oracle's plain loop against torch's float64 matmul on the same values
    T, H, E = 7, 96, 13
    x = synth.make_hidden(T, H, dtype, 5)
    w = synth.make_router_weights(E, H, dtype, 6)
    got = oracle.router_logits(x, w, dtype)
    ref = F.linear(torch.from_numpy(bf.widen(x, dtype)), torch.from_numpy(bf.widen(w, dtype))).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-15)


def test_router_logits_one_hot_rows_pick_hidden_elements():
    # weight row e = one-hot at h_e with value 1: logit e is exactly x[t, h_e];
    # a row of twos doubles the sum of the row (exact: small integers)
    T, H, E = 4, 64, 5
    x16 = (np.arange(T * H, dtype=np.float32).reshape(T, H) % 17 - 8).astype(np.float16)
    x = x16.view(np.uint16)
    w = np.zeros((E, H), dtype=np.float16)
    picks = [0, 7, 31, 63]
    for e, h in enumerate(picks):
        w[e, h] = 1.0
    w[4, :] = 2.0
    got = oracle.router_logits(x, w.view(np.uint16), 1)
    x64 = x16.astype(np.float64)
    assert np.array_equal(got[:, :4], x64[:, picks])
    assert np.array_equal(got[:, 4], 2.0 * x64.sum(axis=1))
    assert np.array_equal(oracle.router_logits(np.zeros_like(x), w.view(np.uint16), 1), np.zeros((T, E)))


# ---------------------------------------------------------------- shared expert
@pytest.mark.parametrize("act,dtype,zp_mode", [(0, 1, "sym"), (1, 2, "u8"), (0, 2, "zpo")])
def test_shared_expert_matches_dense_torch(act, dtype, zp_mode):
    # sigmoid(x . g) * W2 (act(W1g x) * W1u x) with dense float64 torch ops on
    # the brute-force dequantized weights
    spec = synth.custom(T=6, H=64, I=32, E=4, k=2, fc1_bits=4, fc2_bits=2, block_size=16,
                        dtype=dtype, act=act, zp_mode=zp_mode, zpo=1.5 if zp_mode == "zpo" else math.nan,
                        zp_range=(0, 3))
    inp = synth.make_inputs(spec, 8)
    sh = synth.make_shared_expert(spec, 48, 9)
    got = oracle.shared_expert(inp, sh, spec)
    H, Is = spec["H"], 48
    w1 = bf.dense_weights(sh["fc1_codes"], sh["fc1_scales"], sh["fc1_zp"], H, 4, 16,
                          spec["zpo"], dtype)[0]
    w2 = bf.dense_weights(sh["fc2_codes"], sh["fc2_scales"], sh["fc2_zp"], Is, 2, 16,
                          spec["zpo"], dtype)[0]
    x = torch.from_numpy(bf.widen(inp["hidden"], dtype))
    g = torch.sigmoid(x @ torch.from_numpy(bf.widen(sh["gate"], dtype)))
    y1 = x @ torch.from_numpy(w1).T
    gate, up = y1[:, 0::2], y1[:, 1::2]
    a = (F.silu(gate) if act == 0 else F.gelu(gate, approximate="tanh")) * up
    ref = (g[:, None] * (a @ torch.from_numpy(w2).T)).numpy()
    assert np.allclose(got, ref, rtol=1e-11, atol=1e-13)


def test_shared_expert_zero_gate_halves_the_ffn():
    # a zero gate vector: sigmoid(0) = 1/2 exactly, so the contribution is half
    # the plain shared FFN, which is the layer output with one expert (E = 1,
    # k = 1 routes every token to it with weight exactly 1)
    spec = synth.custom(T=5, H=64, I=32, E=1, k=1, fc1_bits=4, fc2_bits=4, block_size=32)
    inp = synth.make_inputs(spec, 3)
    sh = {"fc1_codes": inp["fc1_codes"], "fc1_scales": inp["fc1_scales"], "fc1_zp": None,
          "fc2_codes": inp["fc2_codes"], "fc2_scales": inp["fc2_scales"], "fc2_zp": None,
          "gate": np.zeros(64, dtype=np.uint16), "I": 32}
    half = oracle.shared_expert(inp, sh, spec)
    ref = bf.layer(inp, spec)
    assert np.allclose(half, 0.5 * ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- grouping
@pytest.mark.parametrize("E,R,m_tile,n_tile,N", [(8, 64, 16, 64, 200), (512, 60, 16, 32, 64),
                                                 (3, 1, 128, 128, 128), (8, 1000, 128, 256, 4096),
                                                 (5, 0, 16, 16, 16)])
def test_group_matches_python_sort(E, R, m_tile, n_tile, N):
    rng = np.random.default_rng(R + E)
    ids = rng.integers(0, E, size=R).astype(np.int32)
    if R > 3:
        ids[::5] = 0  # crowd one expert
    off, srt, wl, n = oracle.group(ids, E, m_tile, n_tile, N)
    boff, bsrt, bwl = bf.group(ids, E, m_tile, n_tile, N)
    assert np.array_equal(off, boff) and np.array_equal(srt, bsrt)
    assert n == len(bwl) and np.array_equal(wl, bwl)
    assert off[E] == R


def test_group_skips_out_of_range_ids():
    ids = np.array([3, -1, 0, 7, 3, 2, 9], dtype=np.int32)
    off, srt, wl, n = oracle.group(ids, 4, 2, 8, 8)
    boff, bsrt, bwl = bf.group(ids, 4, 2, 8, 8)
    assert np.array_equal(off, boff) and np.array_equal(srt, bsrt) and np.array_equal(wl, bwl)
    assert off[4] == 4


# ---------------------------------------------------------------- the layer
LAYER_CASES = [
    dict(T=5, H=64, I=32, E=4, k=2, fc1_bits=4, fc2_bits=4, block_size=16, dtype=1, act=0),
    dict(T=4, H=32, I=64, E=3, k=3, fc1_bits=2, fc2_bits=2, block_size=32, dtype=1, act=1,
         zp_mode="zpo", zpo=1.5),
    dict(T=6, H=64, I=48, E=6, k=2, fc1_bits=3, fc2_bits=2, block_size=16, dtype=2, act=0),
    dict(T=3, H=48, I=32, E=5, k=4, fc1_bits=4, fc2_bits=3, block_size=16, dtype=2, act=1,
         zp_mode="u8", zp_range=(0, 7)),
    dict(T=7, H=32, I=32, E=8, k=1, fc1_bits=2, fc2_bits=4, block_size=32, dtype=1, act=0,
         normalize=0),
]


@pytest.mark.parametrize("case", range(len(LAYER_CASES)))
def test_layer_matches_dense_bruteforce(case):
    spec = synth.custom(**LAYER_CASES[case])
    inp = synth.make_inputs(spec, 100 + case)
    got = oracle.forward(inp, spec)
    ref = bf.layer(inp, spec)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_layer_token_subset_equals_full_rows():
    spec = synth.custom(**LAYER_CASES[2])
    inp = synth.make_inputs(spec, 55)
    full = oracle.forward(inp, spec)
    sub = oracle.forward(inp, spec, tokens=np.array([5, 0, 3]))
    assert np.array_equal(sub, full[[5, 0, 3]])


@pytest.mark.parametrize("act", [0, 1])
def test_single_expert_top1_is_dense_gated_ffn(act):
    # E=1, k=1, normalize=1: weight is exactly 1 and the layer is the textbook
    # W2 (act(Wg x) * (Wu x)) with Wg the even and Wu the odd fc1 rows.
    spec = synth.custom(T=6, H=64, I=32, E=1, k=1, fc1_bits=4, fc2_bits=4, block_size=16,
                        dtype=1, act=act)
    inp = synth.make_inputs(spec, 77)
    got = oracle.forward(inp, spec)
    x = torch.from_numpy(bf.widen(inp["hidden"], 1))
    w1 = torch.from_numpy(bf.dense_weights(inp["fc1_codes"], inp["fc1_scales"], None, 64, 4, 16,
                                           math.nan, 1)[0])
    w2 = torch.from_numpy(bf.dense_weights(inp["fc2_codes"], inp["fc2_scales"], None, 32, 4, 16,
                                           math.nan, 1)[0])
    wg, wu = w1[0::2], w1[1::2]
    gate = F.gelu(x @ wg.T, approximate="tanh") if act else F.silu(x @ wg.T)
    ref = ((gate * (x @ wu.T)) @ w2.T).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_all_tokens_on_same_experts_is_weighted_dense_gemm():
    spec = synth.custom(T=8, H=32, I=32, E=4, k=2, fc1_bits=4, fc2_bits=4, block_size=16, dtype=1)
    inp = synth.make_inputs(spec, 8)
    logits = np.tile(np.array([[0.1, 3.0, -2.0, 2.5]], np.float32), (8, 1))
    logits[:, 1] += np.linspace(0, 0.1, 8).astype(np.float32)
    inp["logits"] = logits
    got = oracle.forward(inp, spec)
    x = bf.widen(inp["hidden"], 1)
    w1 = bf.dense_weights(inp["fc1_codes"], inp["fc1_scales"], None, 32, 4, 16, math.nan, 1)
    w2 = bf.dense_weights(inp["fc2_codes"], inp["fc2_scales"], None, 32, 4, 16, math.nan, 1)
    out = np.zeros((8, 32))
    l = logits.astype(np.float64)
    for t in range(8):
        a, b = np.exp(l[t, 1]), np.exp(l[t, 3])
        for e, wt in ((1, a / (a + b)), (3, b / (a + b))):
            y1 = w1[e] @ x[t]
            g = y1[0::2]
            act = g / (1 + np.exp(-g)) * y1[1::2]
            out[t] += wt * (w2[e] @ act)
    assert np.allclose(got, out, rtol=1e-12, atol=1e-13)


def test_named_workload_shapes():
    # the five named workloads draw consistent shapes
    for i in (1, 2):
        spec = synth.workload(i)
        inp = synth.make_inputs(spec, synth.seed_for(i))
        E, I, H = spec["E"], spec["I"], spec["H"]
        assert inp["fc1_codes"].shape == (E, 2 * I, H * spec["fc1_bits"] // 8)
        assert inp["fc2_codes"].shape == (E, H, I * spec["fc2_bits"] // 8)
        assert inp["fc1_scales"].shape == (E, 2 * I, H // spec["block_size"])
