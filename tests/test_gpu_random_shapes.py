"""GPU parity over seeded random layer shapes: widths, block sizes, zero-point
modes, dtypes, activations, expert counts, top-k and token counts drawn
together, so that the path selection (decode plan, streamed and row-block
decode, the three prefill tiles, fc2 K splits, scale staging) meets
combinations the hand-written cases do not list; a second set adds random
operator options (gate/up layouts with fc3, biases, router_weights, SwiGLU
alpha/beta/limit).  Each layer is compared with the oracle on sampled
tokens (first, last and random ones) at the layer bound of the other parity
tests.  A third set draws small decode layers (at most 16 tokens and 32
experts, 2/4-bit, K a power of two up to 2048), often with fewer routes than
experts, for the streamed decode kernels; every fourth one keeps expert 0
out of every token's choice.  Sizes are capped so that one case costs well
under a second of host work."""
from __future__ import annotations

import math

import numpy as np
import pytest

import qmoe_synth as synth
from tests.test_gpu_options import _check as _options_check
from tests.test_gpu_parity import _layer_check

pytestmark = pytest.mark.gpu

N_CASES = 48
N_OPTION_CASES = 24
N_STREAM_CASES = 24


def _draw(i: int) -> tuple[dict, np.ndarray]:
    rng = np.random.default_rng(4242 + i)
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    mult = max(128, bs)
    H = int(mult * rng.integers(1, max(2, 4096 // mult) + 1))
    I = int(mult * rng.integers(1, max(2, 4096 // mult) + 1))
    E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 33, 64, 100, 256, 512]))
    k = int(rng.integers(1, min(E, 10) + 1))
    T = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 24, 40, 64, 100, 300, 700, 1500]))
    b1, b2 = (int(b) for b in rng.choice([1, 2, 3, 4, 8], size=2))
    # packed weights <= 96 MB
    while E * H * I * (2 * b1 + b2) / 8 > 96e6:
        if E > 16:
            E //= 2
        elif H >= I and H > mult:
            H = max(mult, H // 2 // mult * mult)
        elif I > mult:
            I = max(mult, I // 2 // mult * mult)
        else:
            break
    k = min(k, E)
    zp_mode = str(rng.choice(["sym", "u8", "zpo"]))
    mb = min(b1, b2)
    # a fractional zero point inside the code range
    zpo = float(rng.choice([z for z in (0.5, 1.5, 3.0, 7.25) if z <= (1 << mb) - 1] or [0.5]))
    # weights of O(1 / sqrt(K)) keep the layer output well inside fp16's range
    s0 = 2.0 / ((1 << (max(b1, b2) - 1)) * math.sqrt(max(H, I)))
    spec = synth.custom(T=T, H=H, I=I, E=E, k=k, fc1_bits=b1, fc2_bits=b2, block_size=bs,
                        dtype=int(rng.integers(1, 3)), act=int(rng.integers(0, 2)),
                        normalize=int(rng.integers(0, 2)), zp_mode=zp_mode,
                        zpo=zpo if zp_mode == "zpo" else math.nan, zp_range=(0, (1 << mb) - 1),
                        scale_range=(0.5 * s0, 1.5 * s0), name=f"random{i}")
    ntok = int(max(2, min(T, 16, 1e9 // (3 * k * H * I))))
    tokens = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=ntok)])).astype(np.int64)
    return spec, tokens


@pytest.mark.parametrize("i", range(N_CASES))
def test_layer_random_shape(i):
    spec, tokens = _draw(i)
    print(f"  T={spec['T']} H={spec['H']} I={spec['I']} E={spec['E']} k={spec['k']} "
          f"bits={spec['fc1_bits']}/{spec['fc2_bits']} bs={spec['block_size']} zp={spec['zp_mode']} "
          f"dtype={spec['dtype']} act={spec['act']} normalize={spec['normalize']}", flush=True)
    _layer_check(spec, 8800 + i, tokens=tokens)


def _draw_options(i: int) -> tuple[dict, np.ndarray]:
    """A random layer with random operator options: gate/up layout (a
    separate fc3 included), biases, router_weights, SwiGLU alpha/beta/limit."""
    rng = np.random.default_rng(6060 + i)
    bs = int(rng.choice([16, 32, 64, 128, 256]))
    mult = max(128, bs)
    H = int(mult * rng.integers(1, max(2, 3072 // mult) + 1))
    I = int(mult * rng.integers(1, max(2, 3072 // mult) + 1))
    E = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 33, 64, 100, 256]))
    k = int(rng.integers(1, min(E, 8) + 1))
    T = int(rng.choice([1, 2, 3, 5, 8, 13, 16, 24, 40, 64, 100, 300, 700]))
    b1, b2 = (int(b) for b in rng.choice([1, 2, 3, 4, 8], size=2))
    while E * H * I * (2 * b1 + b2) / 8 > 64e6:
        if E > 16:
            E //= 2
        elif H >= I and H > mult:
            H = max(mult, H // 2 // mult * mult)
        elif I > mult:
            I = max(mult, I // 2 // mult * mult)
        else:
            break
    k = min(k, E)
    zp_mode = str(rng.choice(["sym", "u8", "zpo"]))
    mb = min(b1, b2)
    zpo = float(rng.choice([z for z in (0.5, 1.5, 3.0) if z <= (1 << mb) - 1] or [0.5]))
    opts = {}
    fusion = int(rng.choice([0, 1, 2]))
    if fusion != 1:
        opts["swiglu_fusion"] = fusion
    if rng.random() < 0.5:
        opts["bias"] = True
    if rng.random() < 0.4:
        opts["router_weights"] = True
    if rng.random() < 0.5:
        opts.update(alpha=float(rng.choice([1.0, 1.702])), beta=float(rng.choice([0.0, 0.5])),
                    limit=float(rng.choice([0.75, 7.0, math.inf])))
    s0 = 2.0 / ((1 << (max(b1, b2) - 1)) * math.sqrt(max(H, I)))
    spec = synth.custom(T=T, H=H, I=I, E=E, k=k, fc1_bits=b1, fc2_bits=b2, block_size=bs,
                        dtype=int(rng.integers(1, 3)), act=0, normalize=int(rng.integers(0, 2)),
                        zp_mode=zp_mode, zpo=zpo if zp_mode == "zpo" else math.nan,
                        zp_range=(0, (1 << mb) - 1), scale_range=(0.5 * s0, 1.5 * s0),
                        name=f"random_options{i}", **opts)
    ntok = int(max(2, min(T, 16, 1e9 // (3 * k * H * I))))
    tokens = np.unique(np.concatenate([[0, T - 1], rng.integers(0, T, size=ntok)])).astype(np.int64)
    return spec, tokens


@pytest.mark.parametrize("i", range(N_OPTION_CASES))
def test_layer_random_shape_with_options(i):
    spec, tokens = _draw_options(i)
    print(f"  T={spec['T']} H={spec['H']} I={spec['I']} E={spec['E']} k={spec['k']} "
          f"bits={spec['fc1_bits']}/{spec['fc2_bits']} bs={spec['block_size']} zp={spec['zp_mode']} "
          f"fusion={spec.get('swiglu_fusion', 1)} bias={spec.get('bias', False)} "
          f"router_weights={spec.get('router_weights', False)}", flush=True)
    _options_check(spec, 8900 + i, tokens=tokens)


def _draw_stream(i: int) -> tuple[dict, np.ndarray | None]:
    rng = np.random.default_rng(5151 + i)
    bs = int(rng.choice([32, 64, 128, 256]))
    H = max(bs, int(rng.choice([128, 256, 512, 1024, 2048])))
    I = max(bs, int(rng.choice([128, 256, 512, 1024, 2048])))
    E = int(rng.integers(2, 33))
    T = int(rng.choice([1, 1, 2, 2, 3, 4, 5, 8, 12, 16]))
    k = int(rng.integers(1, min(E, 4) + 1))
    b1, b2 = (int(b) for b in rng.choice([2, 4], size=2))
    zp_mode = str(rng.choice(["sym", "zpo"]))
    zpo = float(rng.choice([0.5, 1.5, 3.0])) if zp_mode == "zpo" else math.nan
    if zp_mode == "zpo" and zpo > (1 << min(b1, b2)) - 1:
        zpo = 0.5
    s0 = 2.0 / ((1 << (max(b1, b2) - 1)) * math.sqrt(max(H, I)))
    spec = synth.custom(T=T, H=H, I=I, E=E, k=k, fc1_bits=b1, fc2_bits=b2, block_size=bs,
                        dtype=int(rng.integers(1, 3)), act=int(rng.integers(0, 2)),
                        normalize=int(rng.integers(0, 2)), zp_mode=zp_mode, zpo=zpo,
                        scale_range=(0.5 * s0, 1.5 * s0), name=f"random_stream{i}")
    logits = None
    if i % 4 == 3 and k < E:
        logits = rng.normal(0.0, 1.0, size=(T, E)).astype(np.float32)
        logits[:, 0] = -8.0
    return spec, logits


@pytest.mark.parametrize("i", range(N_STREAM_CASES))
def test_layer_random_small_decode(i):
    spec, logits = _draw_stream(i)
    print(f"  T={spec['T']} H={spec['H']} I={spec['I']} E={spec['E']} k={spec['k']} "
          f"bits={spec['fc1_bits']}/{spec['fc2_bits']} bs={spec['block_size']} zp={spec['zp_mode']} "
          f"expert0_out={logits is not None}", flush=True)
    _layer_check(spec, 8700 + i, logits=logits)
