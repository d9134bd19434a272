"""GPU parity of the layer with a shared expert (qmoe_forward_shared): the
routed output plus sigmoid(x . gate) times the shared expert's FFN, against
the oracle's routed layer plus its shared-expert term, within the layer
tolerance 1e-2 * max|ref| + 1e-3."""
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


def _shared_dev(sh, spec):
    def proj(name, bits):
        zp = sh[name + "_zp"]
        return qm.Projection(torch.from_numpy(sh[name + "_codes"]).cuda(),
                             dv.bits_tensor(sh[name + "_scales"], spec["dtype"]),
                             None if zp is None else torch.from_numpy(zp).cuda(), bits)
    return (proj("fc1", spec["fc1_bits"]), proj("fc2", spec["fc2_bits"]),
            dv.bits_tensor(sh["gate"], spec["dtype"]))


def _check(spec, I_shared, seed, tokens=None):
    inp = synth.make_inputs(spec, seed)
    sh = synth.make_shared_expert(spec, I_shared, seed + 1)
    dev = dv.to_device(inp, spec)
    s1, s2, gate = _shared_dev(sh, spec)
    out, ids, _ = qm.forward_shared(dev["hidden"], dev["logits"], dev["fc1"], dev["fc2"], s1, s2,
                                    gate, top_k=spec["k"], block_size=spec["block_size"],
                                    normalize=spec["normalize"], activation=spec["act"],
                                    zero_point_offset=spec["zpo"], return_routing=True)
    torch.cuda.synchronize()
    ids_ref, _ = oracle.route(inp["logits"], spec["k"], spec["normalize"])
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    ref = oracle.forward(inp, spec, tokens) + oracle.shared_expert(inp, sh, spec, tokens)
    got = dv.as_f64(out)
    if tokens is not None:
        got = got[tokens]
    err = float(np.abs(got - ref).max())
    tol = dv.tolerance(ref)
    print(f"  {spec['name']}: max|err|={err:.3e} tol={tol:.3e}", flush=True)
    assert err <= tol


@pytest.mark.parametrize("cfg,I_shared", [(1, 256), (2, 1024), (4, 768)])
def test_shared_expert_named_decode_layers(cfg, I_shared):
    _check(synth.workload(cfg), I_shared, synth.seed_for(cfg))


def test_shared_expert_512_token_prefill():
    # u8 zero points in the shared projections too; the shared layer's 512
    # routes on one expert run the prefill tiles
    _check(synth.workload(3), 2048, synth.seed_for(3))


@pytest.mark.parametrize("T,dtype,act,zp", [(3, 2, 0, "sym"), (70, 1, 1, "zpo"), (130, 2, 0, "u8")])
def test_shared_expert_small(T, dtype, act, zp):
    spec = synth.custom(T=T, H=256, I=384, E=6, k=2, fc1_bits=4, fc2_bits=2, block_size=64,
                        dtype=dtype, act=act, zp_mode=zp, zpo=1.5 if zp == "zpo" else math.nan,
                        zp_range=(0, 3), name=f"shared_small_{T}")
    _check(spec, 128, 50 + T)


def test_shared_expert_zero_tokens():
    spec = synth.custom(T=1, H=128, I=128, E=4, k=2)
    inp = synth.make_inputs(spec, 1)
    sh = synth.make_shared_expert(spec, 128, 2)
    dev = dv.to_device(inp, spec)
    s1, s2, gate = _shared_dev(sh, spec)
    out = qm.forward_shared(dev["hidden"][:0], dev["logits"][:0], dev["fc1"], dev["fc2"], s1, s2,
                            gate, top_k=2, block_size=32)
    assert out.shape == (0, 128)
