"""qmoe_forward_noalloc: the layer with the library's fixed scratch array as
workspace.  Through the C ABI it must give exactly what qmoe_forward gives
with a caller workspace (the same kernels), call after call, also when a
smaller layer follows a larger one on the same array; and sizes beyond the
array are rejected before anything is launched."""
from __future__ import annotations

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
import qmoe_synth as synth
import quantized_mixture_experts_route_amd as qm
from tests import _device as dv


def test_noalloc_rejects_sizes_beyond_the_scratch():
    # the skewed 4096-token layer needs ~736 MiB of workspace: refused on the
    # host, before any device call (runs without a GPU)
    lib = qm.load_library()
    p = qm._Proj(1 << 20, 1 << 20, None, 4)
    rc = lib.qmoe_forward_noalloc(1 << 20, 1 << 20, 4096, 4096, 14336, 8, ctypes.byref(p),
                                  ctypes.byref(p), math.nan, 128, 2, 1, 0, 2, 1 << 20, None,
                                  None, None)
    assert rc == qm.ERR_WORKSPACE
    assert "qmoe_forward_noalloc" in qm.last_error()
    assert qm.workspace_size(4096, 4096, 14336, 8, 2, 2) > qm.NOALLOC_SCRATCH_BYTES
    # T = 0 is a no-op that needs no scratch
    assert lib.qmoe_forward_noalloc(1 << 20, 1 << 20, 0, 256, 256, 8, ctypes.byref(p),
                                    ctypes.byref(p), math.nan, 32, 2, 1, 0, 1, 1 << 20, None,
                                    None, None) == qm.OK


def _run_both(spec, seed):
    inp = synth.make_inputs(spec, seed)
    dev = dv.to_device(inp, spec)
    ref_out, ref_ids, ref_w = dv.run_layer(dev, spec, return_routing=True)
    out = torch.full_like(ref_out, float("nan"))
    got, ids, w = qm.forward_noalloc(dev["hidden"], dev["logits"], dev["fc1"], dev["fc2"],
                                     top_k=spec["k"], block_size=spec["block_size"],
                                     normalize=spec["normalize"], activation=spec["act"],
                                     zero_point_offset=spec["zpo"], out=out,
                                     return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref_out.view(torch.int16))
    assert torch.equal(ids, ref_ids)
    assert torch.equal(w, ref_w)
    oracle_ref = oracle.forward(inp, spec)
    err = float(np.abs(dv.as_f64(got) - oracle_ref).max())
    assert err <= dv.tolerance(oracle_ref)
    ids_ref, _ = oracle.route(inp["logits"], spec["k"], spec["normalize"])
    assert np.array_equal(ids.cpu().numpy(), ids_ref)


@pytest.mark.gpu
def test_noalloc_matches_forward_two_calls_larger_then_smaller():
    # a prefill layer (R = 600 routes, fc2 K parts in the scratch), then a
    # decode layer on the same scratch array
    big = synth.custom(T=300, H=512, I=768, E=8, k=2, fc1_bits=4, fc2_bits=3, block_size=64,
                       dtype=2, act=0, zp_mode="sym", name="noalloc_big")
    small = synth.custom(T=5, H=256, I=512, E=6, k=2, fc1_bits=2, fc2_bits=4, block_size=128,
                         dtype=1, act=1, zp_mode="zpo", zpo=1.5, name="noalloc_small")
    _run_both(big, 41)
    _run_both(small, 42)


@pytest.mark.gpu
def test_noalloc_named_workloads():
    # the tiny, decode, 512-token prefill and many-expert layers all fit the scratch
    for cfg in (3, 2, 4, 1):
        spec = synth.workload(cfg)
        assert qm.workspace_size(spec["T"], spec["H"], spec["I"], spec["E"], spec["k"],
                                 spec["dtype"]) <= qm.NOALLOC_SCRATCH_BYTES
        _run_both(spec, synth.seed_for(cfg))
