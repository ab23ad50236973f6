"""GPU parity of int8-weight experts in the decode / verify forward against
the fp64 oracle: the container with one int8 code per weight (the MTP layer
and OLMoE-style containers), on every streaming shape, on shapes and batch
sizes (17..64 tokens) served by the general decode kernels, plus batch
invariance."""
import dataclasses

import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import synth
from gpu_util import REL_TOL, forward, gpu_layer, oracle_layer, rel_err, checked_route, run_route

pytestmark = pytest.mark.gpu


def _i8(spec):
    return dataclasses.replace(spec, int8=True)


def _case(spec, T, seed=0, zipf=0.0, tokens=None):
    print("int8 decode case: H=%d I=%d E=%d S=%d k=%d T=%d" % (
        spec.hidden, spec.inter, spec.n_experts, spec.n_shared, spec.top_k, T), flush=True)
    L = gpu_layer(spec, seed=seed)
    assert L.q4.numel() == spec.n_total * 3 * spec.hidden * spec.inter
    lg = synth.make_logits(spec, T, seed=seed, zipf_alpha=zipf).cuda()
    x = synth.make_x(spec, T, seed=seed).cuda()
    r = run_route(L, lg)
    y = forward(L, r, x, "decode")
    g = checked_route(spec, r, lg)
    toks = list(range(T)) if tokens is None else tokens
    ref = oracle_layer(spec, L, g["topk_idx"], g["topk_w"], x, toks, "decode")
    err = rel_err(y.cpu().numpy()[toks], ref)
    print("  rel err %.3g" % err, flush=True)
    assert err < REL_TOL
    return L, lg, x, y


@pytest.mark.parametrize("name,T", [
    ("olmoe", 1), ("olmoe", 4), ("olmoe", 16), ("a3b", 1), ("a3b", 4), ("glm", 1), ("glm", 4),
])
def test_int8_decode_workloads(name, T):
    w = synth.WORKLOADS[name]
    _case(_i8(w.spec), T, zipf=w.zipf_alpha, tokens=[0, T - 1] if name == "glm" else None)


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(4096, 4096, 4, 1, 2, sigmoid=True, renorm=True, int8=True), 3),   # CPL 2
    (synth.LayerSpec(2048, 8192, 3, 1, 1, sigmoid=False, renorm=False, int8=True), 2),  # CPL 4
    (synth.LayerSpec(8192, 512, 5, 0, 2, sigmoid=True, renorm=False, int8=True), 5),    # H 8192
])
def test_int8_decode_edge_shapes(spec, T):
    _case(spec, T, seed=4, zipf=0.5)


def test_int8_decode_batch_invariant_and_deterministic():
    spec = _i8(synth.WORKLOADS["olmoe"].spec)
    L, lg, x, y = _case(spec, 4, seed=2)
    r = run_route(L, lg)
    assert torch.equal(forward(L, r, x, "decode"), y)
    for t in range(4):
        rt = run_route(L, lg[t:t + 1].contiguous())
        assert torch.equal(forward(L, rt, x[t:t + 1].contiguous(), "decode")[0], y[t])


def test_int8_extreme_codes():
    """Every code -128 (and then +127) with unit-ish scales: the bias removal
    and the high-nibble sign hold at the ends of the range."""
    spec = synth.LayerSpec(2048, 1024, 4, 1, 2, sigmoid=True, renorm=True, int8=True)
    for byte in (0x80, 0x7F, 0x01):
        q4 = torch.full((spec.n_total * spec.expert_bytes,), byte, dtype=torch.uint8, device="cuda")
        sc = torch.full((spec.n_total * spec.expert_scales,), 2.0 ** -10, dtype=torch.float16,
                        device="cuda")
        L = coli.Layer.from_spec(spec, q4, sc)
        lg = synth.make_logits(spec, 2, seed=1).cuda()
        x = synth.make_x(spec, 2, seed=1).cuda()
        r = run_route(L, lg)
        y = forward(L, r, x, "decode")
        g = checked_route(spec, r, lg)
        ref = oracle_layer(spec, L, g["topk_idx"], g["topk_w"], x, [0, 1], "decode")
        assert rel_err(y.cpu().numpy(), ref) < REL_TOL, hex(byte)


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(2048, 1024, 64, 1, 8, sigmoid=False, renorm=True, int8=True), 17),
    (synth.LayerSpec(2048, 1024, 64, 1, 8, sigmoid=False, renorm=True, int8=True), 64),
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, int8=True), 1),  # no stream shape
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, int8=True), 9),
    (synth.LayerSpec(2112, 1088, 5, 0, 2, sigmoid=False, renorm=False, int8=True), 33),
])
def test_int8_decode_general_path(spec, T):
    """Shapes without the streaming kernels and batches of 17..64 tokens run
    the general (slot, row block) kernels with the int8 codec."""
    _case(spec, T, seed=6, zipf=0.5)


def test_int8_decode_large_batch_invariant():
    """Among batches of 17..64 tokens a token's result does not depend on the
    rest of the batch: the first 17 tokens of a 40-token batch, alone."""
    spec = synth.LayerSpec(2048, 1024, 64, 1, 8, sigmoid=False, renorm=True, int8=True)
    L = gpu_layer(spec, seed=8)
    lg = synth.make_logits(spec, 40, seed=8, zipf_alpha=0.5).cuda()
    x = synth.make_x(spec, 40, seed=8).cuda()
    y40 = forward(L, run_route(L, lg), x, "decode")
    y17 = forward(L, run_route(L, lg[:17].contiguous()), x[:17].contiguous(), "decode")
    assert torch.equal(y17, y40[:17])
