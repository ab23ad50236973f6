"""GPU parity of the decode / verify forward against the fp64 oracle."""
import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import synth
from gpu_util import (BF16_HALF_ULP, REL_TOL, bf16_ulp_distance, forward, gpu_layer, oracle_layer, rel_err,
                      checked_route, run_route)

pytestmark = pytest.mark.gpu


def _decode_case(spec, T, seed=0, zipf=0.0, layer=0, tokens=None):
    print("decode case: H=%d I=%d E=%d S=%d k=%d T=%d seed=%d" % (
        spec.hidden, spec.inter, spec.n_experts, spec.n_shared, spec.top_k, T, seed), flush=True)
    L = gpu_layer(spec, seed=seed, layer=layer)
    lg = synth.make_logits(spec, T, seed=seed, layer=layer, zipf_alpha=zipf).cuda()
    x = synth.make_x(spec, T, seed=seed, layer=layer).cuda()
    r = run_route(L, lg)
    y = forward(L, r, x, "decode")
    g = checked_route(spec, r, lg)
    toks = range(T) if tokens is None else tokens
    ref = oracle_layer(spec, L, g["topk_idx"], g["topk_w"], x, toks, "decode")
    err = rel_err(y.cpu().numpy()[list(toks)], ref)
    print("  rel err %.3g" % err, flush=True)
    assert err < REL_TOL
    return L, r, x, y, ref


@pytest.mark.parametrize("name,T", [
    ("tiny", 4), ("olmoe", 1), ("a3b", 1), ("a3b", 4), ("a3b", 16), ("glm", 1), ("glm", 4),
])
def test_decode_workloads(name, T):
    w = synth.WORKLOADS[name]
    _decode_case(w.spec, T, zipf=w.zipf_alpha)


@pytest.mark.parametrize("spec,T", [
    # ragged rows: H/32 and I/32 not powers of two (idle lanes per row)
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True), 5),
    # H/32 = 264 chunks: the runtime chunk loop; I/32 = 4 chunks
    (synth.LayerSpec(8448, 128, 4, 0, 2, sigmoid=False, renorm=True), 3),
    # H/32 = 128 and 256 (two and four chunks per lane)
    (synth.LayerSpec(4096, 8192, 3, 1, 1, sigmoid=True, renorm=False), 2),
    # smallest shape, one expert, k = 1
    (synth.LayerSpec(64, 64, 1, 0, 1, sigmoid=False, renorm=False), 1),
    # the maximum decode batch, every expert hot
    (synth.LayerSpec(512, 256, 16, 1, 4, sigmoid=True, renorm=True), 64),
    # the largest hidden size, and the largest decode intermediate size
    (synth.LayerSpec(16384, 128, 4, 1, 2, sigmoid=True, renorm=True), 3),
    (synth.LayerSpec(128, 15360, 3, 1, 1, sigmoid=False, renorm=False), 2),
    # the most experts and the largest top-k: 1024 experts, k = 32, on the
    # general kernels (T = 64: a union of up to 1024 slots) and on the
    # streaming kernels (T = 1, and T = 16 with a union of up to 512 slots)
    (synth.LayerSpec(256, 128, 1024, 1, 32, sigmoid=True, renorm=True), 64),
    (synth.LayerSpec(2048, 512, 1024, 1, 32, sigmoid=False, renorm=True), 1),
    (synth.LayerSpec(2048, 512, 1024, 1, 32, sigmoid=True, renorm=False), 16),
])
def test_decode_edge_shapes(spec, T):
    _decode_case(spec, T, seed=7, zipf=0.5)


def test_decode_bf16_output():
    spec = synth.WORKLOADS["a3b"].spec
    L, r, x, y32, ref = _decode_case(spec, 16, zipf=synth.ZIPF_ALPHA)
    yb = forward(L, r, x, "decode", y_dtype=coli.COLI_OUT_BF16)
    # the bf16 output is exactly the nearest-even rounding of the fp32 output
    assert torch.equal(yb, y32.to(torch.bfloat16))
    # so against the oracle it is within the tolerance plus bf16's half ulp
    assert rel_err(yb.float().cpu().numpy(), ref) < REL_TOL + BF16_HALF_ULP
    # and where the oracle is not tiny, within one bf16 ulp of bf16(oracle)
    big = np.abs(ref) > 0.25 * np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    assert bf16_ulp_distance(yb, np.where(big, ref, yb.float().cpu().numpy())) <= 1


def test_decode_deterministic_and_batch_invariant():
    spec = synth.WORKLOADS["glm"].spec
    L = gpu_layer(spec)
    T = 4
    lg = synth.make_logits(spec, T, zipf_alpha=synth.ZIPF_ALPHA).cuda()
    x = synth.make_x(spec, T).cuda()
    r = run_route(L, lg)
    y1 = forward(L, r, x, "decode")
    y2 = forward(L, r, x, "decode")
    assert torch.equal(y1, y2)
    for t in range(T):
        rt = run_route(L, lg[t:t + 1].contiguous())
        yt = forward(L, rt, x[t:t + 1].contiguous(), "decode")
        assert torch.equal(yt[0], y1[t]), "token %d depends on its batch" % t


def test_decode_zero_scales_give_zero():
    spec = synth.WORKLOADS["a3b"].spec
    q4, sc = synth.make_weights(spec, device="cuda")
    L = coli.Layer.from_spec(spec, q4, torch.zeros_like(sc))
    lg = synth.make_logits(spec, 4).cuda()
    x = synth.make_x(spec, 4).cuda()
    y = forward(L, run_route(L, lg), x, "decode")
    assert not y.any()


def test_decode_stack_layers_independent():
    """Two layers of the GLM-shaped stack, each against the oracle."""
    spec = synth.WORKLOADS["glm"].spec
    for layer in (1, 11):
        _decode_case(spec, 1, layer=layer, zipf=synth.ZIPF_ALPHA)
