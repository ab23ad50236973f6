"""GPU parity of routing: top-k indices, pair lists, union bit-exact vs the
oracle; routing weights to fp32 accuracy."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import gpu_layer, route_host, run_route

pytestmark = pytest.mark.gpu


def _check_route(spec, logits, sel_bias=None):
    print("route case: E=%d k=%d T=%d flags=%d bias=%s" % (
        spec.n_experts, spec.top_k, logits.shape[0], spec.flags, sel_bias is not None), flush=True)
    L = gpu_layer(synth.LayerSpec(64, 64, spec.n_experts, spec.n_shared, spec.top_k,
                                  spec.sigmoid, spec.renorm, spec.routed_scale))
    T = logits.shape[0]
    r = run_route(L, logits.cuda(), None if sel_bias is None else sel_bias.cuda())
    g = route_host(r, T, spec.top_k)
    o = oracle.route(logits.numpy(), spec.top_k, spec.flags, spec.routed_scale,
                     sel_bias=None if sel_bias is None else sel_bias.numpy())
    assert np.array_equal(g["topk_idx"].reshape(T, -1), o["topk_idx"])
    assert np.array_equal(g["counts"], o["counts"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["pairs"], o["pairs"])
    P = T * spec.top_k
    assert np.array_equal(g["pairs"][g["pair_pos"]], np.arange(P))
    nu = int(g["n_union"][0])
    assert np.array_equal(g["union_ids"][:nu], np.nonzero(o["counts"])[0])
    np.testing.assert_allclose(g["topk_w"].reshape(T, -1), o["topk_w"], rtol=3e-6, atol=1e-7)


@pytest.mark.parametrize("name,T", [
    ("tiny", 4), ("olmoe", 1), ("olmoe", 512), ("a3b", 1), ("a3b", 4), ("a3b", 16),
    ("glm", 1), ("glm", 4), ("glm_prefill", 2048),
])
def test_route_workloads(name, T):
    w = synth.WORKLOADS[name]
    lg = synth.make_logits(w.spec, T, seed=0, zipf_alpha=w.zipf_alpha)
    _check_route(w.spec, lg)


@pytest.mark.parametrize("E,k,T,flags", [
    (8, 8, 3, 0), (5, 1, 17, 1), (300, 17, 33, 257), (1024, 32, 40, 1), (1024, 8, 4096, 256),
    (64, 8, 16, 257), (64, 8, 17, 257), (1, 1, 5, 0), (256, 8, 65536 // 8, 257),
    (64, 16, 65536, 257),  # the maximum batch: 65,536 tokens, 2^20 pairs
    # one token (the single-wavefront kernel): E not a multiple of 64, the
    # largest E and k, one expert, k = E
    (300, 17, 1, 257), (1024, 32, 1, 1), (1024, 8, 1, 256), (5, 1, 1, 1), (1, 1, 1, 0),
    (8, 8, 1, 0), (130, 3, 1, 257),
])
def test_route_edges(E, k, T, flags):
    spec = synth.LayerSpec(64, 64, E, 0, k, sigmoid=bool(flags & 1), renorm=bool(flags & 256),
                           routed_scale=2.5)
    g = torch.Generator().manual_seed(E * 1000 + T)
    lg = torch.randn(T, E, generator=g)
    lg[:, ::2] = torch.round(lg[:, ::2] * 2) / 2  # exact ties
    _check_route(spec, lg)


def test_route_selection_bias_and_all_equal():
    spec = synth.WORKLOADS["a3b"].spec
    lg = synth.make_logits(spec, 16, seed=3)
    _check_route(spec, lg, sel_bias=synth.make_sel_bias(spec, seed=3))
    _check_route(spec, torch.zeros(16, spec.n_experts))


def test_route_is_deterministic():
    spec = synth.WORKLOADS["glm_prefill"].spec
    lg = synth.make_logits(spec, 2048, seed=1, zipf_alpha=0.6).cuda()
    L = gpu_layer(synth.LayerSpec(64, 64, spec.n_experts, 1, 8, True, True))
    a = route_host(run_route(L, lg), 2048, 8)
    b = route_host(run_route(L, lg), 2048, 8)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
