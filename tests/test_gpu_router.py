"""GPU parity of the router logit GEMV (coli_moe_route_hidden): logits
against the fp64 oracle within an fp32 summation bound, the routing it feeds
bit-exact against the oracle's top-k of those same logits, and a token's
logits identical whatever batch it is computed in."""
import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth
from gpu_util import route_host

pytestmark = pytest.mark.gpu


def _layer(spec):
    # route_hidden reads only the shape and the routing flags of the layer;
    # a small intermediate size keeps the (unused) expert container small
    small = synth.LayerSpec(spec.hidden, 64, spec.n_experts, spec.n_shared, spec.top_k,
                            spec.sigmoid, spec.renorm, spec.routed_scale)
    q4, sc = synth.make_weights(small, seed=0, device="cuda", experts=1)
    return coli.Layer(spec.hidden, 64, spec.n_experts, spec.n_shared, spec.top_k, spec.flags,
                      q4, sc, spec.routed_scale)


def _route_hidden(spec, w, x, sel_bias=None):
    T = x.shape[0]
    L = _layer(spec)
    r = coli.Route(L, T)
    logits = torch.empty(T, spec.n_experts, dtype=torch.float32, device="cuda")
    coli.coli_moe_route_hidden(L, w.cuda(), x.cuda(), None if sel_bias is None else sel_bias.cuda(),
                               T, logits, r)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), route_host(r, T, spec.top_k)


def _bound(w, x):
    """|fp32 sum - exact| for the kernel's summation: per lane at most H/64
    dot2 steps (bf16 products are exact in fp32; each step rounds at most
    twice), then 6 butterfly additions -- at most 2*H/64 + 6 <= 256 roundings
    for H <= 8192, each off by at most 2^-24 of a partial sum bounded by
    sum |x_k w_k|."""
    xa = np.abs(x.float().numpy().astype(np.float64))
    wa = np.abs(w.float().numpy().astype(np.float64))
    return 2.0 ** -16 * (xa @ wa.T) + 1e-30


def _check(spec, w, x, sel_bias=None):
    T = x.shape[0]
    print("router case: H=%d E=%d k=%d T=%d" % (spec.hidden, spec.n_experts, spec.top_k, T),
          flush=True)
    lg, g = _route_hidden(spec, w, x, sel_bias)
    ref = oracle.router_logits(synth.bf16_bits(w), synth.bf16_bits(x))
    err = np.abs(lg.astype(np.float64) - ref.astype(np.float64))
    assert np.all(err <= _bound(w, x)), float(np.max(err / _bound(w, x)))
    # the routing of exactly these logits is bit-exact
    o = oracle.route(lg, spec.top_k, spec.flags, spec.routed_scale,
                     sel_bias=None if sel_bias is None else sel_bias.numpy())
    assert np.array_equal(g["topk_idx"].reshape(T, -1), o["topk_idx"])
    assert np.array_equal(g["counts"], o["counts"])
    assert np.array_equal(g["offsets"], o["offsets"])
    assert np.array_equal(g["pairs"], o["pairs"])
    np.testing.assert_allclose(g["topk_w"].reshape(T, -1), o["topk_w"], rtol=3e-6, atol=1e-7)
    return lg


@pytest.mark.parametrize("name,T", [
    ("tiny", 4), ("olmoe", 1), ("a3b", 1), ("a3b", 4), ("a3b", 16), ("glm", 1), ("glm", 4),
    ("glm_prefill", 2048),
])
def test_router_workloads(name, T):
    spec = synth.WORKLOADS[name].spec
    w = synth.make_router_weights(spec, seed=1)
    x = synth.make_x(spec, T, seed=1)
    _check(spec, w, x)


@pytest.mark.parametrize("H,E,k,T", [
    (192, 5, 2, 3),      # H not a multiple of 512; E not a multiple of 4
    (576, 37, 3, 17),    # first batch size of the 4-expert x 16-token grouping
    (1024, 1, 1, 33),
    (64, 300, 8, 20),
])
def test_router_edge_shapes(H, E, k, T):
    spec = synth.LayerSpec(H, 64, E, 0, k, sigmoid=True, renorm=True)
    _check(spec, synth.make_router_weights(spec, seed=H), synth.make_x(spec, T, seed=E))


def test_router_selection_bias():
    spec = synth.WORKLOADS["a3b"].spec
    _check(spec, synth.make_router_weights(spec, seed=2), synth.make_x(spec, 9, seed=2),
           sel_bias=synth.make_sel_bias(spec, seed=2))


def test_router_logits_batch_invariant_and_deterministic():
    """A token's logits do not depend on the batch around it (T = 1, 7 and
    40 use different work groupings) and repeat bit for bit."""
    spec = synth.WORKLOADS["glm"].spec
    w = synth.make_router_weights(spec, seed=3)
    x = synth.make_x(spec, 40, seed=3)
    big, _ = _route_hidden(spec, w, x)
    again, _ = _route_hidden(spec, w, x)
    assert np.array_equal(big, again)
    mid, _ = _route_hidden(spec, w, x[11:18].contiguous())
    assert np.array_equal(mid, big[11:18])
    for t in (0, 13, 39):
        one, _ = _route_hidden(spec, w, x[t:t + 1].contiguous())
        assert np.array_equal(one[0], big[t]), t
