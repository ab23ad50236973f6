"""GPU parity of int8-weight experts on the integer prefill path: exact int32
block dots of int8 codes x int8 activations on the matrix cores, bit for bit
against the oracle, and the layer output (Q8_0 activations, gate/up, SwiGLU,
Q8_0 h, down, combine) against the fp64 oracle within 2e-3, plus, where an h
code sits on a Q8_0 rounding boundary, the most that decision can move the
output (gpu_util.prefill_flip_budget)."""
import dataclasses

import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth
from gpu_util import check_prefill_output, forward, gpu_layer, checked_route, cover_tokens, run_route

pytestmark = pytest.mark.gpu


def _i8(spec):
    return dataclasses.replace(spec, int8=True)


@pytest.mark.parametrize("spec,T,experts", [
    (synth.LayerSpec(256, 256, 4, 0, 2, False, False, int8=True), 5, (0, 3)),
    (synth.LayerSpec(2048, 1024, 4, 1, 2, True, True, int8=True), 100, (1, 4)),
    (synth.LayerSpec(6144, 2048, 2, 1, 2, True, True, int8=True), 64, (2,)),
    # reduction lengths that are not multiples of 256 (the per-step kernel)
    (synth.LayerSpec(192, 320, 3, 1, 2, True, True, int8=True), 37, (0, 3)),
])
def test_int8_block_dots_bit_exact(spec, T, experts):
    print("int8 block dots case: H=%d I=%d T=%d" % (spec.hidden, spec.inter, T), flush=True)
    q8, sc = synth.make_weights(spec, seed=6, device="cuda")
    L = coli.Layer.from_spec(spec, q8, sc)
    g = torch.Generator().manual_seed(T + 1)
    for e in experts:
        for m in (0, 1, 2):
            K = spec.inter if m == 2 else spec.hidden
            rows = spec.hidden if m == 2 else spec.inter
            a = torch.randint(-127, 128, (T, K), generator=g, dtype=torch.int8)
            a[0] = 127
            a[1] = -127
            dots = torch.empty(T, rows, K // 32, dtype=torch.int32, device="cuda")
            coli.coli_moe_block_dots(L, e, m, a.cuda(), T, dots)
            torch.cuda.synchronize()
            qh, sh = synth.expert_slice(spec, q8, sc, [e])
            want = oracle.block_dots(spec.hidden, spec.inter, 1, 0, qh, sh, 0, m, a.numpy(),
                                     weights="int8")
            assert np.array_equal(dots.cpu().numpy(), want), (e, m)


def test_int8_block_dots_extremes():
    """Codes -128 and 127 against activations -127 and 127: the largest block
    magnitudes (32 * 128 * 127) come out exact."""
    spec = synth.LayerSpec(256, 256, 1, 0, 1, False, False, int8=True)
    for byte in (0x80, 0x7F):
        q8 = torch.full((spec.n_total * spec.expert_bytes,), byte, dtype=torch.uint8, device="cuda")
        sc = torch.ones(spec.n_total * spec.expert_scales, dtype=torch.float16, device="cuda")
        L = coli.Layer.from_spec(spec, q8, sc)
        a = torch.full((2, 256), 127, dtype=torch.int8)
        a[1] = -127
        dots = torch.empty(2, 256, 8, dtype=torch.int32, device="cuda")
        coli.coli_moe_block_dots(L, 0, 0, a.cuda(), 2, dots)
        torch.cuda.synchronize()
        q = -128 if byte == 0x80 else 127
        d = dots.cpu().numpy()
        assert np.all(d[0] == 32 * q * 127) and np.all(d[1] == -32 * q * 127)


def _case(spec, T, seed=0, zipf=0.0, tokens=None, cover=None):
    print("int8 prefill case: H=%d I=%d E=%d S=%d k=%d T=%d" % (
        spec.hidden, spec.inter, spec.n_experts, spec.n_shared, spec.top_k, T), flush=True)
    L = gpu_layer(spec, seed=seed)
    lg = synth.make_logits(spec, T, seed=seed, zipf_alpha=zipf).cuda()
    x = synth.make_x(spec, T, seed=seed).cuda()
    r = run_route(L, lg)
    y = forward(L, r, x, "prefill")
    g = checked_route(spec, r, lg)
    toks = list(range(T)) if tokens is None else list(tokens)
    if cover is not None:
        toks = sorted(set(toks) | set(cover_tokens(g, T, spec.top_k, **cover)))
    print("  comparing %d tokens" % len(toks), flush=True)
    # int8 weights make a Q8_0 boundary decision of h weigh more than int4
    # codes do, so the comparison allows for those decisions explicitly
    err, n_budget = check_prefill_output(spec, L, g, x, y, toks)
    print("  rel err %.3g, %d elements within the boundary budget" % (err, n_budget), flush=True)
    return L, r, x, y


def test_int8_prefill_olmoe_512_sampled():
    _case(_i8(synth.WORKLOADS["olmoe"].spec), 512, tokens=[0, 1, 63, 64, 200, 511])


@pytest.mark.timeout(600)
def test_int8_prefill_glm_every_tile():
    """GLM-shaped int8 layer at 700 tokens: every (expert, 64-token tile)
    item's first and last row, the shared expert's tile boundaries and all
    tokens of the hottest expert (about 300 tokens)."""
    w = synth.WORKLOADS["glm_prefill"]
    _case(_i8(w.spec), 700, zipf=w.zipf_alpha, tokens=[350], cover=dict(tile=64, hottest=1))


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(256, 256, 6, 1, 2, sigmoid=True, renorm=True, int8=True), 70),
    (synth.LayerSpec(1024, 768, 32, 0, 4, sigmoid=False, renorm=True, int8=True), 129),
    (synth.LayerSpec(512, 256, 1, 0, 1, sigmoid=False, renorm=False, int8=True), 1),
    # H, I not multiples of 256: the per-step kernel
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, int8=True), 70),
    (synth.LayerSpec(2112, 1088, 8, 1, 3, sigmoid=False, renorm=True, int8=True), 150),
])
def test_int8_prefill_edge_shapes(spec, T):
    _case(spec, T, seed=3, zipf=0.6)


def test_int8_prefill_deterministic():
    spec = _i8(synth.WORKLOADS["a3b"].spec)
    L, r, x, y = _case(spec, 96, zipf=synth.ZIPF_ALPHA, tokens=[0, 95])
    assert torch.equal(forward(L, r, x, "prefill"), y)
