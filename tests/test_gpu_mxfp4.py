"""GPU parity of MXFP4 experts (E2M1 codes, one E8M0 scale per 32 weights):
the decode / verify forward against the fp64 oracle (exact E2M1 -> bf16
conversion on the hardware), the integer prefill path's block dots bit for
bit (codes enter the int8 matrix cores doubled), and its layer output with
the Q8_0 boundary budget of gpu_util.check_prefill_output."""
import dataclasses

import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth
from gpu_util import (REL_TOL, check_prefill_output, forward, gpu_layer, oracle_layer, rel_err,
                      checked_route, cover_tokens, run_route)

pytestmark = pytest.mark.gpu


def _f4(spec):
    return dataclasses.replace(spec, mxfp4=True)


def _decode(spec, T, seed=0, zipf=0.0, tokens=None):
    print("mxfp4 decode case: H=%d I=%d E=%d T=%d" % (spec.hidden, spec.inter, spec.n_experts, T),
          flush=True)
    L = gpu_layer(spec, seed=seed)
    assert L.scales.dtype == torch.uint8
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


@pytest.mark.parametrize("name,T", [("olmoe", 1), ("olmoe", 4), ("a3b", 16), ("glm", 1),
                                    ("glm", 4)])
def test_mxfp4_decode_workloads(name, T):
    w = synth.WORKLOADS[name]
    _decode(_f4(w.spec), T, zipf=w.zipf_alpha, tokens=[0, T - 1] if name == "glm" else None)


def test_mxfp4_decode_every_code_and_scale_extremes():
    """All 16 E2M1 codes in every row, E8M0 from 100 to 140 and the
    subnormal-producing 0 and 1 in the shared expert."""
    spec = synth.LayerSpec(2048, 512, 4, 1, 2, sigmoid=True, renorm=True, mxfp4=True)
    q = torch.arange(256, dtype=torch.uint8).repeat(spec.n_total * spec.expert_bytes // 256)
    g = torch.Generator().manual_seed(9)
    sc = torch.randint(100, 141, (spec.n_total * spec.expert_scales,), generator=g,
                       dtype=torch.uint8)
    sc[-64:] = torch.tensor([0, 1] * 32, dtype=torch.uint8)
    L = coli.Layer.from_spec(spec, q.cuda(), sc.cuda())
    lg = synth.make_logits(spec, 3, seed=2).cuda()
    x = synth.make_x(spec, 3, seed=2).cuda()
    r = run_route(L, lg)
    y = forward(L, r, x, "decode")
    gh = checked_route(spec, r, lg)
    ref = oracle_layer(spec, L, gh["topk_idx"], gh["topk_w"], x, [0, 1, 2], "decode")
    assert rel_err(y.cpu().numpy(), ref) < REL_TOL


def test_mxfp4_decode_batch_invariant():
    spec = _f4(synth.WORKLOADS["olmoe"].spec)
    L, lg, x, y = _decode(spec, 4, seed=5)
    for t in range(4):
        rt = run_route(L, lg[t:t + 1].contiguous())
        assert torch.equal(forward(L, rt, x[t:t + 1].contiguous(), "decode")[0], y[t])


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(2048, 1024, 64, 1, 8, sigmoid=False, renorm=True, mxfp4=True), 17),
    (synth.LayerSpec(2048, 1024, 64, 1, 8, sigmoid=False, renorm=True, mxfp4=True), 64),
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, mxfp4=True), 1),  # no stream shape
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, mxfp4=True), 9),
    (synth.LayerSpec(2112, 1088, 5, 0, 2, sigmoid=False, renorm=False, mxfp4=True), 33),
])
def test_mxfp4_decode_general_path(spec, T):
    """Shapes without the streaming kernels and batches of 17..64 tokens run
    the general (slot, row block) kernels with the MXFP4 codec."""
    _decode(spec, T, seed=6, zipf=0.5)


def test_mxfp4_decode_large_batch_invariant():
    """The first 17 tokens of a 40-token batch, alone, give the same bits."""
    spec = synth.LayerSpec(2048, 1024, 64, 1, 8, sigmoid=False, renorm=True, mxfp4=True)
    L = gpu_layer(spec, seed=8)
    lg = synth.make_logits(spec, 40, seed=8, zipf_alpha=0.5).cuda()
    x = synth.make_x(spec, 40, seed=8).cuda()
    y40 = forward(L, run_route(L, lg), x, "decode")
    y17 = forward(L, run_route(L, lg[:17].contiguous()), x[:17].contiguous(), "decode")
    assert torch.equal(y17, y40[:17])


@pytest.mark.parametrize("spec,T,experts", [
    (synth.LayerSpec(256, 256, 4, 0, 2, False, False, mxfp4=True), 5, (0, 3)),
    (synth.LayerSpec(2048, 1024, 4, 1, 2, True, True, mxfp4=True), 100, (1, 4)),
    # reduction lengths that are not multiples of 256 (the per-step kernel)
    (synth.LayerSpec(192, 320, 3, 1, 2, True, True, mxfp4=True), 37, (0, 3)),
])
def test_mxfp4_block_dots_bit_exact(spec, T, experts):
    q4, sc = synth.make_weights(spec, seed=6, device="cuda")
    L = coli.Layer.from_spec(spec, q4, sc)
    g = torch.Generator().manual_seed(T + 2)
    for e in experts:
        for m in (0, 1, 2):
            K = spec.inter if m == 2 else spec.hidden
            rows = spec.hidden if m == 2 else spec.inter
            a = torch.randint(-127, 128, (T, K), generator=g, dtype=torch.int8)
            a[0] = 127
            dots = torch.empty(T, rows, K // 32, dtype=torch.int32, device="cuda")
            coli.coli_moe_block_dots(L, e, m, a.cuda(), T, dots)
            torch.cuda.synchronize()
            qh, sh = synth.expert_slice(spec, q4, sc, [e])
            want = oracle.block_dots(spec.hidden, spec.inter, 1, 0, qh, sh, 0, m, a.numpy(),
                                     weights="mxfp4")
            assert np.array_equal(dots.cpu().numpy(), want), (e, m)


def _prefill(spec, T, seed=0, zipf=0.0, tokens=None, cover=None):
    print("mxfp4 prefill case: H=%d I=%d E=%d T=%d" % (spec.hidden, spec.inter, spec.n_experts, T),
          flush=True)
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
    err, n_budget = check_prefill_output(spec, L, g, x, y, toks)
    print("  rel err %.3g, %d elements within the boundary budget" % (err, n_budget), flush=True)
    return L, r, x, y


def test_mxfp4_prefill_olmoe_sampled():
    _prefill(_f4(synth.WORKLOADS["olmoe"].spec), 512, tokens=[0, 1, 63, 64, 511])


@pytest.mark.timeout(600)
def test_mxfp4_prefill_glm_every_tile():
    """GLM-shaped MXFP4 layer at 600 tokens: every (expert, 64-token tile)
    item's first and last row, the shared expert's tile boundaries and all
    tokens of the hottest expert (about 270 tokens)."""
    w = synth.WORKLOADS["glm_prefill"]
    _prefill(_f4(w.spec), 600, zipf=w.zipf_alpha, tokens=[300], cover=dict(tile=64, hottest=1))


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(256, 256, 6, 1, 2, sigmoid=True, renorm=True, mxfp4=True), 70),
    (synth.LayerSpec(1024, 768, 32, 0, 4, sigmoid=False, renorm=True, mxfp4=True), 129),
    # H, I not multiples of 256: the per-step kernel
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, mxfp4=True), 70),
    (synth.LayerSpec(2112, 1088, 8, 1, 3, sigmoid=False, renorm=True, mxfp4=True), 150),
])
def test_mxfp4_prefill_edge_shapes(spec, T):
    _prefill(spec, T, seed=3, zipf=0.6)
