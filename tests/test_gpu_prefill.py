"""GPU parity of the integer (Q8_0, int8 matrix-core) prefill path."""
import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth
from gpu_util import (check_prefill_output, checked_route, cover_tokens, forward, gpu_layer,
                      run_route, sample_tokens)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ Q8_0

def _q8(src: torch.Tensor, dtype):
    n = src.numel()
    q = torch.empty(n, dtype=torch.int8, device="cuda")
    d = torch.empty(n // 32, dtype=torch.int16, device="cuda")
    coli.coli_moe_quantize_q8_0(src, dtype, n, q, d)
    torch.cuda.synchronize()
    return q.cpu().numpy(), d.cpu().numpy().view(np.uint16)


def test_quantize_q8_0_bit_exact():
    g = torch.Generator().manual_seed(5)
    nb = 4096
    mags = 10.0 ** (torch.rand(nb, generator=g) * 12 - 8)  # 1e-8 .. 1e4
    v = (torch.randn(nb, 32, generator=g) * mags[:, None]).to(torch.float32)
    v[3] = 0.0
    v[4, :] = 0.5
    v[5, ::2] = -1.5e-5
    # fp32 source
    q, d = _q8(v.reshape(-1).cuda(), coli.COLI_SRC_F32)
    qo, do = oracle.quantize_q8_0(v.reshape(-1).numpy())
    assert np.array_equal(q, qo)
    assert np.array_equal(d, do)
    # bf16 source
    vb = v.to(torch.bfloat16)
    q, d = _q8(vb.reshape(-1).cuda(), coli.COLI_SRC_BF16)
    qo, do = oracle.quantize_q8_0(vb.to(torch.float32).reshape(-1).numpy())
    assert np.array_equal(q, qo)
    assert np.array_equal(d, do)


# ------------------------------------------------------------ block dots

@pytest.mark.parametrize("spec,T,experts", [
    (synth.LayerSpec(256, 128, 8, 0, 2, False, False), 4, (0, 7)),
    (synth.LayerSpec(192, 320, 3, 1, 2, True, True), 37, (0, 3)),
    (synth.LayerSpec(2048, 512, 4, 1, 2, True, True), 100, (2, 4)),
    (synth.WORKLOADS["glm"].spec, 64, (17,)),
])
def test_block_dots_bit_exact(spec, T, experts):
    print("block dots case: H=%d I=%d T=%d" % (spec.hidden, spec.inter, T), flush=True)
    n_exp = max(experts) + 1 if spec.hidden < 6144 else spec.n_total
    q4, sc = synth.make_weights(spec, seed=2, device="cuda", experts=n_exp)
    L = coli.Layer(spec.hidden, spec.inter, n_exp - spec.n_shared, spec.n_shared, 1,
                   spec.flags, q4, sc) if spec.hidden < 6144 else coli.Layer.from_spec(spec, q4, sc)
    g = torch.Generator().manual_seed(T)
    for e in experts:
        for m in (0, 1, 2):
            K = spec.inter if m == 2 else spec.hidden
            rows = spec.hidden if m == 2 else spec.inter
            a = torch.randint(-127, 128, (T, K), generator=g, dtype=torch.int8)
            a[0] = 127
            if T > 1:
                a[1] = -127
            dots = torch.empty(T, rows, K // 32, dtype=torch.int32, device="cuda")
            coli.coli_moe_block_dots(L, e, m, a.cuda(), T, dots)
            torch.cuda.synchronize()
            qh, sh = synth.expert_slice(spec, q4, sc, [e])
            want = oracle.block_dots(spec.hidden, spec.inter, 1, 0, qh, sh, 0, m, a.numpy())
            assert np.array_equal(dots.cpu().numpy(), want), (e, m)


# ---------------------------------------------------------- layer output

def _prefill_case(spec, T, seed=0, zipf=0.0, tokens=None, cover=None):
    print("prefill case: H=%d I=%d E=%d S=%d k=%d T=%d" % (
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
    # h is quantised to Q8_0 on both sides from fp32 values that differ by
    # rounding order, so a code on a rounding boundary may differ; the
    # comparison allows exactly those decisions (gpu_util.prefill_flip_budget)
    err, n_budget = check_prefill_output(spec, L, g, x, y, toks)
    print("  rel err %.3g, %d elements within the boundary budget" % (err, n_budget), flush=True)
    return L, r, x, y, toks


def test_prefill_tiny():
    w = synth.WORKLOADS["tiny"]
    _prefill_case(w.spec, 4)


def test_prefill_olmoe_512_sampled():
    w = synth.WORKLOADS["olmoe"]
    _prefill_case(w.spec, 512, tokens=[200, 333], cover=dict(tile=64, hottest=1))


@pytest.mark.timeout(600)
def test_prefill_glm_2048_every_tile():
    """The GLM-shaped prefill at 2,048 tokens: every (expert, 64-token tile)
    item's first and last row, every partial last tile, the shared expert's
    tile boundaries and all tokens of the three hottest experts, element by
    element (about 1,100 of the 2,048 tokens)."""
    w = synth.WORKLOADS["glm_prefill"]
    _prefill_case(w.spec, 2048, zipf=w.zipf_alpha, tokens=[777],
                  cover=dict(tile=64, hottest=3))


@pytest.mark.timeout(900)
def test_prefill_glm_16384_sampled():
    """The GLM-shaped layer at 16,384 tokens, the bench's extra compute-heavy
    run: each expert's first and last token, every tile boundary of the two
    hottest experts (about 570 tokens each) and sampled shared-expert tiles."""
    w = synth.WORKLOADS["glm_prefill"]
    print("prefill case: GLM layer, T=16384 (sampled)", flush=True)
    L = gpu_layer(w.spec, seed=0)
    T = 16384
    lg = synth.make_logits(w.spec, T, seed=0, zipf_alpha=w.zipf_alpha).cuda()
    x = synth.make_x(w.spec, T, seed=0).cuda()
    r = run_route(L, lg)
    y = forward(L, r, x, "prefill")
    g = checked_route(w.spec, r, lg)
    toks = sample_tokens(g, T, w.spec.top_k)
    print("  comparing %d tokens" % len(toks), flush=True)
    err, n_budget = check_prefill_output(w.spec, L, g, x, y, toks)
    print("  rel err %.3g, %d elements within the boundary budget" % (err, n_budget), flush=True)


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True), 70),
    (synth.LayerSpec(2048, 512, 256, 1, 8, sigmoid=True, renorm=True), 16),
    (synth.LayerSpec(64, 64, 1, 0, 1, sigmoid=False, renorm=False), 1),
    (synth.LayerSpec(1024, 448, 32, 0, 4, sigmoid=False, renorm=True), 129),
    # the most experts and the largest top-k (1024 experts, k = 32)
    (synth.LayerSpec(256, 256, 1024, 1, 32, sigmoid=True, renorm=True), 100),
])
def test_prefill_edge_shapes(spec, T):
    _prefill_case(spec, T, seed=3, zipf=0.6)


def test_prefill_maximum_batch_sampled():
    """65,536 tokens (the largest batch the entry point takes) on a small layer."""
    spec = synth.LayerSpec(256, 128, 8, 1, 2, sigmoid=True, renorm=True)
    _prefill_case(spec, 65536, seed=4, zipf=0.5, tokens=[0, 1, 4095, 32768, 65534, 65535])


def test_prefill_largest_hidden_sampled():
    spec = synth.LayerSpec(16384, 256, 4, 1, 2, sigmoid=False, renorm=True)
    _prefill_case(spec, 40, seed=5, tokens=[0, 39])


def test_prefill_deterministic_bf16_and_zero_scales():
    spec = synth.WORKLOADS["a3b"].spec
    L, r, x, y, toks = _prefill_case(spec, 96, zipf=synth.ZIPF_ALPHA)
    y2 = forward(L, r, x, "prefill")
    assert torch.equal(y, y2)
    yb = forward(L, r, x, "prefill", y_dtype=coli.COLI_OUT_BF16)
    assert torch.equal(yb, y.to(torch.bfloat16))
    Lz = coli.Layer.from_spec(spec, L.q4, torch.zeros_like(L.scales))
    assert not forward(Lz, r, x, "prefill").any()
