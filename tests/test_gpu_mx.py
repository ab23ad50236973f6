"""GPU parity of the MX path (MXFP4 experts, COLI_ACT_MXFP8): the MXFP8
quantiser bit for bit, one matrix's MX GEMM against the oracle's exact block
sums within an fp32 accumulation bound, and the prefill layer output against
the oracle with the MXFP8 boundary budget of gpu_util.mx_flip_budget."""
import dataclasses

import numpy as np
import pytest
import torch

import bruteforce as bf
import int4_routed_expert_router_amd as coli
import oracle
import synth
from gpu_util import (check_prefill_output_mx, checked_route, cover_tokens, forward, gpu_layer,
                      run_route, sample_tokens)

pytestmark = pytest.mark.gpu


def _mx(spec):
    return dataclasses.replace(spec, mxfp4=True, mx_act=True)


def _quant(src: torch.Tensor, dtype):
    n = src.numel()
    q = torch.empty(n, dtype=torch.uint8, device="cuda")
    e = torch.empty(n // 32, dtype=torch.uint8, device="cuda")
    coli.coli_moe_quantize_mxfp8(src, dtype, n, q, e)
    torch.cuda.synchronize()
    return q.cpu().numpy(), e.cpu().numpy()


def test_quantize_mxfp8_bit_exact():
    g = torch.Generator().manual_seed(21)
    nb = 4096
    mags = 10.0 ** (torch.rand(nb, generator=g) * 16 - 10)  # 1e-10 .. 1e6
    v = (torch.randn(nb, 32, generator=g) * mags[:, None]).to(torch.float32)
    v[3] = 0.0
    v[4] = -0.0
    tab = torch.tensor(bf.e4m3_table())
    mids = 0.5 * (tab[:-1] + tab[1:])
    v[5, :31] = mids[torch.randint(0, len(mids), (31,), generator=g)] * 2.0 ** -3  # exact ties
    v[5, 31] = 448.0 * 2.0 ** -3
    v[6] = torch.tensor([500.0, 464.0, -470.0, 449.0] * 8)                       # saturation
    v[7] = 2.0 ** -126
    v[8, 1:] = torch.rand(31, generator=g) * 2.0 ** -7                           # subnormal codes
    v[8, 0] = 300.0
    v[9] = torch.tensor([3e38, -1e-30] * 16)
    q, e = _quant(v.reshape(-1).cuda(), coli.COLI_SRC_F32)
    qo, eo = oracle.quantize_mxfp8(v.reshape(-1).numpy())
    assert np.array_equal(e, eo)
    assert np.array_equal(q, qo)
    vb = v.to(torch.bfloat16)
    q, e = _quant(vb.reshape(-1).cuda(), coli.COLI_SRC_BF16)
    qo, eo = oracle.quantize_mxfp8(vb.to(torch.float32).reshape(-1).numpy())
    assert np.array_equal(e, eo)
    assert np.array_equal(q, qo)


def _mx_acts(T, K, g):
    """Valid random MXFP8 rows: codes without the NaN magnitude, E8M0 near 127."""
    qa = torch.randint(0, 256, (T, K), generator=g, dtype=torch.int32).to(torch.uint8)
    qa[(qa & 0x7F) == 0x7F] = 0x7E
    ea = torch.randint(118, 136, (T, K // 32), generator=g, dtype=torch.int32).to(torch.uint8)
    return qa, ea


@pytest.mark.parametrize("spec,T,experts", [
    (synth.LayerSpec(256, 256, 4, 1, 2, True, True, mxfp4=True), 5, (0, 4)),
    (synth.LayerSpec(512, 768, 3, 1, 2, True, True, mxfp4=True), 70, (1, 3)),
    (synth.LayerSpec(2048, 1024, 4, 1, 2, True, True, mxfp4=True), 129, (2,)),
    (synth.WORKLOADS["glm"].spec, 64, (17,)),
])
def test_mx_dots_vs_oracle(spec, T, experts):
    """fp32 MX GEMM of one matrix against the oracle's exact fp64 block sums:
    |err| within 2^-12 of the sum of the terms' magnitudes.  The instruction
    does not sum a block exactly when its E4M3 values span a wide range:
    measured on the GPU (in-bounds probe), E2M1 x E4M3 products over codes
    of every exponent carry errors up to ~2^-14.5 of the largest result,
    while codes of exponent <= 7 (subnormals included) agree to fp32
    rounding.  The layer tests hold the end-to-end bound."""
    spec = dataclasses.replace(spec, mxfp4=True)
    print("mx dots case: H=%d I=%d T=%d" % (spec.hidden, spec.inter, T), flush=True)
    n_exp = max(experts) + 1 if spec.hidden < 6144 else spec.n_total
    q4, sc = synth.make_weights(spec, seed=7, device="cuda", experts=n_exp)
    L = (coli.Layer(spec.hidden, spec.inter, n_exp - spec.n_shared, spec.n_shared, 1,
                    spec.flags, q4, sc, mxfp4=True)
         if spec.hidden < 6144 else coli.Layer.from_spec(spec, q4, sc))
    g = torch.Generator().manual_seed(T)
    for e in experts:
        qh, sh = synth.expert_slice(spec, q4, sc, [e])
        dense = bf.dense_experts(spec.hidden, spec.inter, 1, qh, sh, "mxfp4")[0]
        for m in (0, 1, 2):
            K = spec.inter if m == 2 else spec.hidden
            rows = spec.hidden if m == 2 else spec.inter
            qa, ea = _mx_acts(T, K, g)
            out = torch.empty(T, rows, dtype=torch.float32, device="cuda")
            coli.coli_moe_mx_dots(L, e, m, qa.cuda(), ea.cuda(), T, out)
            torch.cuda.synchronize()
            want = oracle.mx_dots(spec.hidden, spec.inter, 1, 0, qh, sh, 0, m, qa.numpy(),
                                  ea.numpy())
            mag = np.abs(bf.mxfp8_values(qa.numpy(), ea.numpy())) @ np.abs(dense[m]).T
            err = np.abs(out.cpu().numpy().astype(np.float64) - want)
            assert np.all(err <= 2.0 ** -12 * mag + 1e-30), (e, m, float(np.max(err / mag)))
            print("  expert %d matrix %d: max |err| / magnitude %.3g" % (e, m, float(np.max(err / mag))),
                  flush=True)


def _case(spec, T, seed=0, zipf=0.0, tokens=None, cover=None):
    print("mx prefill case: H=%d I=%d E=%d S=%d k=%d T=%d" % (
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
    err, n_budget = check_prefill_output_mx(spec, L, g, x, y, toks)
    print("  rel err %.3g, %d elements within the boundary budget" % (err, n_budget), flush=True)
    return L, r, x, y


@pytest.mark.parametrize("spec,T", [
    (synth.LayerSpec(256, 256, 8, 1, 2, sigmoid=True, renorm=True), 70),
    (synth.LayerSpec(768, 512, 8, 1, 2, sigmoid=True, renorm=True), 70),   # odd stage count
    (synth.LayerSpec(512, 768, 6, 0, 3, sigmoid=False, renorm=True), 129),
    (synth.LayerSpec(256, 256, 1, 1, 1, sigmoid=False, renorm=False), 1),
])
def test_mx_prefill_edge_shapes(spec, T):
    _case(_mx(spec), T, seed=3, zipf=0.6)


def test_mx_prefill_olmoe_sampled():
    _case(_mx(synth.WORKLOADS["olmoe"].spec), 512, tokens=[0, 1, 63, 64, 511],
          cover=dict(tile=64, hottest=1))


@pytest.mark.timeout(600)
def test_mx_prefill_glm_every_tile():
    """GLM-shaped MX layer at 600 tokens: every (expert, 64-token tile) item's
    first and last row, the shared expert's tile boundaries and all tokens
    of the hottest expert."""
    w = synth.WORKLOADS["glm_prefill"]
    _case(_mx(w.spec), 600, zipf=w.zipf_alpha, tokens=[300], cover=dict(tile=64, hottest=1))


@pytest.mark.timeout(900)
def test_mx_prefill_glm_16384_sampled():
    """The GLM-shaped MX layer at 16,384 tokens (the bench's extra run):
    each expert's first and last token, every tile boundary of the two
    hottest experts and sampled shared-expert tiles."""
    w = synth.WORKLOADS["glm_prefill"]
    spec = _mx(w.spec)
    print("mx prefill case: GLM layer, T=16384 (sampled)", flush=True)
    L = gpu_layer(spec, seed=0)
    T = 16384
    lg = synth.make_logits(spec, T, seed=0, zipf_alpha=w.zipf_alpha).cuda()
    x = synth.make_x(spec, T, seed=0).cuda()
    r = run_route(L, lg)
    y = forward(L, r, x, "prefill")
    g = checked_route(spec, r, lg)
    toks = sample_tokens(g, T, spec.top_k)
    print("  comparing %d tokens" % len(toks), flush=True)
    err, n_budget = check_prefill_output_mx(spec, L, g, x, y, toks)
    print("  rel err %.3g, %d elements within the boundary budget" % (err, n_budget), flush=True)


def test_mx_prefill_deterministic_and_bf16():
    spec = _mx(synth.WORKLOADS["a3b"].spec)
    L, r, x, y = _case(spec, 96, zipf=synth.ZIPF_ALPHA, tokens=[0, 95])
    assert torch.equal(forward(L, r, x, "prefill"), y)
    yb = forward(L, r, x, "prefill", y_dtype=coli.COLI_OUT_BF16)
    assert torch.equal(yb, y.to(torch.bfloat16))


def test_mx_prefill_unsupported_shape():
    spec = synth.LayerSpec(192, 320, 6, 1, 2, sigmoid=True, renorm=True, mxfp4=True, mx_act=True)
    L = gpu_layer(spec)
    r = run_route(L, synth.make_logits(spec, 4).cuda())
    with pytest.raises(coli.ColiError) as e:   # H, I not multiples of 256
        forward(L, r, synth.make_x(spec, 4).cuda(), "prefill")
    assert e.value.status == coli.binding.COLI_E_UNSUPPORTED
