"""The Q8_0 boundary budget used by the GPU prefill comparisons, checked on
the CPU: when the brute force's h is perturbed by a few fp32 ulps (the kind of
difference a different summation order makes), its output moves by more
than the plain tolerance on int8 layers, and every such move stays within
the budget prefill_flip_budget derives from the oracle."""
import numpy as np
import pytest

import bruteforce as bf
import oracle
import synth
from gpu_util import prefill_flip_budget


class _HostLayer:
    def __init__(self, q4, scales):
        self.q4, self.scales = q4, scales


@pytest.mark.parametrize("shape,int8", [((256, 256), True), ((1024, 768), True),
                                        ((512, 512), False)])
def test_budget_covers_boundary_decisions(shape, int8):
    spec = synth.LayerSpec(shape[0], shape[1], 6, 1, 2, sigmoid=True, renorm=True, int8=int8)
    q4, sc = synth.make_weights(spec, seed=3)
    T = 24
    lg = synth.make_logits(spec, T, seed=3, zipf_alpha=0.6).numpy()
    r = oracle.route(lg, spec.top_k, spec.flags, spec.routed_scale)
    x = synth.make_x(spec, T, seed=3)
    ref, budget = prefill_flip_budget(spec, _HostLayer(q4, sc), r["topk_idx"].reshape(-1),
                                      r["topk_w"].reshape(-1), x, range(T))
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    assert np.median(budget / den) < 1e-4          # the budget is local, not a blanket
    orig = bf.q8_0
    for trial in range(2):
        rng = np.random.default_rng(trial)
        calls = [0]

        def perturbed(v):
            calls[0] += 1
            v = np.asarray(v, np.float32)
            if calls[0] > 1:  # h only (the first call quantises x)
                v = (v * (1 + 2.0 ** -22 * rng.standard_normal(v.shape))).astype(np.float32)
            return orig(v)

        bf.q8_0 = perturbed
        try:
            y = bf.prefill_layer(spec.hidden, spec.inter, spec.n_experts, spec.n_shared,
                                 q4.numpy(), synth.f16_bits(sc), r["topk_idx"], r["topk_w"],
                                 synth.bf16_bits(x), weights=spec.weights)
        finally:
            bf.q8_0 = orig
        assert np.all(np.abs(y - ref) <= 1e-5 * den + budget)


@pytest.mark.parametrize("shape", [(256, 256), (512, 384)])
def test_mx_budget_covers_boundary_decisions(shape):
    """The same for the MX path (MXFP4 weights, MXFP8 activations):
    mx_flip_budget covers the output moves of h perturbed by 2^-16 relative
    (E4M3 code and shared-exponent decisions), and stays local."""
    from gpu_util import mx_flip_budget
    spec = synth.LayerSpec(shape[0], shape[1], 6, 1, 2, sigmoid=True, renorm=True, mxfp4=True,
                           mx_act=True)
    q4, sc = synth.make_weights(spec, seed=4)
    T = 24
    lg = synth.make_logits(spec, T, seed=4, zipf_alpha=0.6).numpy()
    r = oracle.route(lg, spec.top_k, spec.flags, spec.routed_scale)
    x = synth.make_x(spec, T, seed=4)
    ref, budget = mx_flip_budget(spec, _HostLayer(q4, sc), r["topk_idx"].reshape(-1),
                                 r["topk_w"].reshape(-1), x, range(T))
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    den = np.maximum(np.abs(ref), rms)
    # local, though larger than the Q8_0 one: an E4M3 code step is 1/16 to 1/8
    # of its value, and the band covers the MX instruction's own rounding
    assert np.median(budget / den) < 5e-3
    orig = bf.mxfp8
    moved = 0
    for trial in range(3):
        rng = np.random.default_rng(trial)
        calls = [0]

        def perturbed(v):
            calls[0] += 1
            v = np.asarray(v, np.float32)
            if calls[0] > 1:  # h only (the first call quantises x)
                v = (v * (1 + 2.0 ** -16 * rng.standard_normal(v.shape))).astype(np.float32)
            return orig(v)

        bf.mxfp8 = perturbed
        try:
            y = bf.prefill_layer_mx(spec.hidden, spec.inter, spec.n_experts, spec.n_shared,
                                    q4.numpy(), sc.numpy(), r["topk_idx"], r["topk_w"],
                                    synth.bf16_bits(x))
        finally:
            bf.mxfp8 = orig
        moved += int(np.count_nonzero(np.abs(y - ref) > 1e-5 * den))
        assert np.all(np.abs(y - ref) <= 1e-5 * den + budget)
    assert moved > 0  # the perturbation does flip decisions: the budget is exercised
