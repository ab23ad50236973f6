"""Pins of the CPU oracle against things other than itself (no GPU needed).

Each check compares the oracle with an independent numpy brute force, a
closed form, an invariant, or a hand-worked fixture under tests/golden/.  The
checks are plain functions so that test_oracle_mutants.py can rerun them on
deliberately broken copies of the oracle and see them fail.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import bruteforce as bf
import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# Small layer shapes that still cover several 64-groups per row, the shared
# expert, both routing functions and k > 1.
SOFTMAX_SMALL = synth.LayerSpec(128, 64, 6, 0, 2, sigmoid=False, renorm=False)
SIGMOID_SMALL = synth.LayerSpec(192, 128, 5, 1, 3, sigmoid=True, renorm=True)
TINY = synth.WORKLOADS["tiny"].spec


def _host_layer(spec, seed=0):
    q4, sc = synth.make_weights(spec, seed=seed)
    return q4.numpy(), (sc.numpy() if spec.mxfp4 else synth.f16_bits(sc))


def _x_bits(spec, T, seed=0):
    return synth.bf16_bits(synth.make_x(spec, T, seed=seed))


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------- numbers

def check_f16_rounding():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32) * np.float32(10.0) ** rng.integers(-9, 6, 2000),
        np.array([0.0, -0.0, 1.0, 65504.0, 65519.0, 65520.0, 1e9, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0], np.float32),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16_bits(v) for v in vals], np.uint16)
    assert np.array_equal(got, want)


def test_f16_rounding_matches_numpy():
    check_f16_rounding()


# -------------------------------------------------------------------- Q8_0

def check_q8_0_golden():
    g = json.load(open(os.path.join(GOLDEN, "q8_0_hand.json")))
    q, d = oracle.quantize_q8_0(np.array(g["blocks"], np.float32).reshape(-1))
    assert np.array_equal(q, np.array(g["q"], np.int8).reshape(-1))
    assert np.array_equal(d, np.array(g["d_fp16_bits"], np.uint16))


def check_q8_0_vs_bruteforce():
    rng = np.random.default_rng(2)
    v = (rng.standard_normal(32 * 500) * np.repeat(10.0 ** rng.uniform(-6, 4, 500), 32)).astype(np.float32)
    v[32 * 7:32 * 8] = 0.0  # an all-zero block
    q, d = oracle.quantize_q8_0(v)
    qb, db = bf.q8_0(v)
    assert np.array_equal(q, qb)
    assert np.array_equal(d, db.view(np.uint16))
    # properties: |q| <= 127, the max-magnitude element maps to +-127, and
    # the rounding error is at most half a step of the fp32 scale
    blocks = v.reshape(-1, 32)
    qq = q.reshape(-1, 32).astype(np.int32)
    assert np.abs(qq).max() <= 127
    for b in range(blocks.shape[0]):
        a = np.abs(blocks[b]).max()
        if a == 0:
            assert not qq[b].any()
            continue
        i = int(np.argmax(np.abs(blocks[b])))
        assert abs(qq[b, i]) == 127
        dd = np.float32(a / np.float32(127))
        assert np.all(np.abs(blocks[b].astype(np.float64) - qq[b] * float(dd)) <= 0.5 * float(dd) * (1 + 1e-6))


def test_q8_0_golden():
    check_q8_0_golden()


def test_q8_0_vs_bruteforce_and_properties():
    check_q8_0_vs_bruteforce()


# ------------------------------------------------------------------- route

def check_route_golden():
    g = json.load(open(os.path.join(GOLDEN, "route_hand.json")))
    lg = np.array(g["logits"], np.float32)
    r = oracle.route(lg, g["k"], 0)
    assert np.array_equal(r["topk_idx"], np.array(g["topk_idx"]))
    assert np.array_equal(r["counts"], np.array(g["counts"]))
    assert np.array_equal(r["offsets"], np.array(g["offsets"]))
    assert np.array_equal(r["pairs"], np.array(g["pairs"]))
    z = 2 * math.exp(0.5) + 2 * math.exp(2.0) + math.exp(-1.0)
    want0 = [math.exp(2.0) / z, math.exp(2.0) / z, math.exp(0.5) / z]
    assert np.allclose(r["topk_w"][0], want0, rtol=1e-7, atol=0)
    assert np.allclose(r["topk_w"][1], [0.2, 0.2, 0.2], rtol=1e-7, atol=0)
    rs = oracle.route(lg, g["k"], 1 | 256)
    assert np.allclose(rs["topk_w"][1], [1 / 3] * 3, rtol=1e-7, atol=0)
    s1 = 1 / (1 + math.exp(-2.0))
    s0 = 1 / (1 + math.exp(-0.5))
    assert np.allclose(rs["topk_w"][0], np.array([s1, s1, s0]) / (2 * s1 + s0), rtol=1e-7, atol=0)


def check_route_vs_bruteforce():
    rng = np.random.default_rng(3)
    for T, E, k in ((37, 8, 2), (50, 64, 8), (20, 256, 8), (9, 5, 5), (3, 300, 17)):
        lg = rng.standard_normal((T, E)).astype(np.float32)
        lg[:, ::3] = np.round(lg[:, ::3] * 2) / 2  # many exact ties
        bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
        for flags in (0, 256, 1, 1 | 256):
            for sb in (None, bias):
                r = oracle.route(lg, k, flags, 1.5, sel_bias=sb)
                idx = bf.topk(lg, k, sb)
                assert np.array_equal(r["topk_idx"], idx)
                w = bf.route_weights(lg, idx, flags & 1, flags & 256, 1.5)
                assert np.allclose(r["topk_w"], w, rtol=2e-7, atol=0)
                c, o, p = bf.group(idx, E)
                assert np.array_equal(r["counts"], c)
                assert np.array_equal(r["offsets"], o)
                assert np.array_equal(r["pairs"], p)


def check_route_invariants():
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((16, 12)).astype(np.float32)
    # softmax, k = E: the weights are the full softmax and sum to 1
    r = oracle.route(lg, 12, 0)
    assert np.allclose(r["topk_w"].astype(np.float64).sum(1), 1.0, atol=1e-6)
    # renormalised weights over the top-k sum to 1 for both functions
    for flags in (256, 1 | 256):
        r = oracle.route(lg, 4, flags)
        assert np.allclose(r["topk_w"].astype(np.float64).sum(1), 1.0, atol=1e-6)
    # equal logits and k = E: every weight is 1/E
    r = oracle.route(np.full((3, 12), 0.7, np.float32), 12, 0)
    assert np.allclose(r["topk_w"], 1 / 12, rtol=1e-6)
    assert np.array_equal(r["topk_idx"], np.tile(np.arange(12), (3, 1)))
    # a selection bias changes the choice but not the weights' source logits
    bias = np.zeros(12, np.float32)
    bias[11] = 100.0
    r = oracle.route(lg, 2, 1, sel_bias=bias)
    assert np.all(r["topk_idx"][:, 0] == 11)
    assert np.allclose(r["topk_w"][:, 0], 1 / (1 + np.exp(-lg[:, 11].astype(np.float64))), rtol=1e-7)


def test_route_golden():
    check_route_golden()


def test_route_vs_bruteforce():
    check_route_vs_bruteforce()


def test_route_invariants():
    check_route_invariants()


# ------------------------------------------------------------ decode layer

def _decode_case(spec, T, seed=0, zipf=0.0):
    q4, sc = _host_layer(spec, seed)
    lg = synth.make_logits(spec, T, seed=seed, zipf_alpha=zipf).numpy()
    r = oracle.route(lg, spec.top_k, spec.flags, spec.routed_scale)
    x = _x_bits(spec, T, seed)
    return q4, sc, r, x


def check_decode_vs_bruteforce():
    for spec, T in ((TINY, 4), (SOFTMAX_SMALL, 5), (SIGMOID_SMALL, 7)):
        q4, sc, r, x = _decode_case(spec, T, seed=5, zipf=0.3)
        s = spec
        y = oracle.forward_decode(s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k,
                                  q4, sc, r["topk_idx"], r["topk_w"], x)
        yb = bf.decode_layer(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sc,
                             r["topk_idx"], r["topk_w"], x)
        assert _rel(y, yb) < 1e-10


def check_decode_mean_invariant():
    # k = E, equal logits, softmax: y = mean over experts of FFN_e(x)
    spec = synth.LayerSpec(128, 64, 4, 0, 4, sigmoid=False, renorm=False)
    q4, sc = _host_layer(spec, 6)
    T = 3
    x = _x_bits(spec, T, 6)
    r = oracle.route(np.zeros((T, 4), np.float32), 4, 0)
    y = oracle.forward_decode(128, 64, 4, 0, 4, q4, sc, r["topk_idx"], r["topk_w"], x)
    outs = []
    for e in range(4):
        one = np.zeros((T, 1), np.int32) + e
        outs.append(oracle.forward_decode(128, 64, 4, 0, 1, q4, sc, one,
                                          np.ones((T, 1), np.float32), x))
    assert _rel(y, np.mean(outs, axis=0)) < 1e-12


def check_decode_zero_scales():
    spec = SIGMOID_SMALL
    q4, sc, r, x = _decode_case(spec, 3, seed=7)
    y = oracle.forward_decode(spec.hidden, spec.inter, spec.n_experts, spec.n_shared,
                              spec.top_k, q4, np.zeros_like(sc), r["topk_idx"], r["topk_w"], x)
    assert np.all(y == 0.0)


def check_decode_swiglu_mlp():
    # E = 1, k = 1, no shared expert: a plain SwiGLU MLP on the dequantised
    # weights, evaluated with torch's silu in fp64
    spec = synth.LayerSpec(192, 128, 1, 0, 1, sigmoid=False, renorm=False)
    q4, sc = _host_layer(spec, 8)
    T = 4
    x = _x_bits(spec, T, 8)
    r = oracle.route(np.zeros((T, 1), np.float32), 1, 0)
    y = oracle.forward_decode(192, 128, 1, 0, 1, q4, sc, r["topk_idx"], r["topk_w"], x)
    wg, wu, wd = (torch.from_numpy(m) for m in bf.dense_experts(192, 128, 1, q4, sc)[0])
    xt = torch.from_numpy(bf.bf16_to_f64(x))
    want = torch.nn.functional.linear(
        torch.nn.functional.silu(torch.nn.functional.linear(xt, wg))
        * torch.nn.functional.linear(xt, wu), wd)
    assert _rel(y, want.numpy()) < 1e-12


def _const_layer(H, I, gate_byte, up_byte, down_byte, s_gate, s_up, s_down):
    spec = synth.LayerSpec(H, I, 1, 0, 1, sigmoid=False, renorm=False)
    q4 = np.concatenate([np.full(I * H // 2, gate_byte, np.uint8),
                         np.full(I * H // 2, up_byte, np.uint8),
                         np.full(H * I // 2, down_byte, np.uint8)])
    sc = np.concatenate([np.full(I * H // 64, s_gate, np.float16),
                         np.full(I * H // 64, s_up, np.float16),
                         np.full(H * I // 64, s_down, np.float16)]).view(np.uint16)
    return spec, q4, sc


def check_decode_closed_form():
    # Nibble sign and order, scale grouping and SwiGLU by closed forms.
    H, I = 128, 64
    # gate byte 0x0F: even k -> low nibble 0xF = -1, odd k -> high nibble 0
    # up byte 0x2E: even k -> 0xE = -2, odd k -> 2
    # down byte 0x31: even n -> 1, odd n -> 3
    spec, q4, sc = _const_layer(H, I, 0x0F, 0x2E, 0x31, 0.5, 0.25, 2.0)
    xv = np.where(np.arange(H) % 2 == 0, 1.0, 3.0)  # x = 1 on even k, 3 on odd k
    x = (xv.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)[None, :]
    y = oracle.forward_decode(H, I, 1, 0, 1, q4, sc, np.zeros((1, 1), np.int32),
                              np.ones((1, 1), np.float32), x)
    g = 0.5 * (H // 2) * (-1 * 1.0)                          # = -32
    u = 0.25 * (H // 2) * ((-2) * 1.0 + 2 * 3.0)             # = 64
    h = g / (1 + math.exp(-g)) * u
    o = 2.0 * (I // 2) * (1 * h + 3 * h)
    assert np.allclose(y, o, rtol=1e-13, atol=0)
    # a per-group scale change: scale of group 1 of every gate row doubled
    sc2 = sc.copy().view(np.float16)
    sc2[1:I * H // 64:H // 64] = np.float16(1.0)
    y2 = oracle.forward_decode(H, I, 1, 0, 1, q4, sc2.view(np.uint16), np.zeros((1, 1), np.int32),
                               np.ones((1, 1), np.float32), x)
    g2 = 0.5 * 32 * -1 + 1.0 * 32 * -1                       # group 0 at 0.5, group 1 at 1.0
    h2 = g2 / (1 + math.exp(-g2)) * u
    assert np.allclose(y2, 2.0 * 32 * 4 * h2, rtol=1e-13, atol=0)


def test_decode_vs_bruteforce():
    check_decode_vs_bruteforce()


def test_decode_mean_invariant():
    check_decode_mean_invariant()


def test_decode_zero_scales():
    check_decode_zero_scales()


def test_decode_swiglu_mlp():
    check_decode_swiglu_mlp()


def test_decode_closed_form():
    check_decode_closed_form()


# ----------------------------------------------------- integer (Q8_0) path

def check_block_dots_vs_bruteforce():
    spec = SIGMOID_SMALL
    q4, sc = _host_layer(spec, 9)
    rng = np.random.default_rng(9)
    for m in (0, 1, 2):
        K = spec.inter if m == 2 else spec.hidden
        a = rng.integers(-127, 128, (3, K)).astype(np.int8)
        a[0, :32] = 127
        for e in (0, spec.n_total - 1):
            d = oracle.block_dots(spec.hidden, spec.inter, spec.n_experts, spec.n_shared, q4, sc,
                                  e, m, a)
            assert np.array_equal(d, bf.block_dots(spec.hidden, spec.inter, q4, e, m, a))
    # the full int4 x int8 product table: row 0 of a gate matrix holds the
    # nibbles 0..15 at k = 0..15; activation row (n, v) is v at k = n only
    H, I = 64, 64
    q4t = np.zeros(3 * H * I // 2, np.uint8)
    nib = np.arange(16, dtype=np.uint8)
    q4t[:8] = nib[0::2] | (nib[1::2] << 4)
    vals = np.arange(-127, 128)
    a = np.zeros((16 * vals.size, H), np.int8)
    for n in range(16):
        a[n * vals.size:(n + 1) * vals.size, n] = vals
    d = oracle.block_dots(H, I, 1, 0, q4t, np.zeros(3 * H * I // 64, np.uint16), 0, 0, a)
    signed = np.where(nib >= 8, nib.astype(np.int32) - 16, nib.astype(np.int32))
    want = (signed[:, None] * vals[None, :]).reshape(-1)
    assert np.array_equal(d[:, 0, 0], want)
    assert not d[:, 0, 1].any() and not d[:, 1:, :].any()
    worst = np.full(3 * H * I // 2, 0x88, np.uint8)  # every nibble -8
    a = np.full((1, H), -127, np.int8)
    d = oracle.block_dots(H, I, 1, 0, worst, np.zeros(3 * H * I // 64, np.uint16), 0, 0, a)
    assert np.all(d == 32 * 8 * 127)


def check_prefill_vs_bruteforce():
    for spec, T in ((TINY, 4), (SIGMOID_SMALL, 6)):
        q4, sc, r, x = _decode_case(spec, T, seed=10, zipf=0.3)
        s = spec
        y = oracle.forward_prefill(s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k,
                                   q4, sc, r["topk_idx"], r["topk_w"], x)
        yb = bf.prefill_layer(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sc,
                              r["topk_idx"], r["topk_w"], x)
        assert _rel(y, yb) < 1e-10
        # the integer path approximates the decode path to Q8_0 accuracy
        yd = oracle.forward_decode(s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k,
                                   q4, sc, r["topk_idx"], r["topk_w"], x)
        assert 1e-6 < _rel(y, yd) < 5e-2


def check_prefill_zero_scales():
    spec = SIGMOID_SMALL
    q4, sc, r, x = _decode_case(spec, 3, seed=11)
    y = oracle.forward_prefill(spec.hidden, spec.inter, spec.n_experts, spec.n_shared,
                               spec.top_k, q4, np.zeros_like(sc), r["topk_idx"], r["topk_w"], x)
    assert np.all(y == 0.0)


SIGMOID_SMALL_I8 = synth.LayerSpec(192, 128, 5, 1, 3, sigmoid=True, renorm=True, int8=True)
SOFTMAX_SMALL_I8 = synth.LayerSpec(128, 64, 6, 0, 2, sigmoid=False, renorm=False, int8=True)


def check_int8_decode_prefill_vs_bruteforce():
    for spec, T in ((SOFTMAX_SMALL_I8, 4), (SIGMOID_SMALL_I8, 5)):
        q4, sc, r, x = _decode_case(spec, T, seed=12, zipf=0.3)
        s = spec
        assert q4.size == s.n_total * 3 * s.hidden * s.inter  # one byte per weight
        args = (s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k, q4, sc, r["topk_idx"],
                r["topk_w"], x)
        y = oracle.forward_decode(*args, weights="int8")
        yb = bf.decode_layer(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sc,
                             r["topk_idx"], r["topk_w"], x, weights="int8")
        assert _rel(y, yb) < 1e-10
        yp = oracle.forward_prefill(*args, weights="int8")
        ypb = bf.prefill_layer(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sc,
                               r["topk_idx"], r["topk_w"], x, weights="int8")
        assert _rel(yp, ypb) < 1e-10
        assert 1e-6 < _rel(yp, y) < 5e-2


def check_int8_block_dots():
    spec = SIGMOID_SMALL_I8
    q4, sc = _host_layer(spec, 13)
    rng = np.random.default_rng(13)
    for m in (0, 2):
        K = spec.inter if m == 2 else spec.hidden
        a = rng.integers(-127, 128, (3, K)).astype(np.int8)
        for e in (0, spec.n_total - 1):
            d = oracle.block_dots(spec.hidden, spec.inter, spec.n_experts, spec.n_shared, q4, sc,
                                  e, m, a, weights="int8")
            assert np.array_equal(d, bf.block_dots(spec.hidden, spec.inter, q4, e, m, a,
                                                   weights="int8"))
    # every int8 code: row 0 of a gate matrix holds byte values 0..255 at
    # k = 0..255; activation row j is 127 (or -1) at k = j only
    H, I = 256, 64
    q8 = np.zeros(3 * H * I, np.uint8)
    q8[:256] = np.arange(256)
    a = np.zeros((512, H), np.int8)
    a[np.arange(256), np.arange(256)] = 127
    a[256 + np.arange(256), np.arange(256)] = -1
    z = np.zeros(3 * H * I // 64, np.uint16)
    d = oracle.block_dots(H, I, 1, 0, q8, z, 0, 0, a, weights="int8")
    code = np.arange(256).astype(np.uint8).view(np.int8).astype(np.int32)
    j = np.arange(256)
    assert np.array_equal(d[j, 0, j // 32], 127 * code)
    assert np.array_equal(d[256 + j, 0, j // 32], -code)
    assert not d[:, 1:, :].any()
    worst = np.full(3 * H * I, 0x80, np.uint8)  # every code -128
    d = oracle.block_dots(H, I, 1, 0, worst, z, 0, 0, np.full((1, H), -127, np.int8),
                          weights="int8")
    assert np.all(d == 32 * 128 * 127)


SIGMOID_SMALL_F4 = synth.LayerSpec(192, 128, 5, 1, 3, sigmoid=True, renorm=True, mxfp4=True)
SOFTMAX_SMALL_F4 = synth.LayerSpec(128, 64, 6, 0, 2, sigmoid=False, renorm=False, mxfp4=True)


def check_mxfp4_decode_prefill_vs_bruteforce():
    for spec, T in ((SOFTMAX_SMALL_F4, 4), (SIGMOID_SMALL_F4, 5)):
        q4, sc, r, x = _decode_case(spec, T, seed=14, zipf=0.3)
        s = spec
        assert sc.dtype == np.uint8 and sc.size == s.n_total * 3 * s.hidden * s.inter // 32
        # E8M0 extremes in the first expert's gate scales (fp64 decode path)
        sx = sc.copy()
        sx[:7] = (0, 1, 127, 128, 200, 254, 60)
        args = (s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k, q4, sx, r["topk_idx"],
                r["topk_w"], x)
        y = oracle.forward_decode(*args, weights="mxfp4")
        with np.errstate(over="ignore"):  # silu of a huge negative gate is -0
            yb = bf.decode_layer(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sx,
                                 r["topk_idx"], r["topk_w"], x, weights="mxfp4")
        assert _rel(y, yb) < 1e-10
        # the integer path keeps h in fp32: scales that keep it finite
        sc = sc.copy()
        sc[:7] = (100, 110, 127, 128, 130, 135, 60)
        args = (s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k, q4, sc, r["topk_idx"],
                r["topk_w"], x)
        yp = oracle.forward_prefill(*args, weights="mxfp4")
        ypb = bf.prefill_layer(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sc,
                               r["topk_idx"], r["topk_w"], x, weights="mxfp4")
        assert _rel(yp, ypb) < 1e-10


def check_mxfp4_block_dots():
    # the 16 E2M1 codes at k = 0..15 of row 0 (two per byte, low nibble
    # first); activation row j is 127 (or -1) at k = j only
    H, I = 64, 64
    q = np.zeros(3 * H * I // 2, np.uint8)
    nib = np.arange(16, dtype=np.uint8)
    q[:8] = nib[0::2] | (nib[1::2] << 4)
    a = np.zeros((32, H), np.int8)
    a[np.arange(16), np.arange(16)] = 127
    a[16 + np.arange(16), np.arange(16)] = -1
    z = np.full(3 * H * I // 32, 127, np.uint8)
    d = oracle.block_dots(H, I, 1, 0, q, z, 0, 0, a, weights="mxfp4")
    doubled = np.array([0, 1, 2, 3, 4, 6, 8, 12, 0, -1, -2, -3, -4, -6, -8, -12])
    assert np.array_equal(d[np.arange(16), 0, 0], 127 * doubled)
    assert np.array_equal(d[16 + np.arange(16), 0, 0], -doubled)
    assert not d[:, 1:, :].any() and not d[:, 0, 1:].any()
    spec = SIGMOID_SMALL_F4
    q4, sc = _host_layer(spec, 15)
    rng = np.random.default_rng(15)
    for m in (0, 2):
        K = spec.inter if m == 2 else spec.hidden
        a = rng.integers(-127, 128, (3, K)).astype(np.int8)
        dd = oracle.block_dots(spec.hidden, spec.inter, spec.n_experts, spec.n_shared, q4, sc,
                               spec.n_total - 1, m, a, weights="mxfp4")
        assert np.array_equal(dd, bf.block_dots(spec.hidden, spec.inter, q4, spec.n_total - 1,
                                                m, a, weights="mxfp4"))


def test_mxfp4_decode_prefill_vs_bruteforce():
    check_mxfp4_decode_prefill_vs_bruteforce()


def test_mxfp4_block_dots():
    check_mxfp4_block_dots()


def test_block_dots_vs_bruteforce():
    check_block_dots_vs_bruteforce()


def test_int8_decode_prefill_vs_bruteforce():
    check_int8_decode_prefill_vs_bruteforce()


def test_int8_block_dots():
    check_int8_block_dots()


def test_prefill_vs_bruteforce():
    check_prefill_vs_bruteforce()


def test_prefill_zero_scales():
    check_prefill_zero_scales()


# ----------------------------------------------------------- router logits

def _bf16(a):
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def check_router_logits_closed_form():
    """Integer inputs make every partial sum exact: the logits are the exact
    integer matrix product.  A one-hot activation selects a weight column."""
    rng = np.random.default_rng(21)
    T, E, H = 4, 7, 160
    xi = rng.integers(-8, 9, size=(T, H))
    wi = rng.integers(-8, 9, size=(E, H))
    lg = oracle.router_logits(synth.bf16_bits(_bf16(wi)), synth.bf16_bits(_bf16(xi)))
    assert np.array_equal(lg, (xi @ wi.T).astype(np.float32))
    onehot = np.zeros((1, H), np.float32)
    onehot[0, 37] = 1.0
    w = rng.standard_normal((E, H)).astype(np.float32)
    wb = _bf16(w)
    lg1 = oracle.router_logits(synth.bf16_bits(wb), synth.bf16_bits(_bf16(onehot)))
    assert np.array_equal(lg1[0], wb.float().numpy()[:, 37])


def check_router_logits_vs_bruteforce():
    """Random bf16 inputs against a dense fp64 product (summation order may
    differ, so the fp32 results agree to one unit in the last place)."""
    rng = np.random.default_rng(22)
    T, E, H = 5, 12, 192
    xb = _bf16(rng.standard_normal((T, H)))
    wb = _bf16(rng.standard_normal((E, H)) * 0.05)
    lg = oracle.router_logits(synth.bf16_bits(wb), synth.bf16_bits(xb))
    ref = (xb.double().numpy() @ wb.double().numpy().T).astype(np.float32)
    assert np.all(np.abs(lg - ref) <= np.spacing(np.abs(ref)))


def test_router_logits_closed_form():
    check_router_logits_closed_form()


def test_router_logits_vs_bruteforce():
    check_router_logits_vs_bruteforce()


# ------------------------------------------------------- int4 quantiser

def _int4_bruteforce(w):
    """Independent numpy statement of the container quantiser."""
    w = np.asarray(w, np.float32)
    rows, K = w.shape
    g = w.reshape(rows, K // 64, 64)
    a = np.max(np.abs(g), axis=2)
    s16 = (a / np.float32(7.0)).astype(np.float16)          # fp32 division, RNE to fp16
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / sf[:, :, None]).astype(np.float64)      # fp32 division, exact widen
    r = np.sign(ratio) * np.floor(np.abs(ratio) + 0.5)        # half away from zero
    r = np.where(sf[:, :, None] == 0, 0, np.clip(r, -8, 7)).astype(np.int64).reshape(rows, K)
    nib = (r & 15).astype(np.uint8)
    q4 = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return q4, s16.view(np.uint16)


def _int4_cases():
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                                    # all-zero group
    w[1, 64:128] = -np.abs(w[1, 64:128])               # negative-only group
    w[2, :64] = np.round(rng.standard_normal(64) * 4) / 8  # exact halves after scaling
    w[3, :64] = rng.uniform(-5e-7, 5e-7, 64)           # subnormal fp16 scales
    w[3, 0] = -5e-7                                    # negative max: the scale rounds down,
    w[3, 64:128] = rng.uniform(-3e-7, 3e-7, 64)        # so this group reaches -8
    w[4] = rng.uniform(-400000, 400000, 256)           # near the largest valid scale
    return w


def check_int4_quant_vs_bruteforce():
    w = _int4_cases()
    q4, sc = oracle.quantize_int4_gs64(w)
    bq, bs = _int4_bruteforce(w)
    assert np.any(q4[3] & 15 == 8) or np.any(q4[3] >> 4 == 8)   # the case reaches -8
    assert np.array_equal(sc, bs)
    assert np.array_equal(q4, bq)


def check_int4_quant_closed_form():
    """w = q * 2^-6 with max |q| = 7 in every group gives back q and 2^-6."""
    rng = np.random.default_rng(32)
    q = rng.integers(-7, 8, size=(4, 128))
    q[:, 0] = 7
    q[:, 64] = -7
    w = (q * 2.0 ** -6).astype(np.float32)
    q4, sc = oracle.quantize_int4_gs64(w)
    assert np.all(sc == 0x2400)                      # fp16 bits of 2^-6
    nib = (q & 15).astype(np.uint8)
    assert np.array_equal(q4, nib[:, 0::2] | (nib[:, 1::2] << 4))
    # exact halves (scale 2^-6 again) round away from zero
    h = np.concatenate([[7.0], np.arange(-6.5, 7.0, 1.0), np.full(49, 0.5)])
    q4, sc = oracle.quantize_int4_gs64((h * 2.0 ** -6).astype(np.float32)[None, :])
    qh = np.sign(h) * np.floor(np.abs(h) + 0.5)
    nib = (qh.astype(np.int64) & 15).astype(np.uint8)
    assert sc[0, 0] == 0x2400
    assert np.array_equal(q4[0], nib[0::2] | (nib[1::2] << 4))
    z4, zs = oracle.quantize_int4_gs64(np.zeros((2, 64), np.float32))
    assert np.all(z4 == 0) and np.all(zs == 0)


def check_int4_quant_properties():
    rng = np.random.default_rng(33)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    q4, sc = oracle.quantize_int4_gs64(w)
    lo = (q4 & 15).astype(np.int64)
    hi = (q4 >> 4).astype(np.int64)
    q = np.empty((16, 512), np.int64)
    q[:, 0::2], q[:, 1::2] = lo, hi
    q = np.where(q >= 8, q - 16, q)
    sf = sc.view(np.float16).astype(np.float64).repeat(64, axis=1)
    assert np.all(np.abs(w - q * sf) <= sf / 2 * (1 + 1e-6))
    g = np.abs(w).reshape(16, 8, 64).argmax(axis=2)
    qg = q.reshape(16, 8, 64)
    assert np.all(np.abs(np.take_along_axis(qg, g[:, :, None], 2)) == 7)


def _int8_bruteforce(w):
    w = np.asarray(w, np.float32)
    rows, K = w.shape
    g = w.reshape(rows, K // 64, 64)
    a = np.max(np.abs(g), axis=2)
    s16 = (a / np.float32(127.0)).astype(np.float16)
    sf = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / sf[:, :, None]).astype(np.float64)
    r = np.sign(ratio) * np.floor(np.abs(ratio) + 0.5)
    r = np.where(sf[:, :, None] == 0, 0, np.clip(r, -128, 127))
    return r.astype(np.int8).reshape(rows, K), s16.view(np.uint16)


def check_int8_quant():
    w = _int4_cases()
    # a negative maximum whose fp16 scale (a subnormal, 10 * 2^-24) rounds
    # down by 4.5 %: its code would be -132.7, clamped to -128
    w[5, :64] = np.linspace(-7e-5, 7e-5, 64)
    w[5, 0] = -127 * 10.45 * 2.0 ** -24
    q, sc = oracle.quantize_int8_gs64(w)
    bq, bs = _int8_bruteforce(w)
    assert np.array_equal(sc, bs) and np.array_equal(q, bq)
    assert (q == -128).any()                     # the subnormal-scale groups reach -128
    # closed form: w = q * 2^-6 with max |q| = 127 gives back q and 2^-6
    rng = np.random.default_rng(34)
    qq = rng.integers(-127, 128, size=(3, 128))
    qq[:, 0], qq[:, 64] = 127, -127
    q2, s2 = oracle.quantize_int8_gs64((qq * 2.0 ** -6).astype(np.float32))
    assert np.all(s2 == 0x2400) and np.array_equal(q2, qq)


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mxfp4_bruteforce(w):
    """Shared exponent from the fp32 bit patterns; each element the nearest
    of the 16 codes' values, ties to the code with an even magnitude index."""
    w = np.asarray(w, np.float32)
    rows, K = w.shape
    blk = w.reshape(rows, K // 32, 32)
    a = np.max(np.abs(blk), axis=2)
    bits = a.view(np.uint32)
    expf = ((bits >> 23) & 0xFF).astype(np.int64)
    floor_log2 = np.where(expf > 0, expf - 127, 0)
    sub = (expf == 0) & (a > 0)
    if sub.any():                                   # subnormal maxima: E clamps to 0 anyway
        floor_log2 = np.where(sub, -150, floor_log2)
    E = np.where(a > 0, np.clip(floor_log2 - 2 + 127, 0, 254), 0).astype(np.int64)
    v = blk.astype(np.float64) * np.exp2(127.0 - E)[:, :, None]
    m = np.abs(v)
    dist = np.abs(m[..., None] - E2M1_VALUES)
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best
    even = cand & (np.arange(8) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    idx = np.where(m > 6.0, 7, idx)
    code = idx | np.where(np.signbit(blk), 8, 0)
    code = code.reshape(rows, K).astype(np.uint8)
    return code[:, 0::2] | (code[:, 1::2] << 4), E.astype(np.uint8)


def check_mxfp4_quant():
    rng = np.random.default_rng(35)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    w[0, :32] = 0.0
    w[0, 32:64] = -0.0
    w[1, :32] = rng.uniform(-1e-39, 1e-39, 32)               # subnormal maximum
    w[2, :32] = np.array([6, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, 5] * 4) * 2.0 ** -9  # ties
    w[2, 32:64] = np.array([7, 6.5, -7.9, 0.3] * 8) * 2.0 ** -9                      # saturation
    w[3] = rng.uniform(-3e38, 3e38, 128)                     # near the fp32 maximum
    w[4, :32] = 2.0 ** -126                                  # exact power of two maxima
    q, e = oracle.quantize_mxfp4(w)
    bq, be = _mxfp4_bruteforce(w)
    assert np.array_equal(e, be) and np.array_equal(q, bq)
    # the tie row: max 6 * 2^-9 gives X = -9 (E 118); ties go to the even code
    assert e[2, 0] == 118
    codes = np.stack([q[2] & 15, q[2] >> 4], axis=1).reshape(-1)[:8]
    assert list(codes) == [7, 6, 4, 4, 2, 2, 0, 6]
    # closed form: values on the grid times 2^X round-trip
    vals = rng.choice(np.concatenate([E2M1_VALUES, -E2M1_VALUES[1:]]), size=(2, 64))
    vals[:, 0] = vals[:, 32] = 6.0
    q2, e2 = oracle.quantize_mxfp4((vals * 2.0 ** -5).astype(np.float32))
    assert np.all(e2 == 127 - 5)
    c2 = np.stack([q2 & 15, q2 >> 4], axis=2).reshape(2, 64)
    dec = E2M1_VALUES[c2 & 7] * np.where(c2 & 8, -1.0, 1.0)
    assert np.array_equal(dec, vals)


# ---------------------------------------------------- MX activation path

def check_mxfp8_quant():
    rng = np.random.default_rng(41)
    v = (rng.standard_normal((8, 64)) * 10.0 ** rng.uniform(-6, 6, (8, 1))).astype(np.float32)
    v[0, :32] = 0.0
    v[0, 32:] = -0.0
    v[1, :32] = rng.uniform(-1e-39, 1e-39, 32)                     # fp32 subnormal maximum
    tab = bf.e4m3_table()
    mids = 0.5 * (tab[:-1] + tab[1:])
    v[2, :31] = mids[rng.choice(len(mids), 31)] * 2.0 ** -20        # exact ties
    v[2, 31] = 448.0 * 2.0 ** -20                                   # fixes the block exponent
    v[2, 32:64] = np.array([500.0, 464.0, -470.0, 449.0] * 8) * 2.0 ** 3   # saturation at 448
    v[3] = rng.uniform(-3e38, 3e38, 64)                             # near the fp32 maximum
    v[4, :32] = 2.0 ** -126                                         # exact power-of-two maxima
    v[5, :32] = np.concatenate([[256.0], rng.uniform(-2.0 ** -6, 2.0 ** -6, 31)])  # E4M3 subnormals
    q, e = oracle.quantize_mxfp8(v)
    bq, be = bf.mxfp8(v)
    assert np.array_equal(e, be) and np.array_equal(q, bq)
    # scale bytes are [row * 2 + block]: the tie block has max 448 * 2^-20
    # (E 127 - 20), the saturation block 500 * 2^3 (floor log2 = 11, E 130),
    # 2^-126 maxima clamp E to 0, and a block whose maximum is 256 has E 127
    assert e[4] == 107 and e[5] == 130 and e[8] == 0 and e[10] == 127
    assert np.all(q[128 + 32:128 + 64] & 0x7F == 0x7E)             # saturated magnitudes
    assert np.all(q[256:256 + 32] == 0x40)                          # 2^-126 / 2^-127 = 2.0
    assert q[0] == 0x00 and q[32] == 0x80                           # +0 and -0
    # closed form: table values times 2^X round-trip
    vals = rng.choice(np.concatenate([tab, -tab[1:]]), size=(3, 64))
    vals[:, 0] = vals[:, 32] = 448.0
    q2, e2 = oracle.quantize_mxfp8((vals * 2.0 ** -11).astype(np.float32))
    assert np.all(e2 == 127 - 11)
    assert np.array_equal(bf.mxfp8_values(q2.reshape(3, 64), e2.reshape(3, 2)),
                          vals * 2.0 ** -11)


def check_mx_dots():
    # E2M1 codes 0..15 at k = 0..15 of row 0, activation row j one-hot at k = j
    H, I = 64, 64
    q = np.zeros(3 * H * I // 2, np.uint8)
    nib = np.arange(16, dtype=np.uint8)
    q[:8] = nib[0::2] | (nib[1::2] << 4)
    z = np.full(3 * H * I // 32, 127, np.uint8)
    z[0] = 130                                                      # 2^3 on row 0, block 0
    qa = np.zeros((16, H), np.uint8)
    qa[np.arange(16), np.arange(16)] = 0x3A                         # E4M3 1.25
    ea = np.full((16, H // 32), 125, np.uint8)                      # 2^-2
    out = oracle.mx_dots(H, I, 1, 0, q, z, 0, 0, qa, ea)
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6])
    assert np.array_equal(out[:, 0], e2m1 * 1.25 * 2.0 ** 3 * 2.0 ** -2)
    assert not out[:, 1:].any()
    # random codes and scales against the dense brute force
    spec = SIGMOID_SMALL_F4
    q4, sc = _host_layer(spec, 16)
    rng = np.random.default_rng(16)
    for m in (0, 1, 2):
        K = spec.inter if m == 2 else spec.hidden
        qa = rng.integers(0, 256, (3, K)).astype(np.uint8)
        qa[(qa & 0x7F) == 0x7F] = 0x7E
        ea = rng.integers(117, 138, (3, K // 32)).astype(np.uint8)
        got = oracle.mx_dots(spec.hidden, spec.inter, spec.n_experts, spec.n_shared, q4, sc,
                             spec.n_total - 1, m, qa, ea)
        wmat = bf.dense_experts(spec.hidden, spec.inter, spec.n_total, q4, sc, "mxfp4")[-1][m]
        want = bf.mxfp8_values(qa, ea) @ wmat.T
        assert _rel(got, want) < 1e-12


def check_prefill_mx_vs_bruteforce():
    for spec, T in ((SOFTMAX_SMALL_F4, 4), (SIGMOID_SMALL_F4, 5)):
        q4, sc, r, x = _decode_case(spec, T, seed=17, zipf=0.3)
        s = spec
        sc = sc.copy()
        sc[:7] = (100, 110, 127, 128, 130, 135, 60)
        args = (s.hidden, s.inter, s.n_experts, s.n_shared, s.top_k, q4, sc, r["topk_idx"],
                r["topk_w"], x)
        y = oracle.forward_prefill_mx(*args)
        yb = bf.prefill_layer_mx(s.hidden, s.inter, s.n_experts, s.n_shared, q4, sc,
                                 r["topk_idx"], r["topk_w"], x)
        assert _rel(y, yb) < 1e-10


def test_mxfp8_quant():
    check_mxfp8_quant()


def test_mx_dots():
    check_mx_dots()


def test_prefill_mx_vs_bruteforce():
    check_prefill_mx_vs_bruteforce()


def test_int8_quant():
    check_int8_quant()


def test_mxfp4_quant():
    check_mxfp4_quant()


def test_int4_quant_vs_bruteforce():
    check_int4_quant_vs_bruteforce()


def test_int4_quant_closed_form():
    check_int4_quant_closed_form()


def test_int4_quant_properties():
    check_int4_quant_properties()


# ------------------------------------------------------- container identity

def test_container_sizes_match_the_pages():
    """One GLM-shaped expert is about 19 MB and 19,456 of them about 370 GB
    (tantan.ink post on colibri, section 它的核心判断); twelve resident layers
    of 257 experts are about 58 GB.  These pin gs64 with fp16 scales."""
    glm = synth.WORKLOADS["glm"].spec
    assert glm.expert_bytes == 18_874_368
    assert glm.expert_total_bytes == 20_054_016
    assert 18.5 < glm.expert_total_bytes / 2**20 < 19.5          # ~19 MB (MiB)
    assert 350 < 19_456 * glm.expert_total_bytes / 2**30 < 375  # ~370 GB
    assert 57 < synth.container_gib(glm, 12) < 59               # ~58 GB
    # per-row scales (the superseded container) would be ~5% smaller
    assert glm.expert_total_bytes / glm.expert_bytes == pytest.approx(1 + 1 / 16)


def test_zipf_counts_shape():
    """The prefill workload's skew gives per-expert counts of about 0-400."""
    w = synth.WORKLOADS["glm_prefill"]
    lg = synth.make_logits(w.spec, 2048, seed=0, zipf_alpha=w.zipf_alpha).numpy()
    idx = bf.topk(lg, 8)
    c = np.bincount(idx.reshape(-1), minlength=256)
    assert c.sum() == 2048 * 8
    assert 250 <= c.max() <= 500
    assert c.min() <= 40
