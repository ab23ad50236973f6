"""GPU parity of the float -> int8 gs64 quantiser (coli_moe_quantize_int8_gs64)
and the float -> MXFP4 conversion (coli_moe_quantize_mxfp4): codes and scales
bit-exact against the oracle for bf16 and fp32 sources, on seeded weights at
small ragged sizes, on edge groups and blocks (zeros, signed zeros, exact
ties, fp16-subnormal scales, the -128 code, E8M0 clamped at 0, fp32
subnormal inputs, saturation, the largest magnitudes), and on a 32-expert
shard of a H6144 I2048 container, sampled group by group, with the rounding
property checked on every group."""
import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth

pytestmark = pytest.mark.gpu

SRC = {"bf16": (torch.bfloat16, coli.COLI_SRC_BF16), "f32": (torch.float32, coli.COLI_SRC_F32)}
E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _code(w):
    return SRC["bf16"][1] if w.dtype == torch.bfloat16 else SRC["f32"][1]


def _int8(w: torch.Tensor, rows: int, K: int):
    q = torch.full((rows * K,), 0x5A, dtype=torch.int8, device="cuda")
    sc = torch.full((rows * K // 64,), 0x7E00, dtype=torch.int16, device="cuda")
    coli.coli_moe_quantize_int8_gs64(w, _code(w), rows, K, q, sc)
    torch.cuda.synchronize()
    return q, sc


def _mxfp4(w: torch.Tensor, rows: int, K: int):
    q = torch.full((rows * K // 2,), 0xA5, dtype=torch.uint8, device="cuda")
    e = torch.full((rows * K // 32,), 0xFF, dtype=torch.uint8, device="cuda")
    coli.coli_moe_quantize_mxfp4(w, _code(w), rows, K, q, e)
    torch.cuda.synchronize()
    return q, e


def _equal(name, got: torch.Tensor, want: np.ndarray):
    got = got.cpu().numpy().reshape(-1).view(want.dtype)
    bad = np.flatnonzero(got != want.reshape(-1))
    assert bad.size == 0, f"{bad.size} {name} differ, first at {bad[0]}"


def _int8_edges():
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                                      # zero group -> scale 0
    w[0, 64:128] = -np.abs(w[0, 64:128])                 # negative-only group
    h = np.concatenate([[127.0], np.arange(-126.5, 127.0, 4.0)[:63]])
    w[1, :64] = h * 2.0 ** -6                            # exact halves at scale 2^-6
    w[1, 64:128] = -h * 2.0 ** -3
    a = 127 * 2.4 * 2.0 ** -24                           # scale rounds down to 2^-23:
    w[2, :64] = rng.uniform(-a, a, 64)                   # codes clamp, -128 reached
    w[2, 0] = -a
    w[2, 64:128] = rng.uniform(-3e-6, 3e-6, 64)          # fp16-subnormal scales
    w[2, 128:192] = 1e-9                                 # a/127 below half the least fp16
    w[3] = rng.uniform(-8.3e6, 8.3e6, 256)               # largest valid magnitudes
    w[4, :64] = 1e-40                                    # fp32 subnormal inputs
    w[5, ::2] = 0.02
    w[5, 1::2] = -0.02                                   # all codes +-127
    return w


def _mxfp4_edges():
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], np.float32)
    t = np.concatenate([ties, -ties, ties * 0.5, -ties * 0.5])   # max 4 or 2: ties at
    w[0, :32] = t                                                # the block's scale 1
    w[0, 32:64] = t * 2.0 ** -20
    w[0, 64:96] = 0.0                                    # zero block -> E 0, codes 0
    w[0, 96:128] = -0.0                                  # ... with the sign kept
    w[0, 128:160] = np.linspace(-7.9, 7.9, 32)           # saturation at +-6
    w[1, :32] = 2.0 ** -131 * np.arange(32)              # fp32 subnormals: E clamps to 0
    w[1, 32:64] = 2.0 ** -126                            # least normal maximum
    w[1, 64:96] = -(2.0 ** -124) * 1.9                   # E 1, saturated codes
    w[1, 96:128] = rng.uniform(-3e38, 3e38, 32)          # largest exponents
    w[1, 128:160] = 1e-42
    w[2] = rng.standard_normal(256) * np.exp2(rng.integers(-40, 40, 256))  # mixed ranges
    w[3, 1::2] = -0.0
    return w


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("rows,K", [(1, 64), (3, 192), (7, 320), (33, 2048), (5, 6144)])
def test_int8_seeded_bit_exact(src, rows, K):
    w = synth.make_float_weights(rows * K, seed=3 * rows + K, dtype=SRC[src][0])
    q, sc = _int8(w.cuda(), rows, K)
    oq, osc = oracle.quantize_int8_gs64(w.float().numpy().reshape(rows, K))
    _equal("scales", sc, osc)
    _equal("codes", q, oq)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_int8_edges_bit_exact(src):
    w = torch.from_numpy(_int8_edges()).to(SRC[src][0])
    q, sc = _int8(w.reshape(-1).cuda(), 8, 256)
    oq, osc = oracle.quantize_int8_gs64(w.float().numpy())
    _equal("scales", sc, osc)
    _equal("codes", q, oq)
    assert np.any(oq[2, :64] == -128) and osc[0, 0] == 0 and np.all(oq[0, :64] == 0)


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("rows,K", [(1, 32), (3, 96), (7, 320), (33, 2048), (5, 6144)])
def test_mxfp4_seeded_bit_exact(src, rows, K):
    w = synth.make_float_weights(rows * K, seed=5 * rows + K, dtype=SRC[src][0])
    q, e = _mxfp4(w.cuda(), rows, K)
    oq, oe = oracle.quantize_mxfp4(w.float().numpy().reshape(rows, K))
    _equal("exponents", e, oe)
    _equal("codes", q, oq)


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_mxfp4_edges_bit_exact(src):
    w = torch.from_numpy(_mxfp4_edges()).to(SRC[src][0])
    q, e = _mxfp4(w.reshape(-1).cuda(), 8, 256)
    oq, oe = oracle.quantize_mxfp4(w.float().numpy())
    _equal("exponents", e, oe)
    _equal("codes", q, oq)
    assert oe[0, 2] == 0 and np.all(oq[0, 32:48] == 0) and np.all(oq[0, 48:64] == 0x88)
    assert oe[1, 0] == 0 and oe[1, 3] > 250


def _shard(seed):
    spec = synth.WORKLOADS["glm"].spec
    n = 32 * 3 * spec.inter * spec.hidden
    return synth.make_float_weights(n, seed=seed, device="cuda"), n // spec.hidden, spec.hidden


def _sample(nunits, seed):
    return torch.from_numpy(np.sort(np.random.default_rng(seed).choice(nunits, 4096,
                                                                       replace=False))).cuda()


def test_int8_full_shard_sampled_and_bounded():
    """32 experts of a H6144 I2048 container (gate | up | down each), bf16."""
    w, rows, K = _shard(23)
    q, sc = _int8(w, rows, K)
    ng = rows * K // 64
    gi = _sample(ng, 6)
    oq, osc = oracle.quantize_int8_gs64(w.view(ng, 64)[gi].float().cpu().numpy())
    _equal("scales", sc[gi], osc)
    _equal("codes", q.view(ng, 64)[gi], oq)
    step = 1 << 22
    for g0 in range(0, ng, step):
        g1 = min(ng, g0 + step)
        qq = q.view(ng, 64)[g0:g1].float()
        s = sc[g0:g1].view(torch.float16).float()[:, None]
        wf = w.view(ng, 64)[g0:g1].float()
        assert bool(torch.all(s[:, 0] >= 2.0 ** -14))
        assert bool(torch.all((wf - qq * s).abs() <= s * (0.5 + 2.0 ** -18)))
        amax = wf.abs().argmax(dim=1, keepdim=True)
        assert bool(torch.all(qq.gather(1, amax).abs() == 127))


def test_mxfp4_full_shard_sampled_and_nearest():
    """32 experts of a H6144 I2048 container, bf16: every code is a nearest
    E2M1 point of its weight over the block's power of two, and every
    block's largest weight takes code 4.0 or 6.0."""
    w, rows, K = _shard(29)
    q, e = _mxfp4(w, rows, K)
    nb = rows * K // 32
    bi = _sample(nb, 8)
    oq, oe = oracle.quantize_mxfp4(w.view(nb, 32)[bi].float().cpu().numpy())
    _equal("exponents", e[bi], oe)
    _equal("codes", q.view(nb, 16)[bi], oq)
    grid = torch.tensor(E2M1, device="cuda")
    lo = torch.tensor([0, .25, .25, .25, .25, .5, .5, 1.0], device="cuda")
    hi = torch.tensor([.25, .25, .25, .25, .5, .5, 1.0, float("inf")], device="cuda")
    step = 1 << 21
    for b0 in range(0, nb, step):
        b1 = min(nb, b0 + step)
        by = q.view(nb, 16)[b0:b1].to(torch.int64)
        c = torch.stack([by & 15, by >> 4], dim=2).reshape(b1 - b0, 32)
        mag = c & 7
        E = e[b0:b1].to(torch.int32)
        assert bool(torch.all(E > 0))
        m = torch.ldexp(w.view(nb, 32)[b0:b1].float(), (127 - E)[:, None].float()).abs()
        assert bool(torch.all((m >= grid[mag] - lo[mag]) & (m <= grid[mag] + hi[mag])))
        amax = m.argmax(dim=1, keepdim=True)
        assert bool(torch.all(mag.gather(1, amax) >= 6))
        assert bool(torch.all((c >= 8) == torch.signbit(w.view(nb, 32)[b0:b1])))
