"""GPU parity of the float -> int4 gs64 quantiser (coli_moe_quantize_int4_gs64):
nibbles and fp16 scales bit-exact against the oracle for bf16 and fp32 sources,
on seeded weights at small ragged sizes, on edge groups (zeros, exact halves,
fp16-subnormal scales, the -8 code, the largest valid magnitudes), and on a
32-expert shard of a H6144 I2048 container, sampled group by group, with the
error bound checked on every group."""
import numpy as np
import pytest
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth

pytestmark = pytest.mark.gpu

SRC = {"bf16": (torch.bfloat16, coli.COLI_SRC_BF16), "f32": (torch.float32, coli.COLI_SRC_F32)}


def _quantize(w: torch.Tensor, rows: int, K: int):
    """w: device tensor of rows*K values (bf16 or fp32)."""
    code = SRC["bf16"][1] if w.dtype == torch.bfloat16 else SRC["f32"][1]
    q4 = torch.full((rows * K // 2,), 0xA5, dtype=torch.uint8, device="cuda")
    sc = torch.full((rows * K // 64,), 0x7E00, dtype=torch.int16, device="cuda")
    coli.coli_moe_quantize_int4_gs64(w, code, rows, K, q4, sc)
    torch.cuda.synchronize()
    return q4, sc


def _oracle(w_host: torch.Tensor, rows: int, K: int):
    q4, sc = oracle.quantize_int4_gs64(w_host.float().numpy().reshape(rows, K))
    return q4.reshape(-1), sc.reshape(-1)


def _edge_matrix():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                                      # zero group -> scale 0
    w[0, 64:128] = -np.abs(w[0, 64:128])                 # negative-only group
    h = np.concatenate([[7.0], np.arange(-6.5, 7.0, 1.0), rng.integers(-14, 15, 49) / 2])
    w[1, :64] = h * 2.0 ** -6                            # exact halves at scale 2^-6
    w[1, 64:128] = -h * 2.0 ** -3
    w[2, :64] = rng.uniform(-5e-7, 5e-7, 64)             # fp16-subnormal scales
    w[2, 0] = -5e-7                                      # scale rounds down: reaches -8
    w[2, 64:128] = rng.uniform(-3e-7, 3e-7, 64)
    w[2, 128:192] = 1e-9                                 # a/7 below half the least fp16
    w[3] = rng.uniform(-458000, 458000, 256)             # largest valid magnitudes
    w[4, :64] = 1e-40                                    # fp32 subnormal inputs
    w[5, ::2] = 0.02
    w[5, 1::2] = -0.02                                   # all codes +-7
    return w


def _check_equal(q4, sc, oq, osc):
    q4 = q4.cpu().numpy()
    sc = sc.cpu().numpy().view(np.uint16)
    bad = np.flatnonzero(sc != osc)
    assert bad.size == 0, f"{bad.size} scales differ, first group {bad[0]}"
    bad = np.flatnonzero(q4 != oq)
    assert bad.size == 0, f"{bad.size} nibble bytes differ, first byte {bad[0]}"


@pytest.mark.parametrize("src", ["bf16", "f32"])
@pytest.mark.parametrize("rows,K", [(1, 64), (3, 192), (7, 320), (33, 2048), (5, 6144)])
def test_seeded_weights_bit_exact(src, rows, K):
    dtype, _ = SRC[src]
    w = synth.make_float_weights(rows * K, seed=rows + K, dtype=dtype)
    q4, sc = _quantize(w.cuda(), rows, K)
    _check_equal(q4, sc, *_oracle(w, rows, K))


@pytest.mark.parametrize("src", ["bf16", "f32"])
def test_edge_groups_bit_exact(src):
    dtype, _ = SRC[src]
    w = torch.from_numpy(_edge_matrix()).to(dtype)
    q4, sc = _quantize(w.reshape(-1).cuda(), 8, 256)
    oq, osc = _oracle(w, 8, 256)
    _check_equal(q4, sc, oq, osc)
    nib = np.stack([oq & 15, oq >> 4], axis=1).reshape(-1)
    assert np.any(nib[512:576] == 8)                     # the -8 code was exercised
    assert osc[0] == 0 and np.all(oq[:32] == 0)


def test_full_shard_sampled_and_bounded():
    """32 experts of a H6144 I2048 container (gate | up | down each), bf16."""
    spec = synth.WORKLOADS["glm"].spec
    n = 32 * 3 * spec.inter * spec.hidden
    w = synth.make_float_weights(n, seed=11, device="cuda")
    q4, sc = _quantize(w, n // spec.hidden, spec.hidden)
    ngroups = n // 64
    # bit-exact on 4096 sampled groups: each group is independent, so the
    # sampled groups form a [4096, 64] matrix for the oracle
    g = np.sort(np.random.default_rng(5).choice(ngroups, 4096, replace=False))
    gi = torch.from_numpy(g).cuda()
    wg = w.view(ngroups, 64)[gi].cpu()
    oq, osc = oracle.quantize_int4_gs64(wg.float().numpy())
    _check_equal(q4.view(ngroups, 32)[gi], sc[gi], oq.reshape(-1, 32), osc.reshape(-1))
    # every group: |w - q s| <= s/2 and the largest magnitude coded as 7
    step = 1 << 22
    for g0 in range(0, ngroups, step):
        g1 = min(ngroups, g0 + step)
        b = q4.view(ngroups, 32)[g0:g1].to(torch.int32)
        q = torch.stack([b & 15, b >> 4], dim=2).reshape(g1 - g0, 64)
        q = torch.where(q >= 8, q - 16, q)
        s = sc[g0:g1].view(torch.float16).float()[:, None]
        wf = w.view(ngroups, 64)[g0:g1].float()
        normal = s[:, 0] >= 2.0 ** -14          # fp16-normal scales: no clamping
        assert bool(torch.all(normal))
        assert bool(torch.all((wf - q * s).abs() <= s * (0.5 + 2.0 ** -18)))
        amax = wf.abs().argmax(dim=1, keepdim=True)
        assert bool(torch.all(q.gather(1, amax).abs() == 7))
