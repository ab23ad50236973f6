"""The allocation-free decode entry point (library-owned scratch) against the
workspace entry point: the same kernels, so the outputs must be identical,
on two calls in a row with the second smaller, on two layer shapes."""
import pytest
import torch

import int4_routed_expert_router_amd as coli
import synth
from gpu_util import forward, gpu_layer, run_route

pytestmark = pytest.mark.gpu


def _noalloc(L, r, x, y_dtype):
    T = x.shape[0]
    y = torch.empty(T, L.hidden, device="cuda",
                    dtype=torch.float32 if y_dtype == coli.COLI_OUT_F32 else torch.bfloat16)
    coli.coli_moe_forward_decode_noalloc(L, r, x, T, y, y_dtype)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name,sizes", [("a3b", (16, 3)), ("glm", (4, 1))])
def test_noalloc_matches_workspace_entry(name, sizes):
    w = synth.WORKLOADS[name]
    spec = w.spec
    L = gpu_layer(spec, seed=7)
    for i, T in enumerate(sizes):
        print("noalloc case: %s T=%d (call %d)" % (name, T, i + 1), flush=True)
        lg = synth.make_logits(spec, T, seed=7 + i, zipf_alpha=w.zipf_alpha).cuda()
        x = synth.make_x(spec, T, seed=7 + i).cuda()
        r = run_route(L, lg)
        for y_dtype in (coli.COLI_OUT_F32, coli.COLI_OUT_BF16):
            want = forward(L, r, x, "decode", y_dtype=y_dtype)
            got = _noalloc(L, r, x, y_dtype)
            assert torch.equal(got, want), (name, T, y_dtype)


def test_noalloc_rejects_a_call_past_its_scratch():
    # 64 tokens, k = 32, H = 16384: T*(k+S)*(H+I)*4 bytes is far above 32 MiB
    spec = synth.LayerSpec(16384, 512, 64, 1, 32, sigmoid=True, renorm=True)
    L = coli.Layer.from_spec(spec, torch.zeros(16, dtype=torch.uint8, device="cuda"),
                             torch.zeros(16, dtype=torch.float16, device="cuda"))
    assert coli.coli_moe_workspace_bytes(L, 64, coli.COLI_ENTRY_DECODE) > 32 << 20
    r = coli.Route(L, 64)
    x = torch.zeros(64, spec.hidden, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(64, spec.hidden, dtype=torch.float32, device="cuda")
    with pytest.raises(coli.ColiError) as e:
        coli.coli_moe_forward_decode_noalloc(L, r, x, 64, y, coli.COLI_OUT_F32)
    assert e.value.status == -3
