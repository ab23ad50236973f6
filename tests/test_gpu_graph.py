"""HIP graph capture of the library's calls.  Route + decode (1, 4 and 16
tokens) and route + prefill are captured for two layers and two sets of
logits, then replayed several times with eager work and synchronisations
between the replays; every replay's output must equal the eager result bit
for bit (all kernels are deterministic).  The library issues no memset or
allocation, so every entry point can be captured."""
import pytest
import torch

import int4_routed_expert_router_amd as coli
import synth
from gpu_util import gpu_layer

pytestmark = pytest.mark.gpu


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # the first launches outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,T,entry", [
    ("glm", 1, "decode"), ("glm", 4, "decode"), ("a3b", 16, "decode"),
    ("olmoe", 64, "prefill"), ("a3b", 96, "prefill"),
])
def test_graph_replays_match_eager(name, T, entry):
    print("graph case: %s T=%d %s" % (name, T, entry), flush=True)
    w = synth.WORKLOADS[name]
    spec = w.spec
    layers = [gpu_layer(spec, layer=l) for l in range(2)]
    logits = [[synth.make_logits(spec, T, layer=l, zipf_alpha=w.zipf_alpha, step=r).cuda()
               for l in range(2)] for r in range(2)]
    x = [synth.make_x(spec, T, layer=l).cuda() for l in range(2)]
    route = coli.Route(layers[0], T)
    ent = coli.COLI_ENTRY_DECODE if entry == "decode" else coli.COLI_ENTRY_PREFILL
    fwd = coli.coli_moe_forward_decode if entry == "decode" else coli.coli_moe_forward_prefill
    ws = coli.workspace(layers[0], T, ent)
    y = [torch.empty(T, spec.hidden, dtype=torch.bfloat16, device="cuda") for _ in range(2)]

    def step(r):
        for l in range(2):
            coli.coli_moe_route(layers[l], logits[r][l], None, T, route)
            fwd(layers[l], route, x[l], T, y[l], coli.COLI_OUT_BF16, ws)

    ref = []
    for r in range(2):
        step(r)
        torch.cuda.synchronize()
        ref.append([t.clone() for t in y])
    assert not torch.equal(ref[0][0], ref[1][0])  # the two logit sets route differently
    graphs = [_capture(lambda r=r: step(r)) for r in range(2)]
    for i in range(6):
        r = i % 2
        for t in y:
            t.fill_(-1.0)  # eager work between replays
        if i == 3:
            step(1 - r)    # and a full eager step on the same buffers
        torch.cuda.synchronize()
        graphs[r].replay()
        torch.cuda.synchronize()
        for l in range(2):
            assert torch.equal(y[l], ref[r][l]), (i, l)
