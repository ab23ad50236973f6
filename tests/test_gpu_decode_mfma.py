"""GPU parity of the decode down GEMV on the matrix cores (I = 2048) at every
batch shape it has: one token, 2..8 tokens (one operand tile), 9..16 tokens
(two tiles), slots holding many tokens (few experts, so each is chosen by
most of the batch), H of one and two gate/up chunks per lane, and the int4,
int8 and MXFP4 codecs -- against the fp64 oracle, and bit for bit against
the same tokens decoded one at a time (a token's result may not depend on
its batch)."""
import dataclasses

import pytest
import torch

import int4_routed_expert_router_amd as coli
import synth
import test_gpu_decode as dec
import test_gpu_int8_decode as dec8
import test_gpu_mxfp4 as decf4
from gpu_util import forward, gpu_layer, run_route

pytestmark = pytest.mark.gpu

# few experts: every slot holds several tokens, the shared slot all T
SMALL = synth.LayerSpec(2048, 2048, 4, 1, 2, sigmoid=True, renorm=True)
WIDE = synth.LayerSpec(4096, 2048, 6, 1, 3, sigmoid=False, renorm=True)


@pytest.mark.parametrize("spec,T", [(SMALL, 2), (SMALL, 8), (SMALL, 9), (SMALL, 16), (WIDE, 12)])
def test_int4_parity(spec, T):
    dec._decode_case(spec, T, seed=3, zipf=0.5)


@pytest.mark.parametrize("spec,T", [(SMALL, 9), (SMALL, 16), (WIDE, 5)])
def test_int8_parity(spec, T):
    dec8._case(dataclasses.replace(spec, int8=True), T, seed=5, zipf=0.5)


@pytest.mark.parametrize("spec,T", [(SMALL, 11), (SMALL, 16), (WIDE, 3)])
def test_mxfp4_parity(spec, T):
    decf4._decode(dataclasses.replace(spec, mxfp4=True), T, seed=6, zipf=0.5)


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4"])
@pytest.mark.parametrize("T", [5, 16])
def test_batch_invariant(fmt, T):
    spec = dataclasses.replace(SMALL, int8=fmt == "int8", mxfp4=fmt == "mxfp4")
    print("batch invariance: %s T=%d" % (fmt, T), flush=True)
    L = gpu_layer(spec, seed=9)
    lg = synth.make_logits(spec, T, seed=9, zipf_alpha=0.5).cuda()
    x = synth.make_x(spec, T, seed=9).cuda()
    y = forward(L, run_route(L, lg), x, "decode")
    for t in range(T):
        yt = forward(L, run_route(L, lg[t:t + 1].contiguous()), x[t:t + 1].contiguous(), "decode")
        assert torch.equal(yt[0], y[t]), "%s token %d of %d depends on its batch" % (fmt, t, T)


# 17..64 tokens: the vector decode kernels, at the same width (int4; the
# int8 and MXFP4 containers decode at most 16 tokens)
@pytest.mark.parametrize("T", [17, 40, 64])
def test_large_batch_parity(T):
    dec._decode_case(SMALL, T, seed=11, zipf=0.5)


def test_large_batch_invariant():
    """Among batches of 17..64 tokens a token's result does not depend on the
    rest of the batch: the first 17 tokens of a 40-token batch, alone."""
    L = gpu_layer(SMALL, seed=13)
    lg = synth.make_logits(SMALL, 40, seed=13, zipf_alpha=0.5).cuda()
    x = synth.make_x(SMALL, 40, seed=13).cuda()
    y40 = forward(L, run_route(L, lg), x, "decode")
    y17 = forward(L, run_route(L, lg[:17].contiguous()), x[:17].contiguous(), "decode")
    assert torch.equal(y17, y40[:17])


@pytest.mark.parametrize("fmt", ["int8", "mxfp4"])
def test_large_batch_int8_mxfp4(fmt):
    """17 tokens on the matrix-core shape run the general kernels with the
    int8 or MXFP4 codec."""
    dec._decode_case(dataclasses.replace(SMALL, int8=fmt == "int8", mxfp4=fmt == "mxfp4"), 17,
                     seed=1, zipf=0.5)
