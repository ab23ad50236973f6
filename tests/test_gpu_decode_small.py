"""GPU parity of the small-layer decode (H 2048 with I 512 or 1024), where
gate/up as well as down run on the matrix cores, at every batch shape it
has: one token, slots holding one token and slots holding up to 16 (few
experts, so each is chosen by most of the batch), the int4, int8 and MXFP4
codecs -- against the fp64 oracle, and bit for bit against the same tokens
decoded one at a time (a token's result may not depend on its batch)."""
import dataclasses

import pytest
import torch

import synth
import test_gpu_decode as dec
import test_gpu_int8_decode as dec8
import test_gpu_mxfp4 as decf4
from gpu_util import forward, gpu_layer, run_route

pytestmark = pytest.mark.gpu

# few experts: every slot holds several tokens, the shared slot all T
FEW = synth.LayerSpec(2048, 512, 4, 1, 2, sigmoid=True, renorm=True)
# many experts: most slots hold one token
MANY = synth.LayerSpec(2048, 1024, 64, 0, 4, sigmoid=False, renorm=True)


def _spec(spec, fmt):
    return dataclasses.replace(spec, int8=fmt == "int8", mxfp4=fmt == "mxfp4")


def _parity(spec, fmt, T, seed):
    if fmt == "int4":
        dec._decode_case(spec, T, seed=seed, zipf=0.5)
    elif fmt == "int8":
        dec8._case(spec, T, seed=seed, zipf=0.5)
    else:
        decf4._decode(spec, T, seed=seed, zipf=0.5)


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4"])
@pytest.mark.parametrize("which,T", [("few", 1), ("few", 3), ("few", 16), ("many", 1), ("many", 11)])
def test_small_layer_parity(fmt, which, T):
    spec = _spec(FEW if which == "few" else MANY, fmt)
    print("small-layer parity: %s %s T=%d" % (fmt, which, T), flush=True)
    _parity(spec, fmt, T, seed=21)


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4"])
@pytest.mark.parametrize("which,T", [("few", 16), ("many", 9)])
def test_small_layer_batch_invariant(fmt, which, T):
    spec = _spec(FEW if which == "few" else MANY, fmt)
    print("small-layer batch invariance: %s %s T=%d" % (fmt, which, T), flush=True)
    L = gpu_layer(spec, seed=23)
    lg = synth.make_logits(spec, T, seed=23, zipf_alpha=0.5).cuda()
    x = synth.make_x(spec, T, seed=23).cuda()
    y = forward(L, run_route(L, lg), x, "decode")
    assert torch.equal(forward(L, run_route(L, lg), x, "decode"), y)
    for t in range(T):
        yt = forward(L, run_route(L, lg[t:t + 1].contiguous()), x[t:t + 1].contiguous(), "decode")
        assert torch.equal(yt[0], y[t]), "%s token %d of %d depends on its batch" % (fmt, t, T)


# every batch size of the one-launch multi-token decode: each workgroup runs
# its slot's one-token or general code, and a token's result matches the
# same token decoded alone
A3B = synth.WORKLOADS["a3b"].spec
LARGE_I = synth.LayerSpec(2048, 2048, 6, 1, 3, sigmoid=True, renorm=True)


@pytest.mark.parametrize("fmt", ["int4", "int8", "mxfp4"])
@pytest.mark.parametrize("which", ["a3b", "large_i"])
def test_batch_invariant_every_T(fmt, which):
    spec = _spec(A3B if which == "a3b" else LARGE_I, fmt)
    print("batch invariance at T = 2..16: %s %s" % (fmt, which), flush=True)
    L = gpu_layer(spec, seed=31)
    lg = synth.make_logits(spec, 16, seed=31, zipf_alpha=synth.ZIPF_ALPHA).cuda()
    x = synth.make_x(spec, 16, seed=31).cuda()
    alone = [forward(L, run_route(L, lg[t:t + 1].contiguous()), x[t:t + 1].contiguous(),
                     "decode")[0] for t in range(16)]
    for T in range(2, 17):
        y = forward(L, run_route(L, lg[:T].contiguous()), x[:T].contiguous(), "decode")
        for t in range(T):
            assert torch.equal(y[t], alone[t]), "%s %s: token %d of %d" % (fmt, which, t, T)
