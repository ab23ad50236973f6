"""Seeded synthetic inputs for the routed-expert MoE layer.

Shared by the tests, the smoke check and the benchmark; imported by both the
oracle side and the HIP side of the tests, so it holds none of the layer's
arithmetic: only random draws, their encoding as bf16 / fp16 / packed
nibbles, and the byte sizes of the int4 gs64 container.

Workload shapes.  The pages about the colibri engine name the model families
(OLMoE, a 35B-A3B Qwen, the GLM-5.2 744B MoE) but publish no weights or
router traces for this layer, so every input here is drawn from a seeded
generator with the shape of those layers:

* int4 weights uniform over [-8, 7] (uniform random bytes give uniform
  two's-complement nibbles), fp16 scales |N(0, 0.02)|;
* activations N(0, 1) rounded to bf16;
* router logits N(0, 1) fp32, plus an optional Zipf-like per-expert skew
  -alpha * s * ln(rank_e) with s = 1.1 and a seeded rank permutation, so a
  few experts are hot and many are cold.

Draws use torch generators on the requested device (CPU or a GPU).  The same
(seed, layer, kind) always gives the same values on one device kind; a test
hands the very same bytes to both the oracle and the HIP library, copying
them to the host where needed.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

ZIPF_S = 1.1
# alpha of the per-expert skew; at 2,048 tokens x top-8 over 256 experts with
# seed 0 it gives per-expert token counts of roughly 20 to 400.
ZIPF_ALPHA = 0.21

_KIND = {"q4": 1, "scales": 2, "logits": 3, "x": 4, "rank": 5, "bias": 6, "router": 7, "float_w": 8}


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """Shape and routing kind of one MoE layer (fields match the C struct)."""

    hidden: int
    inter: int
    n_experts: int
    n_shared: int
    top_k: int
    sigmoid: bool
    renorm: bool
    routed_scale: float = 1.0
    int8: bool = False   # one int8 byte per weight instead of a nibble
    mxfp4: bool = False  # E2M1 nibbles with one E8M0 scale byte per 32 weights
    mx_act: bool = False  # prefill activations in MXFP8 (MXFP4 layers; flag bit 1 << 16)

    @property
    def flags(self) -> int:
        return (1 if self.sigmoid else 0) | (256 if self.renorm else 0) | (
            1 << 16 if self.mx_act else 0)

    @property
    def weights(self) -> str:
        return "mxfp4" if self.mxfp4 else ("int8" if self.int8 else "int4")

    @property
    def n_total(self) -> int:
        return self.n_experts + self.n_shared

    @property
    def expert_bytes(self) -> int:
        """Code bytes of one expert: gate, up and down (3*I*H weights), a
        nibble or a byte each."""
        return 3 * self.inter * self.hidden // (1 if self.int8 else 2)

    @property
    def expert_scales(self) -> int:
        """Scales of one expert: one fp16 per 64 weights, or one E8M0 byte per
        32 weights (mxfp4)."""
        return 3 * self.inter * self.hidden // (32 if self.mxfp4 else 64)

    @property
    def scale_bytes(self) -> int:
        return 1 if self.mxfp4 else 2

    @property
    def expert_total_bytes(self) -> int:
        return self.expert_bytes + self.scale_bytes * self.expert_scales


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    spec: LayerSpec
    tokens: tuple
    zipf_alpha: float
    layers: int = 1
    description: str = ""


WORKLOADS = {
    "tiny": Workload(
        "tiny", LayerSpec(256, 128, 8, 0, 2, sigmoid=False, renorm=False), (4,), 0.0,
        description="H256 I128, 8 experts, top-2 softmax, 4 tokens"),
    "olmoe": Workload(
        "olmoe", LayerSpec(2048, 1024, 64, 0, 8, sigmoid=False, renorm=False), (1, 512), 0.0,
        description="OLMoE-like: H2048 I1024, 64 experts, top-8 softmax"),
    "a3b": Workload(
        "a3b", LayerSpec(2048, 512, 256, 1, 8, sigmoid=True, renorm=True), (1, 4, 16), ZIPF_ALPHA,
        description="35B-A3B-class: H2048 I512, 256 experts + 1 shared, top-8 sigmoid renorm, Zipf skew"),
    "glm": Workload(
        "glm", LayerSpec(6144, 2048, 256, 1, 8, sigmoid=True, renorm=True), (1, 4), ZIPF_ALPHA,
        layers=12,
        description="GLM-5.2-shaped decode stack: H6144 I2048, 256 experts + 1 shared, top-8 sigmoid renorm, 12 layers"),
    "glm_prefill": Workload(
        "glm_prefill", LayerSpec(6144, 2048, 256, 1, 8, sigmoid=True, renorm=True), (2048,), ZIPF_ALPHA,
        description="GLM-5.2-shaped prefill: one layer, 2048 tokens, Q8_0 activations"),
}


def _gen(device, seed: int, layer: int, kind: str, extra: int = 0) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    # a fixed mixing of the four integers into one 63-bit seed
    s = (seed * 1_000_003 + layer * 10_007 + _KIND[kind] * 101 + extra) & ((1 << 63) - 1)
    g.manual_seed(s)
    return g


def make_weights(spec: LayerSpec, seed: int = 0, layer: int = 0, device="cpu",
                 experts: int | None = None):
    """Container of one layer: (q4 uint8 [n*expert_bytes], scales fp16 [n*expert_scales]).

    `experts` defaults to E + S.  Uniform random bytes are uniform nibbles
    (or uniform int8 codes).  Scales are |N(0, 0.02)| for int4 codes and 16x
    smaller for int8 codes, so both give weights of the same size.
    """
    n = spec.n_total if experts is None else experts
    g = _gen(device, seed, layer, "q4")
    q4 = torch.randint(0, 256, (n * spec.expert_bytes,), dtype=torch.uint8,
                       generator=g, device=device)
    g = _gen(device, seed, layer, "scales")
    if spec.mxfp4:  # E8M0 exponents 118..122: 2^-9 .. 2^-5 (E2M1 codes reach 6)
        scales = torch.randint(118, 123, (n * spec.expert_scales,), dtype=torch.uint8,
                               generator=g, device=device)
        return q4, scales
    sc = torch.randn(n * spec.expert_scales, generator=g, device=device,
                     dtype=torch.float32)
    scales = (sc * (0.02 / 16 if spec.int8 else 0.02)).abs_().to(torch.float16)
    return q4, scales


def expert_rank(spec: LayerSpec, seed: int = 0, layer: int = 0) -> np.ndarray:
    """Seeded popularity rank (1 = hottest) of every routed expert."""
    g = _gen("cpu", seed, layer, "rank")
    return torch.randperm(spec.n_experts, generator=g).numpy() + 1


def make_logits(spec: LayerSpec, T: int, seed: int = 0, layer: int = 0,
                zipf_alpha: float = 0.0, device="cpu", step: int = 0) -> torch.Tensor:
    """Router logits fp32 [T, E]: N(0,1) plus the per-expert Zipf skew."""
    g = _gen(device, seed, layer, "logits", extra=step * 7919 + T)
    lg = torch.randn(T, spec.n_experts, generator=g, device=device, dtype=torch.float32)
    if zipf_alpha:
        rank = torch.from_numpy(expert_rank(spec, seed, layer)).to(torch.float64)
        bias = (-zipf_alpha * ZIPF_S * torch.log(rank)).to(torch.float32).to(device)
        lg = lg + bias[None, :]
    return lg


def make_x(spec: LayerSpec, T: int, seed: int = 0, layer: int = 0, device="cpu",
           step: int = 0) -> torch.Tensor:
    """Activations: N(0,1) rounded to bf16 (nearest-even), [T, H]."""
    g = _gen(device, seed, layer, "x", extra=step * 7919 + T)
    return torch.randn(T, spec.hidden, generator=g, device=device,
                       dtype=torch.float32).to(torch.bfloat16)


def make_router_weights(spec: LayerSpec, seed: int = 0, layer: int = 0, device="cpu"
                        ) -> torch.Tensor:
    """Router weights bf16 [E, H], N(0, 1/H): with N(0, 1) activations the
    logits come out about N(0, 1)."""
    g = _gen(device, seed, layer, "router")
    w = torch.randn(spec.n_experts, spec.hidden, generator=g, device=device,
                    dtype=torch.float32)
    return (w * spec.hidden ** -0.5).to(torch.bfloat16)


def make_float_weights(n: int, seed: int = 0, layer: int = 0, device="cpu",
                       dtype=torch.bfloat16) -> torch.Tensor:
    """n float weights before quantisation, flat (container order): N(0, 0.02^2)
    with one value in 1000 made 8x larger, so group maxima vary as in trained
    checkpoints."""
    g = _gen(device, seed, layer, "float_w")
    w = torch.randn(n, generator=g, device=device, dtype=torch.float32) * 0.02
    big = torch.rand(n, generator=g, device=device) < 1e-3
    w = torch.where(big, w * 8.0, w)
    return w.to(dtype)


def make_sel_bias(spec: LayerSpec, seed: int = 0, layer: int = 0) -> torch.Tensor:
    """A selection-only bias [E] fp32 (N(0, 0.5)), for tests of that input."""
    g = _gen("cpu", seed, layer, "bias")
    return torch.randn(spec.n_experts, generator=g, dtype=torch.float32) * 0.5


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def f16_bits(t: torch.Tensor) -> np.ndarray:
    """fp16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def expert_slice(spec: LayerSpec, q4: torch.Tensor, scales: torch.Tensor, experts):
    """Host copies (uint8, uint16) of the listed experts, renumbered 0..len-1."""
    eb, es = spec.expert_bytes, spec.expert_scales
    qs = [q4[e * eb:(e + 1) * eb].cpu() for e in experts]
    ss = [scales[e * es:(e + 1) * es].cpu() for e in experts]
    sc = torch.cat(ss)
    return (torch.cat(qs).numpy(), sc.numpy() if spec.mxfp4 else f16_bits(sc))


def container_gib(spec: LayerSpec, layers: int = 1) -> float:
    return layers * spec.n_total * spec.expert_total_bytes / 2**30


def zipf_bias_float(spec: LayerSpec, seed=0, layer=0, alpha=ZIPF_ALPHA) -> np.ndarray:
    rank = expert_rank(spec, seed, layer).astype(np.float64)
    return (-alpha * ZIPF_S * np.log(rank)).astype(np.float32)


__all__ = [
    "LayerSpec", "Workload", "WORKLOADS", "ZIPF_ALPHA", "ZIPF_S", "make_weights",
    "make_logits", "make_x", "make_sel_bias", "expert_rank", "bf16_bits", "f16_bits",
    "expert_slice", "container_gib", "zipf_bias_float",
]
