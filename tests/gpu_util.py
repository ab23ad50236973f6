"""Helpers for the GPU parity tests: device layers, oracle on a token subset,
and the tolerance metric."""
from __future__ import annotations

import numpy as np
import torch

import int4_routed_expert_router_amd as coli
import oracle
import synth

# Layer outputs: fp32 accumulation against the fp64 oracle.  The bound is
# max_i |y_i - r_i| / max(|r_i|, rms of r's row), so values near zero are
# measured against the row's scale rather than against themselves.
REL_TOL = 2e-3
# relative rounding error of bf16 round-to-nearest-even
BF16_HALF_ULP = 2.0 ** -9


def gpu_layer(spec: synth.LayerSpec, seed=0, layer=0):
    q4, sc = synth.make_weights(spec, seed=seed, layer=layer, device="cuda")
    return coli.Layer.from_spec(spec, q4, sc)


def run_route(L: coli.Layer, logits: torch.Tensor, sel_bias=None) -> coli.Route:
    T = logits.shape[0]
    r = coli.Route(L, T)
    coli.coli_moe_route(L, logits, sel_bias, T, r)
    torch.cuda.synchronize()
    return r


def route_host(r: coli.Route, T: int, k: int):
    return {n: getattr(r, n).cpu().numpy() for n in (
        "topk_idx", "topk_w", "counts", "offsets", "pairs", "pair_pos", "union_ids", "n_union")}


def forward(L: coli.Layer, r: coli.Route, x: torch.Tensor, entry: str, y_dtype=coli.COLI_OUT_F32):
    T = x.shape[0]
    ent = coli.COLI_ENTRY_DECODE if entry == "decode" else coli.COLI_ENTRY_PREFILL
    ws = coli.workspace(L, T, ent)
    y = torch.empty(T, L.hidden, device="cuda",
                    dtype=torch.float32 if y_dtype == coli.COLI_OUT_F32 else torch.bfloat16)
    fn = coli.coli_moe_forward_decode if entry == "decode" else coli.coli_moe_forward_prefill
    fn(L, r, x, T, y, y_dtype, ws)
    torch.cuda.synchronize()
    return y


def oracle_layer(spec: synth.LayerSpec, L: coli.Layer, topk_idx: np.ndarray, topk_w: np.ndarray,
                 x: torch.Tensor, tokens, entry: str):
    """fp64 oracle output of the listed tokens, from host copies of only the
    experts those tokens use (renumbered), so full-size layers stay cheap."""
    tokens = list(tokens)
    idx = topk_idx.reshape(-1, spec.top_k)[tokens]
    w = topk_w.reshape(-1, spec.top_k)[tokens]
    used = sorted(set(int(e) for e in idx.ravel()))
    experts = used + ([spec.n_experts] if spec.n_shared else [])
    q4h, sch = synth.expert_slice(spec, L.q4, L.scales, experts)
    remap = np.zeros(spec.n_experts, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    xb = synth.bf16_bits(x)[tokens]
    fn = oracle.forward_decode if entry == "decode" else oracle.forward_prefill
    return fn(spec.hidden, spec.inter, len(used), spec.n_shared, spec.top_k, q4h, sch,
              remap[idx], w, xb, int8_weights=spec.int8)


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    denom = np.maximum(np.abs(ref), rms)
    denom = np.where(denom == 0, 1.0, denom)
    return float(np.max(np.abs(y - ref) / denom))


def bf16_ulp_distance(y_bf16: torch.Tensor, ref: np.ndarray) -> int:
    """Largest distance in bf16 units between y and bf16(ref) (ties-to-even)."""
    r = torch.from_numpy(np.asarray(ref, np.float64)).to(torch.float32).to(torch.bfloat16)
    a = y_bf16.cpu().view(torch.int16).to(torch.int32)
    b = r.view(torch.int16).to(torch.int32)
    # map sign-magnitude bit patterns onto a monotonic integer line
    a = torch.where(a < 0, -(a & 0x7FFF), a)
    b = torch.where(b < 0, -(b & 0x7FFF), b)
    return int((a - b).abs().max())
