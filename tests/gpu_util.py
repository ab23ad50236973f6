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


def checked_route(spec: synth.LayerSpec, r: coli.Route, logits: torch.Tensor, sel_bias=None):
    """The oracle's route of the same logits, after checking the device route
    against it: top-k indices, counts, offsets and pair lists bit for bit,
    routing weights within 3e-6 relative.  End-to-end comparisons feed the
    oracle's own routing to the oracle layer, so a device routing mistake
    cannot hide behind both sides using the same wrong experts."""
    T = logits.shape[0]
    k = spec.top_k
    g = route_host(r, T, k)
    sb = None if sel_bias is None else sel_bias.float().cpu().numpy()
    o = oracle.route(logits.float().cpu().numpy(), k, spec.flags, spec.routed_scale, sel_bias=sb)
    assert np.array_equal(g["topk_idx"].reshape(T, k), o["topk_idx"]), "device top-k differs"
    assert np.array_equal(g["counts"], o["counts"]), "device counts differ"
    assert np.array_equal(g["offsets"], o["offsets"]), "device offsets differ"
    assert np.array_equal(g["pairs"], o["pairs"]), "device pair lists differ"
    np.testing.assert_allclose(g["topk_w"].reshape(T, k), o["topk_w"], rtol=3e-6, atol=1e-7)
    return o


def cover_tokens(g, T: int, k: int, tile: int = 64, hottest: int = 0, shared: bool = True):
    """Tokens that touch every (expert, token tile) work item of a batched
    union: for each expert, the first and the last row of each run of `tile`
    rows of its token list (so every partial last tile's last row too), the
    shared expert's tile boundaries (tokens 0, tile-1, tile, ...), and every
    token of the `hottest` most-loaded experts.  g is a route dict
    (counts, offsets, pairs)."""
    counts, offsets, pairs = g["counts"], g["offsets"], np.asarray(g["pairs"]).ravel()
    toks = set()
    for e in range(len(counts)):
        n = int(counts[e])
        for pos in range(n):
            if pos % tile in (0, tile - 1) or pos == n - 1:
                toks.add(int(pairs[offsets[e] + pos]) // k)
    if shared:
        toks.update(t for t in range(T) if t % tile in (0, tile - 1) or t == T - 1)
    for e in np.argsort(-np.asarray(counts), kind="stable")[:hottest]:
        toks.update(int(p) // k for p in pairs[offsets[e]:offsets[e + 1]])
    return sorted(toks)


def sample_tokens(g, T: int, k: int, tile: int = 64, hottest: int = 2, every: int = 16):
    """A bounded sample for batches too large to compare every tile: for each
    expert, the first row of its first tile and the last row of its last
    tile; for the `hottest` most-loaded experts, the first and last row of
    every tile; the shared expert's first and last token and the first row
    of every `every`-th tile."""
    counts, offsets, pairs = g["counts"], g["offsets"], np.asarray(g["pairs"]).ravel()
    toks = set()
    for e in range(len(counts)):
        n = int(counts[e])
        if n:
            toks.add(int(pairs[offsets[e]]) // k)
            toks.add(int(pairs[offsets[e] + n - 1]) // k)
    for e in np.argsort(-np.asarray(counts), kind="stable")[:hottest]:
        n = int(counts[e])
        for pos in range(n):
            if pos % tile in (0, tile - 1) or pos == n - 1:
                toks.add(int(pairs[offsets[e] + pos]) // k)
    toks.update(range(0, T, tile * every))
    toks.add(T - 1)
    return sorted(toks)


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
              remap[idx], w, xb, weights=spec.weights)


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


def prefill_flip_budget(spec: synth.LayerSpec, L: coli.Layer, topk_idx: np.ndarray,
                        topk_w: np.ndarray, x: torch.Tensor, tokens, band=1e-5):
    """Oracle prefill output of `tokens` and, per output element, the most that
    Q8_0 decisions of h sitting on a rounding boundary can move it.

    The integer path quantises h (fp32) to Q8_0 on both sides; the GPU's h
    differs from the oracle's by fp32 rounding-order ulps, so a code whose
    h / d lies within `band` (absolute, in code units, plus 2^-19 relative,
    about 16 ulps) of a .5 boundary may round the other way, and a block
    whose fp32 scale lies within 2^-19 of an fp16 tie may store the
    neighbouring fp16 scale.  A
    code change of 1 moves down output m by at most d * |W_down[m, n]|; a
    scale change by one fp16 step moves it by at most 2^-10 * |q d W[m, n]|
    summed over the block.  Returns (ref [len(tokens), H], budget [same]).
    """
    tokens = list(tokens)
    H, I, k, S = spec.hidden, spec.inter, spec.top_k, spec.n_shared
    idx = topk_idx.reshape(-1, k)[tokens]
    w = topk_w.reshape(-1, k)[tokens]
    used = sorted(set(int(e) for e in idx.ravel()))
    experts = used + ([spec.n_experts] if S else [])
    q4h, sch = synth.expert_slice(spec, L.q4, L.scales, experts)
    remap = np.zeros(spec.n_experts, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    xb = synth.bf16_bits(x)[tokens]
    ref, h = oracle.forward_prefill(H, I, len(used), S, k, q4h, sch, remap[idx], w, xb,
                                    want_h=True, weights=spec.weights)
    mb = I * H if spec.int8 else I * H // 2
    ms = I * H // (32 if spec.mxfp4 else 64)      # scale elements per matrix
    eb, es = 3 * mb, 3 * ms
    scf = (np.exp2(sch.astype(np.float64) - 128.0) if spec.mxfp4       # halved: codes are 2v
           else sch.view(np.float16).astype(np.float64))
    budget = np.zeros((len(tokens), H))
    for ti in range(len(tokens)):
        for j in range(k + S):
            le = int(remap[idx[ti, j]]) if j < k else len(used)
            wj = float(np.float32(w[ti, j])) if j < k else 1.0
            hv = h[ti, j].astype(np.float32).reshape(I // 32, 32)
            amax = np.abs(hv).max(axis=1)
            d32 = (amax / np.float32(127.0)).astype(np.float32)
            safe = np.where(d32 == 0, np.float32(1.0), d32)
            ratio = np.abs((hv / safe[:, None]).astype(np.float32)).astype(np.float64)
            frac = ratio - np.floor(ratio)
            code_risk = np.abs(frac - 0.5) < band + 2.0 ** -19 * ratio
            d16 = d32.astype(np.float16).astype(np.float64)
            up = np.nextafter(d32.astype(np.float16), np.float16(np.inf)).astype(np.float64)
            dn = np.nextafter(d32.astype(np.float16), np.float16(0)).astype(np.float64)
            nb = np.where(d32 >= d16, up, dn)
            scale_risk = np.abs(d32 - (d16 + nb) / 2) < 2.0 ** -19 * d32
            # per column n: the most a decision there moves o[m] / |W_down[m, n]|
            q = np.floor(ratio + 0.5)
            col = (code_risk * d16[:, None]
                   + scale_risk[:, None] * 2.0 ** -10 * q * d16[:, None]).reshape(I)
            cols = np.flatnonzero(col)
            if cols.size == 0:
                continue
            base = le * eb + 2 * mb
            if spec.int8:
                rows = np.asarray(q4h[base:base + mb], np.uint8).view(np.int8).reshape(H, I)
                wq = rows[:, cols].astype(np.float64)
            else:
                b = np.asarray(q4h[base:base + mb], np.uint8).reshape(H, I // 2)[:, cols // 2]
                nib = np.where(cols % 2 == 1, b >> 4, b & 15).astype(np.int64)
                if spec.mxfp4:
                    from bruteforce import E2M1
                    wq = 2.0 * E2M1[nib & 7]
                else:
                    wq = np.where(nib >= 8, nib - 16, nib).astype(np.float64)
            gsz = 32 if spec.mxfp4 else 64
            s = scf[le * es + 2 * ms:le * es + 3 * ms].reshape(H, I // gsz)
            wabs = np.abs(wq) * s[:, cols // gsz]
            budget[ti] += wj * (wabs @ col[cols])
    return ref, budget


def check_prefill_output(spec, L, g, x, y, tokens, tol=REL_TOL):
    """|y - ref| <= tol * max(|ref|, rms of ref's row) + the Q8_0 boundary
    budget of prefill_flip_budget, element by element.  Returns the plain
    metric and the number of elements that needed budget."""
    tokens = list(tokens)
    ref, budget = prefill_flip_budget(spec, L, g["topk_idx"], g["topk_w"], x, tokens)
    yv = y.float().cpu().numpy()[tokens].astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    denom = np.maximum(np.abs(ref), rms)
    err = np.abs(yv - ref)
    over = (err - budget) / denom
    worst = np.unravel_index(int(np.argmax(over)), over.shape)
    print("  worst element: token %d, column %d: |err| / scale %.3g, budget / scale %.3g"
          % (tokens[worst[0]], worst[1], err[worst] / denom[worst], budget[worst] / denom[worst]),
          flush=True)
    assert np.all(err <= tol * denom + budget), float(np.max(over))
    return rel_err(yv, ref), int(np.count_nonzero(err > tol * denom))


def mx_flip_budget(spec: synth.LayerSpec, L: coli.Layer, topk_idx: np.ndarray,
                   topk_w: np.ndarray, x: torch.Tensor, tokens, band=2.0 ** -12):
    """Oracle MX-path output of `tokens` and, per output element, the most
    that MXFP8 decisions of h sitting on a boundary can move it.

    Both sides quantise h (fp32) to MXFP8; the GPU's h differs from the
    oracle's by the MX instruction's own rounding (up to ~2^-14 of a
    block's largest terms when its E4M3 values span a wide range, measured)
    and the SwiGLU's exp, so an E4M3 code whose scaled value lies within `band`
    (relative) of a rounding midpoint may round the other way (one code step
    of that binade), and a block whose maximum lies within `band` of a power
    of two may take the neighbouring shared exponent (every element then
    moves by at most two code steps of its own magnitude).  A change of dh in
    h[n] moves down output m by at most |dh| * |W_down[m, n]|.  Returns
    (ref [len(tokens), H], budget [same])."""
    from bruteforce import E2M1, e4m3_table
    tokens = list(tokens)
    H, I, k, S = spec.hidden, spec.inter, spec.top_k, spec.n_shared
    idx = topk_idx.reshape(-1, k)[tokens]
    w = topk_w.reshape(-1, k)[tokens]
    used = sorted(set(int(e) for e in idx.ravel()))
    experts = used + ([spec.n_experts] if S else [])
    q4h, sch = synth.expert_slice(spec, L.q4, L.scales, experts)
    remap = np.zeros(spec.n_experts, np.int32)
    remap[used] = np.arange(len(used), dtype=np.int32)
    xb = synth.bf16_bits(x)[tokens]
    ref, h = oracle.forward_prefill_mx(H, I, len(used), S, k, q4h, sch, remap[idx], w, xb,
                                       want_h=True)
    tab = e4m3_table()
    mids = 0.5 * (tab[:-1] + tab[1:])
    mb, ms = I * H // 2, I * H // 32
    eb, es = 3 * mb, 3 * ms
    budget = np.zeros((len(tokens), H))
    for ti in range(len(tokens)):
        for j in range(k + S):
            le = int(remap[idx[ti, j]]) if j < k else len(used)
            wj = float(np.float32(w[ti, j])) if j < k else 1.0
            hv = h[ti, j].astype(np.float64).reshape(I // 32, 32)
            amax = np.abs(hv).max(axis=1)
            with np.errstate(divide="ignore"):
                fl = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))), 0.0)
            X = np.clip(fl - 8 + 127, 0, 254) - 127
            m = np.abs(hv) * np.exp2(-X)[:, None]
            near = np.min(np.abs(m[..., None] - mids), axis=-1)
            with np.errstate(divide="ignore"):
                e = np.floor(np.log2(np.where(m > 0, m, 1.0)))
            step = np.where(m < 2.0 ** -6, 2.0 ** -9, np.exp2(e - 3)) * np.exp2(X)[:, None]
            # the instruction's error follows the magnitude of a dot's terms, not its
            # result: a floor of 2^-4 of the band at the block's largest value
            code_risk = (near < band * np.maximum(m, 2.0 ** -4 * m.max(axis=1, keepdims=True))) & (
                m < 448.0)
            pow2 = np.exp2(fl)
            exp_risk = (amax > 0) & ((np.abs(amax - pow2) < band * amax)
                                     | (np.abs(amax - 2 * pow2) < band * amax))
            col = (code_risk * step + exp_risk[:, None] * 2.0 * step).reshape(I)
            cols = np.flatnonzero(col)
            if cols.size == 0:
                continue
            base = le * eb + 2 * mb
            b = np.asarray(q4h[base:base + mb], np.uint8).reshape(H, I // 2)[:, cols // 2]
            nib = np.where(cols % 2 == 1, b >> 4, b & 15).astype(np.int64)
            sc = np.asarray(sch[le * es + 2 * ms:le * es + 3 * ms], np.uint8).reshape(H, I // 32)
            wabs = E2M1[nib & 7] * np.exp2(sc[:, cols // 32].astype(np.float64) - 127.0)
            budget[ti] += wj * (wabs @ col[cols])
    return ref, budget


def check_prefill_output_mx(spec, L, g, x, y, tokens, tol=REL_TOL):
    """check_prefill_output for the MX path (mx_flip_budget)."""
    tokens = list(tokens)
    ref, budget = mx_flip_budget(spec, L, g["topk_idx"], g["topk_w"], x, tokens)
    yv = y.float().cpu().numpy()[tokens].astype(np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=1, keepdims=True))
    denom = np.maximum(np.abs(ref), rms)
    err = np.abs(yv - ref)
    over = (err - budget) / denom
    worst = np.unravel_index(int(np.argmax(over)), over.shape)
    print("  worst element: token %d, column %d: |err| / scale %.3g, budget / scale %.3g"
          % (tokens[worst[0]], worst[1], err[worst] / denom[worst], budget[worst] / denom[worst]),
          flush=True)
    assert np.all(err <= tol * denom + budget), float(np.max(over))
    return rel_err(yv, ref), int(np.count_nonzero(err > tol * denom))
