"""Dense numpy brute force of the MoE layer, used to pin the oracle.

Written independently of the C oracle: it unpacks every expert of the
container to dense fp64 matrices with vectorised numpy, runs every expert on
every token with plain matrix products, and combines them with a dense
[T, E] routing-weight matrix that is zero for unselected experts.  Top-k uses
numpy's lexsort and grouping uses a stable argsort.  Small shapes only.
"""
from __future__ import annotations

import numpy as np


def unpack_nibbles(rows_bytes: np.ndarray) -> np.ndarray:
    """[rows, K/2] uint8 -> [rows, K] int8: even k = low nibble, odd k = high."""
    b = rows_bytes.astype(np.int16)
    lo = b & 15
    hi = b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((b.shape[0], b.shape[1] * 2), np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# FP4 E2M1 magnitudes of codes 0..7 as tabulated in the OCP microscaling
# formats specification; bit 3 of a code is its sign.
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def codes(qb: np.ndarray, rows: int, K: int, weights: str) -> np.ndarray:
    """[rows, K] integer codes of one matrix's bytes (mxfp4: twice the E2M1
    value, an integer)."""
    if weights == "int8":
        return np.asarray(qb, np.uint8).view(np.int8).reshape(rows, K)
    b = np.asarray(qb, np.uint8).reshape(rows, K // 2)
    if weights == "mxfp4":
        nib = np.empty((rows, K), np.uint8)
        nib[:, 0::2], nib[:, 1::2] = b & 15, b >> 4
        v = E2M1[nib & 7] * np.where(nib & 8, -2.0, 2.0)
        return v.astype(np.int8)
    return unpack_nibbles(b)


def scale_matrix(sb: np.ndarray, rows: int, K: int, weights: str) -> np.ndarray:
    """[rows, K] fp64 scale of every weight (mxfp4: halved, for the doubled codes)."""
    if weights == "mxfp4":
        e = np.asarray(sb, np.uint8).reshape(rows, K // 32).astype(np.float64)
        return np.repeat(np.exp2(e - 128.0), 32, axis=1)
    s = np.asarray(sb, np.uint16).view(np.float16).astype(np.float64).reshape(rows, K // 64)
    return np.repeat(s, 64, axis=1)


def dense_experts(H, I, n, q4, scales, weights="int4"):
    """Dequantised fp64 (Wg [I,H], Wu [I,H], Wd [H,I]) for experts 0..n-1."""
    q4 = np.asarray(q4, np.uint8)
    sc = np.asarray(scales, np.uint8 if weights == "mxfp4" else np.uint16)
    mb = I * H if weights == "int8" else I * H // 2
    ms = I * H // (32 if weights == "mxfp4" else 64)
    eb, es = 3 * mb, 3 * ms
    out = []
    for e in range(n):
        qe, se = q4[e * eb:(e + 1) * eb], sc[e * es:(e + 1) * es]
        mats = []
        for m, (rows, K) in enumerate(((I, H), (I, H), (H, I))):
            qm = codes(qe[m * mb:(m + 1) * mb], rows, K, weights)
            sm = scale_matrix(se[m * ms:(m + 1) * ms], rows, K, weights)
            mats.append(qm.astype(np.float64) * sm)
        out.append(tuple(mats))
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def topk(logits, k, sel_bias=None):
    score = np.asarray(logits, np.float32)
    if sel_bias is not None:
        score = (score + np.asarray(sel_bias, np.float32)[None, :]).astype(np.float32)
    T, E = score.shape
    idx = np.empty((T, k), np.int32)
    for t in range(T):
        order = np.lexsort((np.arange(E), -score[t].astype(np.float64)))
        idx[t] = order[:k]
    return idx


def route_weights(logits, idx, sigmoid, renorm, routed_scale=1.0):
    l = np.asarray(logits, np.float64)
    if sigmoid:
        w = 1.0 / (1.0 + np.exp(-np.take_along_axis(l, idx, axis=1)))
    else:
        z = l - l.max(axis=1, keepdims=True)
        p = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, idx, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w * routed_scale


def group(idx, E):
    flat = np.asarray(idx).reshape(-1)
    pairs = np.argsort(flat, kind="stable").astype(np.int32)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return counts, offsets, pairs


def silu(g):
    return g / (1.0 + np.exp(-g))


def decode_layer(H, I, E, S, q4, scales, topk_idx, topk_w, x_bits, weights="int4"):
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    experts = dense_experts(H, I, E + S, q4, scales, weights)
    wmat = np.zeros((T, E + S))
    for t in range(T):
        for j in range(topk_idx.shape[1]):
            wmat[t, topk_idx[t, j]] += float(np.float32(topk_w[t, j]))
    if S:
        wmat[:, E] = 1.0
    y = np.zeros((T, H))
    for e, (wg, wu, wd) in enumerate(experts):
        o = (silu(x @ wg.T) * (x @ wu.T)) @ wd.T
        y += wmat[:, e:e + 1] * o
    return y


def q8_0(v):
    """Q8_0 per 32 values: (int8 q, fp16 d) with half-away-from-zero rounding."""
    v = np.asarray(v, np.float32).reshape(-1, 32)
    a = np.abs(v).max(axis=1)
    d = (a / np.float32(127.0)).astype(np.float32)
    safe = np.where(a == 0, np.float32(1.0), d).astype(np.float32)
    r = (v / safe[:, None]).astype(np.float32).astype(np.float64)
    q = np.sign(r) * np.floor(np.abs(r) + 0.5)
    q = np.clip(q, -127, 127)
    q[a == 0] = 0
    return q.astype(np.int8).reshape(-1), d.astype(np.float16)


def prefill_layer(H, I, E, S, q4, scales, topk_idx, topk_w, x_bits, weights="int4"):
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    T = x32.shape[0]
    qx, dx = q8_0(x32)
    xh = qx.reshape(T, H // 32, 32).astype(np.float64) * dx.astype(np.float64).reshape(T, H // 32, 1)
    xh = xh.reshape(T, H)
    experts = dense_experts(H, I, E + S, q4, scales, weights)
    wmat = np.zeros((T, E + S))
    for t in range(T):
        for j in range(topk_idx.shape[1]):
            wmat[t, topk_idx[t, j]] += float(np.float32(topk_w[t, j]))
    if S:
        wmat[:, E] = 1.0
    y = np.zeros((T, H))
    for e, (wg, wu, wd) in enumerate(experts):
        h = (silu(xh @ wg.T) * (xh @ wu.T)).astype(np.float32)
        qh, dh = q8_0(h)
        hh = (qh.reshape(T, I // 32, 32).astype(np.float64)
              * dh.astype(np.float64).reshape(T, I // 32, 1)).reshape(T, I)
        y += wmat[:, e:e + 1] * (hh @ wd.T)
    return y


def block_dots(H, I, q4, expert, matrix, q_act, weights="int4"):
    mb = I * H if weights == "int8" else I * H // 2
    eb = 3 * mb
    rows, K = ((I, H), (I, H), (H, I))[matrix]
    qb = np.asarray(q4, np.uint8)[expert * eb + matrix * mb:expert * eb + (matrix + 1) * mb]
    w = codes(qb, rows, K, weights).astype(np.int64)
    a = np.asarray(q_act, np.int8).reshape(-1, K).astype(np.int64)
    T = a.shape[0]
    prod = w[None, :, :] * a[:, None, :]
    return prod.reshape(T, rows, K // 32, 32).sum(axis=3).astype(np.int32)


# ------------------------------------------------------------ MX activations

def e4m3_table() -> np.ndarray:
    """Magnitudes of FP8 E4M3 codes 0..126 (OCP 8-bit floating point) from
    their integer significands: code (e, m) is (8 + m) * 2^(e - 10) for e > 0
    and m * 2^-9 for e = 0.  Code 127 (NaN) is left out."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e > 0, (8 + m) * np.exp2(e - 10.0), m * 2.0 ** -9)


def mxfp8(v):
    """MXFP8 E4M3 per 32 values -> (uint8 codes, uint8 E8M0).  Shared exponent
    from the fp32 bit pattern of the block maximum (floor(log2) - 8, biased
    by 127, clamped to [0, 254], 0 for an all-zero block); each element the
    nearest table magnitude of v / 2^(E-127), ties to the even code, and
    nothing above 448 (the table's last entry); sign from the sign bit."""
    v = np.asarray(v, np.float32).reshape(-1, 32)
    a = np.max(np.abs(v), axis=1)
    expf = ((a.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    floor_log2 = np.where(expf > 0, expf - 127, -150)  # fp32 subnormal maxima clamp to E = 0
    E = np.where(a > 0, np.clip(floor_log2 - 8 + 127, 0, 254), 0).astype(np.int64)
    m = np.abs(v.astype(np.float64) * np.exp2(127.0 - E)[:, None])
    tab = e4m3_table()
    dist = np.abs(m[..., None] - tab)
    cand = dist == dist.min(axis=-1, keepdims=True)
    even = cand & (np.arange(127) % 2 == 0)
    idx = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    code = idx | np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8).reshape(-1), E.astype(np.uint8)


def mxfp8_values(codes, e8) -> np.ndarray:
    """fp64 values of MXFP8 codes [..., K] with E8M0 [..., K/32]."""
    codes = np.asarray(codes, np.uint8)
    mag = e4m3_table()[np.minimum(codes & 0x7F, 126)]
    val = np.where(codes & 0x80, -mag, mag)
    sc = np.repeat(np.exp2(np.asarray(e8, np.float64) - 127.0), 32, axis=-1)
    return val * sc


def prefill_layer_mx(H, I, E, S, q4, scales, topk_idx, topk_w, x_bits):
    """MX-path layer of an MXFP4 container: MXFP8(x), dense experts, fp32 h,
    MXFP8(h), down, routing-weighted combine."""
    x32 = bf16_to_f64(x_bits).astype(np.float32)
    T = x32.shape[0]
    qx, ex = mxfp8(x32)
    xh = mxfp8_values(qx.reshape(T, H), ex.reshape(T, H // 32))
    experts = dense_experts(H, I, E + S, q4, scales, "mxfp4")
    wmat = np.zeros((T, E + S))
    for t in range(T):
        for j in range(topk_idx.shape[1]):
            wmat[t, topk_idx[t, j]] += float(np.float32(topk_w[t, j]))
    if S:
        wmat[:, E] = 1.0
    y = np.zeros((T, H))
    for e, (wg, wu, wd) in enumerate(experts):
        h = (silu(xh @ wg.T) * (xh @ wu.T)).astype(np.float32)
        qh, eh = mxfp8(h)
        hh = mxfp8_values(qh.reshape(T, I), eh.reshape(T, I // 32))
        y += wmat[:, e:e + 1] * (hh @ wd.T)
    return y
