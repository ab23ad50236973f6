"""CPU oracle of the routed-expert MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package.  It wraps the plain C oracle (coli_oracle.c: loops, fp64
accumulation, no shared code with the HIP library) with ctypes and numpy.

`build()` compiles liboracle.so next to the source with gcc; the wrappers
build it on first use if it is missing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coli_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle (gcc, -O2, OpenMP, no FP contraction, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path):
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i32, i64, u32, f32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float
    lib.oracle_route.argtypes = [i32, i32, i32, u32, f32, p, p, p, p, p, p, p]
    lib.oracle_forward_decode.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, i64, p, i32]
    lib.oracle_forward_prefill.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, i64, p, p,
                                           i32]
    lib.oracle_quantize_q8_0.argtypes = [p, i64, p, p]
    lib.oracle_block_dots.argtypes = [i64, i64, i64, i64, p, p, i64, ctypes.c_int, p, i64, p,
                                      i32]
    lib.oracle_router_logits.argtypes = [i64, i64, i64, p, p, p]
    lib.oracle_quantize_int4_gs64.argtypes = [p, i64, i64, p, p]
    lib.oracle_quantize_int8_gs64.argtypes = [p, i64, i64, p, p]
    lib.oracle_quantize_mxfp4.argtypes = [p, i64, i64, p, p]
    lib.oracle_quantize_mxfp8.argtypes = [p, i64, p, p]
    lib.oracle_mx_dots.argtypes = [i64, i64, i64, i64, p, p, i64, ctypes.c_int, p, p, i64, p]
    lib.oracle_forward_prefill_mx.argtypes = [i64, i64, i64, i64, i64, p, p, p, p, p, i64, p, p]
    lib.oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    for f in ("oracle_route", "oracle_forward_decode", "oracle_forward_prefill",
              "oracle_quantize_q8_0", "oracle_block_dots", "oracle_router_logits",
              "oracle_quantize_int4_gs64", "oracle_quantize_int8_gs64", "oracle_quantize_mxfp4",
              "oracle_quantize_mxfp8", "oracle_mx_dots", "oracle_forward_prefill_mx"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(_LIB)
    return _lib


class use_library:
    """Context manager: route every wrapper through another build of the
    oracle (the mutation tests use it to run the pins on broken copies)."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = _bind(self.path)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def compile_variant(src_text: str, out_path: str) -> str:
    """Compile C source text (a modified copy of the oracle) to out_path."""
    c_path = out_path + ".c"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-ffp-contract=off", "-w", "-o", out_path, c_path, "-lm"], check=True)
    return out_path


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def route(logits, top_k: int, flags: int, routed_scale: float = 1.0, sel_bias=None):
    """Top-k selection, routing weights and grouping.  logits fp32 [T, E]."""
    lib = _load()
    logits = _c(logits, np.float32)
    T, E = logits.shape
    P = T * top_k
    out = {
        "topk_idx": np.zeros(P, np.int32), "topk_w": np.zeros(P, np.float32),
        "counts": np.zeros(E, np.int32), "offsets": np.zeros(E + 1, np.int32),
        "pairs": np.zeros(P, np.int32),
    }
    sb = None if sel_bias is None else _c(sel_bias, np.float32)
    rc = lib.oracle_route(T, E, top_k, flags, routed_scale, _ptr(logits), _ptr(sb),
                          _ptr(out["topk_idx"]), _ptr(out["topk_w"]), _ptr(out["counts"]),
                          _ptr(out["offsets"]), _ptr(out["pairs"]))
    if rc != 0:
        raise ValueError("oracle_route: invalid arguments")
    out["topk_idx"] = out["topk_idx"].reshape(T, top_k)
    out["topk_w"] = out["topk_w"].reshape(T, top_k)
    return out


def quantize_int4_gs64(w):
    """int4 gs64 container of fp32 weights [rows, K] -> (uint8 [rows, K/2],
    uint16 fp16-bits [rows, K/64])."""
    lib = _load()
    w = _c(w, np.float32)
    rows, K = w.shape
    q4 = np.zeros((rows, K // 2), np.uint8)
    sc = np.zeros((rows, K // 64), np.uint16)
    if lib.oracle_quantize_int4_gs64(_ptr(w), rows, K, _ptr(q4), _ptr(sc)) != 0:
        raise ValueError("oracle_quantize_int4_gs64: invalid arguments")
    return q4, sc


def quantize_int8_gs64(w):
    """int8 gs64 container of fp32 weights [rows, K] -> (int8 [rows, K],
    uint16 fp16-bits [rows, K/64])."""
    lib = _load()
    w = _c(w, np.float32)
    rows, K = w.shape
    q = np.zeros((rows, K), np.int8)
    sc = np.zeros((rows, K // 64), np.uint16)
    if lib.oracle_quantize_int8_gs64(_ptr(w), rows, K, _ptr(q), _ptr(sc)) != 0:
        raise ValueError("oracle_quantize_int8_gs64: invalid arguments")
    return q, sc


def quantize_mxfp4(w):
    """MXFP4 of fp32 weights [rows, K] -> (uint8 nibbles [rows, K/2], uint8
    E8M0 [rows, K/32])."""
    lib = _load()
    w = _c(w, np.float32)
    rows, K = w.shape
    q = np.zeros((rows, K // 2), np.uint8)
    e = np.zeros((rows, K // 32), np.uint8)
    if lib.oracle_quantize_mxfp4(_ptr(w), rows, K, _ptr(q), _ptr(e)) != 0:
        raise ValueError("oracle_quantize_mxfp4: invalid arguments")
    return q, e


def router_logits(w_bf16, x_bf16):
    """Router logits fp32 [T, E] = x [T, H] . w [E, H]^T (bf16 bit patterns in)."""
    lib = _load()
    w = _c(w_bf16, np.uint16)
    x = _c(x_bf16, np.uint16)
    E, H = w.shape
    T = x.shape[0]
    if x.shape[1] != H:
        raise ValueError("router_logits: x and w disagree on H")
    out = np.zeros((T, E), np.float32)
    if lib.oracle_router_logits(T, E, H, _ptr(w), _ptr(x), _ptr(out)) != 0:
        raise ValueError("oracle_router_logits: invalid arguments")
    return out


WEIGHT_FORMATS = {"int4": 0, "int8": 1, "mxfp4": 2}


def _weights(q4, scales, weights):
    """Codes as bytes and scales as fp16 bits (int4, int8) or E8M0 bytes (mxfp4)."""
    fmt = WEIGHT_FORMATS[weights]
    return _c(q4, np.uint8), _c(scales, np.uint8 if weights == "mxfp4" else np.uint16), fmt


def forward_decode(H, I, E, S, k, q4, scales, topk_idx, topk_w, x_bf16, weights="int4"):
    """Decode-mode layer output, fp64 [T, H].  x_bf16: uint16 bits [T, H].
    weights: "int4" (nibbles + fp16 per 64), "int8" (bytes + fp16 per 64) or
    "mxfp4" (E2M1 nibbles + E8M0 byte per 32)."""
    lib = _load()
    q4, scales, fmt = _weights(q4, scales, weights)
    topk_idx, topk_w = _c(topk_idx, np.int32), _c(topk_w, np.float32)
    x = _c(x_bf16, np.uint16)
    T = x.shape[0]
    y = np.zeros((T, H), np.float64)
    rc = lib.oracle_forward_decode(H, I, E, S, k, _ptr(q4), _ptr(scales), _ptr(topk_idx),
                                   _ptr(topk_w), _ptr(x), T, _ptr(y), fmt)
    if rc != 0:
        raise ValueError("oracle_forward_decode failed")
    return y


def forward_prefill(H, I, E, S, k, q4, scales, topk_idx, topk_w, x_bf16, want_h=False,
                    weights="int4"):
    """Integer-path (Q8_0) layer output, fp64 [T, H] (and fp32 h [T, k+S, I])."""
    lib = _load()
    q4, scales, fmt = _weights(q4, scales, weights)
    topk_idx, topk_w = _c(topk_idx, np.int32), _c(topk_w, np.float32)
    x = _c(x_bf16, np.uint16)
    T = x.shape[0]
    y = np.zeros((T, H), np.float64)
    h = np.zeros((T, k + S, I), np.float32) if want_h else None
    rc = lib.oracle_forward_prefill(H, I, E, S, k, _ptr(q4), _ptr(scales), _ptr(topk_idx),
                                    _ptr(topk_w), _ptr(x), T, _ptr(y), _ptr(h), fmt)
    if rc != 0:
        raise ValueError("oracle_forward_prefill failed")
    return (y, h) if want_h else y


def quantize_q8_0(v):
    """Q8_0 of fp32 values (length % 32 == 0) -> (int8 q, uint16 fp16-bits d)."""
    lib = _load()
    v = _c(v, np.float32).reshape(-1)
    q = np.zeros(v.size, np.int8)
    d = np.zeros(v.size // 32, np.uint16)
    if lib.oracle_quantize_q8_0(_ptr(v), v.size, _ptr(q), _ptr(d)) != 0:
        raise ValueError("oracle_quantize_q8_0: length must be a multiple of 32")
    return q, d


def block_dots(H, I, E, S, q4, scales, expert, matrix, q_act, weights="int4"):
    """Exact int32 block dots [T, rows, K/32] of one matrix of one expert
    (mxfp4: of the doubled E2M1 values, integers in [-12, 12])."""
    lib = _load()
    q4, scales, fmt = _weights(q4, scales, weights)
    q_act = _c(q_act, np.int8)
    K = I if matrix == 2 else H
    rows = H if matrix == 2 else I
    T = q_act.reshape(-1, K).shape[0]
    dots = np.zeros((T, rows, K // 32), np.int32)
    rc = lib.oracle_block_dots(H, I, E, S, _ptr(q4), _ptr(scales), expert, matrix,
                               _ptr(q_act), T, _ptr(dots), fmt)
    if rc != 0:
        raise ValueError("oracle_block_dots: invalid arguments")
    return dots


def quantize_mxfp8(v):
    """MXFP8 (E4M3 elements, one E8M0 scale per 32) of fp32 values (length %
    32 == 0) -> (uint8 codes, uint8 E8M0 per 32)."""
    lib = _load()
    v = _c(v, np.float32).reshape(-1)
    q = np.zeros(v.size, np.uint8)
    e = np.zeros(v.size // 32, np.uint8)
    if lib.oracle_quantize_mxfp8(_ptr(v), v.size, _ptr(q), _ptr(e)) != 0:
        raise ValueError("oracle_quantize_mxfp8: length must be a multiple of 32")
    return q, e


def mx_dots(H, I, E, S, q4, scales, expert, matrix, qa, ea):
    """fp64 [T, rows]: matrix `matrix` of expert `expert` of an MXFP4 container
    against MXFP8 activation rows (qa uint8 [T, K] codes, ea uint8 [T, K/32])."""
    lib = _load()
    q4, scales = _c(q4, np.uint8), _c(scales, np.uint8)
    K = I if matrix == 2 else H
    rows = H if matrix == 2 else I
    qa = _c(qa, np.uint8).reshape(-1, K)
    ea = _c(ea, np.uint8).reshape(-1, K // 32)
    T = qa.shape[0]
    out = np.zeros((T, rows), np.float64)
    rc = lib.oracle_mx_dots(H, I, E, S, _ptr(q4), _ptr(scales), expert, matrix, _ptr(qa),
                            _ptr(ea), T, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_mx_dots: invalid arguments")
    return out


def forward_prefill_mx(H, I, E, S, k, q4, scales, topk_idx, topk_w, x_bf16, want_h=False):
    """MX-path layer output of an MXFP4 container (MXFP8 activations), fp64
    [T, H] (and fp32 h [T, k+S, I])."""
    lib = _load()
    q4, scales = _c(q4, np.uint8), _c(scales, np.uint8)
    topk_idx, topk_w = _c(topk_idx, np.int32), _c(topk_w, np.float32)
    x = _c(x_bf16, np.uint16)
    T = x.shape[0]
    y = np.zeros((T, H), np.float64)
    h = np.zeros((T, k + S, I), np.float32) if want_h else None
    rc = lib.oracle_forward_prefill_mx(H, I, E, S, k, _ptr(q4), _ptr(scales), _ptr(topk_idx),
                                       _ptr(topk_w), _ptr(x), T, _ptr(y), _ptr(h))
    if rc != 0:
        raise ValueError("oracle_forward_prefill_mx failed")
    return (y, h) if want_h else y


def f32_to_f16_bits(v: float) -> int:
    return int(_load().oracle_f32_to_f16(float(v)))


def threads() -> int:
    """OpenMP threads the oracle will use (OMP_NUM_THREADS or all cores)."""
    n = os.environ.get("OMP_NUM_THREADS")
    return int(n) if n and n.isdigit() else (os.cpu_count() or 1)
