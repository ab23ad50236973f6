"""ctypes binding of libcoli_moe.so: argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libcoli_moe.so")

COLI_OK, COLI_E_INVALID, COLI_E_UNSUPPORTED, COLI_E_WORKSPACE, COLI_E_ALIGN, COLI_E_HIP = (
    0, -1, -2, -3, -4, -5)
COLI_ROUTE_SOFTMAX, COLI_ROUTE_SIGMOID, COLI_ROUTE_RENORM = 0, 1, 256
COLI_OUT_BF16, COLI_OUT_F32 = 0, 1
COLI_SRC_BF16, COLI_SRC_F32 = 0, 1
COLI_ENTRY_ROUTE, COLI_ENTRY_DECODE, COLI_ENTRY_PREFILL = 0, 1, 2
COLI_WEIGHTS_INT4, COLI_WEIGHTS_INT8, COLI_WEIGHTS_MXFP4 = 0, 1, 2
COLI_ACT_MXFP8 = 1 << 16


class ColiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s: %s (status %d)" % (fn, coli_moe_strerror(status), status))
        self.status = status


class _LayerC(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("n_shared", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("flags", ctypes.c_uint32),
        ("routed_scale", ctypes.c_float),
        ("q4", ctypes.c_void_p), ("scales", ctypes.c_void_p),
        ("weight_format", ctypes.c_int32),
    ]


class _TraceC(ctypes.Structure):
    _fields_ = [("start", ctypes.POINTER(ctypes.c_void_p)), ("stop", ctypes.POINTER(ctypes.c_void_p)),
                ("kernel", ctypes.POINTER(ctypes.c_int32)), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32)]


KERNEL_NAMES = ["route_fused", "route_topk", "route_group", "decode_gateup", "decode_down",
                "combine", "quantize_q8_0", "plan", "gemm_gateup", "gemm_down", "block_dots",
                "router_logits", "quantize_int4", "quantize_int8", "quantize_mxfp4", "read_probe",
                "mfma_probe"]


class _RouteC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "topk_idx", "topk_w", "counts", "offsets", "pairs", "pair_pos", "union_ids", "n_union")]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(
                "libcoli_moe.so is not built (expected at %s); run "
                "`python -m int4_routed_expert_router_amd.build`" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        lib.coli_moe_workspace_bytes.argtypes = [P(_LayerC), i32, i32]
        lib.coli_moe_workspace_bytes.restype = sz
        lib.coli_moe_route.argtypes = [P(_LayerC), vp, vp, i32, P(_RouteC), vp, sz, vp]
        lib.coli_moe_route_hidden.argtypes = [P(_LayerC), vp, vp, vp, i32, vp, P(_RouteC), vp,
                                              sz, vp]
        lib.coli_moe_forward_decode.argtypes = [P(_LayerC), P(_RouteC), vp, i32, vp, i32, vp, sz, vp]
        lib.coli_moe_forward_prefill.argtypes = [P(_LayerC), P(_RouteC), vp, i32, vp, i32, vp, sz, vp]
        lib.coli_moe_forward_decode_noalloc.argtypes = [P(_LayerC), P(_RouteC), vp, i32, vp, i32, vp]
        lib.coli_moe_quantize_q8_0.argtypes = [vp, i32, i64, vp, vp, vp]
        lib.coli_moe_quantize_int4_gs64.argtypes = [vp, i32, i64, i64, vp, vp, vp]
        lib.coli_moe_quantize_int8_gs64.argtypes = [vp, i32, i64, i64, vp, vp, vp]
        lib.coli_moe_quantize_mxfp4.argtypes = [vp, i32, i64, i64, vp, vp, vp]
        lib.coli_moe_read_probe.argtypes = [vp, i64, vp, vp]
        lib.coli_moe_mfma_probe.argtypes = [i32, i32, i32, vp, vp]
        lib.coli_moe_block_dots.argtypes = [P(_LayerC), i32, i32, vp, i32, vp, vp]
        lib.coli_moe_quantize_mxfp8.argtypes = [vp, i32, i64, vp, vp, vp]
        lib.coli_moe_mx_dots.argtypes = [P(_LayerC), i32, i32, vp, vp, i32, vp, vp]
        lib.coli_moe_strerror.argtypes = [ctypes.c_int]
        lib.coli_moe_strerror.restype = ctypes.c_char_p
        lib.coli_moe_set_trace.argtypes = [ctypes.POINTER(_TraceC)]
        lib.coli_moe_set_trace.restype = ctypes.c_int
        lib.coli_moe_version.argtypes = []
        lib.coli_moe_version.restype = ctypes.c_char_p
        for f in ("coli_moe_route", "coli_moe_route_hidden", "coli_moe_forward_decode",
                  "coli_moe_forward_decode_noalloc", "coli_moe_forward_prefill", "coli_moe_quantize_q8_0", "coli_moe_block_dots",
                  "coli_moe_quantize_int4_gs64", "coli_moe_quantize_int8_gs64",
                  "coli_moe_quantize_mxfp4", "coli_moe_read_probe",
                  "coli_moe_mfma_probe", "coli_moe_quantize_mxfp8", "coli_moe_mx_dots"):
            getattr(lib, f).restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Layer:
    """One MoE layer: shape, routing kind and the device gs64 container.

    q4: uint8 tensor of (E+S)*3*I*H/2 bytes (int4 or MXFP4 codes) or
    (E+S)*3*I*H bytes (int8 codes, int8=True); scales: fp16 tensor of
    (E+S)*3*I*H/64 values, or for MXFP4 (mxfp4=True) a uint8 tensor of
    (E+S)*3*I*H/32 E8M0 bytes (see include/coli_moe.h for the byte layout).
    """

    def __init__(self, hidden, inter, n_experts, n_shared, top_k, flags, q4, scales,
                 routed_scale=1.0, int8=False, mxfp4=False):
        self.q4, self.scales = q4, scales  # keep the tensors alive
        fmt = COLI_WEIGHTS_MXFP4 if mxfp4 else (COLI_WEIGHTS_INT8 if int8 else COLI_WEIGHTS_INT4)
        self.c = _LayerC(hidden, inter, n_experts, n_shared, top_k, flags, routed_scale,
                         _ptr(q4), _ptr(scales), fmt)

    @classmethod
    def from_spec(cls, spec, q4, scales):
        return cls(spec.hidden, spec.inter, spec.n_experts, spec.n_shared, spec.top_k,
                   spec.flags, q4, scales, spec.routed_scale, getattr(spec, "int8", False),
                   getattr(spec, "mxfp4", False))

    hidden = property(lambda s: s.c.hidden)
    inter = property(lambda s: s.c.inter)
    n_experts = property(lambda s: s.c.n_experts)
    n_shared = property(lambda s: s.c.n_shared)
    top_k = property(lambda s: s.c.top_k)


class Route:
    """Device buffers written by coli_moe_route for up to `max_tokens` tokens."""

    def __init__(self, layer: Layer, max_tokens: int, device="cuda"):
        P = max_tokens * layer.top_k
        E = layer.n_experts
        i32 = dict(dtype=torch.int32, device=device)
        self.topk_idx = torch.empty(P, **i32)
        self.topk_w = torch.empty(P, dtype=torch.float32, device=device)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.pairs = torch.empty(P, **i32)
        self.pair_pos = torch.empty(P, **i32)
        self.union_ids = torch.empty(E, **i32)
        self.n_union = torch.empty(1, **i32)
        self.c = _RouteC(*[_ptr(getattr(self, n)) for n, _ in _RouteC._fields_])


def coli_moe_strerror(status: int) -> str:
    return _load().coli_moe_strerror(status).decode()


def coli_moe_version() -> str:
    return _load().coli_moe_version().decode()


def coli_moe_workspace_bytes(layer: Layer, T: int, entry: int) -> int:
    return int(_load().coli_moe_workspace_bytes(ctypes.byref(layer.c), T, entry))


def workspace(layer: Layer, T: int, entry: int, device="cuda") -> torch.Tensor:
    """A device buffer large enough for `entry` at T tokens (256-byte aligned)."""
    n = coli_moe_workspace_bytes(layer, T, entry)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def _check(fn, rc):
    if rc != COLI_OK:
        raise ColiError(fn, rc)


def coli_moe_route(layer: Layer, logits, sel_bias, T: int, route: Route, ws=None, stream=None):
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("coli_moe_route", _load().coli_moe_route(
        ctypes.byref(layer.c), _ptr(logits), _ptr(sel_bias), T, ctypes.byref(route.c),
        _ptr(ws), nb, _stream(stream)))


def coli_moe_route_hidden(layer: Layer, w_router, x, sel_bias, T: int, logits, route: Route,
                          ws=None, stream=None):
    nb = 0 if ws is None else ws.numel() * ws.element_size()
    _check("coli_moe_route_hidden", _load().coli_moe_route_hidden(
        ctypes.byref(layer.c), _ptr(w_router), _ptr(x), _ptr(sel_bias), T, _ptr(logits),
        ctypes.byref(route.c), _ptr(ws), nb, _stream(stream)))


def coli_moe_forward_decode(layer: Layer, route: Route, x, T: int, y, y_dtype: int, ws,
                            stream=None):
    _check("coli_moe_forward_decode", _load().coli_moe_forward_decode(
        ctypes.byref(layer.c), ctypes.byref(route.c), _ptr(x), T, _ptr(y), y_dtype,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def coli_moe_forward_decode_noalloc(layer: Layer, route: Route, x, T: int, y, y_dtype: int,
                                    stream=None):
    _check("coli_moe_forward_decode_noalloc", _load().coli_moe_forward_decode_noalloc(
        ctypes.byref(layer.c), ctypes.byref(route.c), _ptr(x), T, _ptr(y), y_dtype,
        _stream(stream)))


def coli_moe_forward_prefill(layer: Layer, route: Route, x, T: int, y, y_dtype: int, ws,
                             stream=None):
    _check("coli_moe_forward_prefill", _load().coli_moe_forward_prefill(
        ctypes.byref(layer.c), ctypes.byref(route.c), _ptr(x), T, _ptr(y), y_dtype,
        _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def coli_moe_quantize_q8_0(src, src_dtype: int, n: int, q, d, stream=None):
    _check("coli_moe_quantize_q8_0", _load().coli_moe_quantize_q8_0(
        _ptr(src), src_dtype, n, _ptr(q), _ptr(d), _stream(stream)))


def coli_moe_quantize_int4_gs64(src, src_dtype: int, rows: int, K: int, q4, scales,
                                stream=None):
    _check("coli_moe_quantize_int4_gs64", _load().coli_moe_quantize_int4_gs64(
        _ptr(src), src_dtype, rows, K, _ptr(q4), _ptr(scales), _stream(stream)))


def coli_moe_quantize_int8_gs64(src, src_dtype: int, rows: int, K: int, q, scales,
                                stream=None):
    _check("coli_moe_quantize_int8_gs64", _load().coli_moe_quantize_int8_gs64(
        _ptr(src), src_dtype, rows, K, _ptr(q), _ptr(scales), _stream(stream)))


def coli_moe_quantize_mxfp4(src, src_dtype: int, rows: int, K: int, q4, e8m0, stream=None):
    _check("coli_moe_quantize_mxfp4", _load().coli_moe_quantize_mxfp4(
        _ptr(src), src_dtype, rows, K, _ptr(q4), _ptr(e8m0), _stream(stream)))


def coli_moe_read_probe(src, nbytes: int, sink, stream=None):
    _check("coli_moe_read_probe", _load().coli_moe_read_probe(
        _ptr(src), nbytes, _ptr(sink), _stream(stream)))


COLI_MFMA_I8_K32, COLI_MFMA_I8_K64, COLI_MFMA_BF16_K32 = 0, 1, 2
MFMA_PROBE_OPS = {COLI_MFMA_I8_K32: 2 * 16 * 16 * 32, COLI_MFMA_I8_K64: 2 * 16 * 16 * 64,
                  COLI_MFMA_BF16_K32: 2 * 16 * 16 * 32}


def coli_moe_mfma_probe(kind: int, iters: int, workgroups: int, sink, stream=None):
    """Returns the operations the launch performs."""
    _check("coli_moe_mfma_probe", _load().coli_moe_mfma_probe(
        kind, iters, workgroups, _ptr(sink), _stream(stream)))
    return workgroups * 4 * iters * 4 * MFMA_PROBE_OPS[kind]


def coli_moe_block_dots(layer: Layer, expert: int, matrix: int, q_act, T: int, dots,
                        stream=None):
    _check("coli_moe_block_dots", _load().coli_moe_block_dots(
        ctypes.byref(layer.c), expert, matrix, _ptr(q_act), T, _ptr(dots), _stream(stream)))


def coli_moe_quantize_mxfp8(src, src_dtype: int, n: int, q, e8m0, stream=None):
    _check("coli_moe_quantize_mxfp8", _load().coli_moe_quantize_mxfp8(
        _ptr(src), src_dtype, n, _ptr(q), _ptr(e8m0), _stream(stream)))


def coli_moe_mx_dots(layer: Layer, expert: int, matrix: int, q_act, e_act, T: int, out,
                     stream=None):
    _check("coli_moe_mx_dots", _load().coli_moe_mx_dots(
        ctypes.byref(layer.c), expert, matrix, _ptr(q_act), _ptr(e_act), T, _ptr(out),
        _stream(stream)))


def _hip_runtime():
    """The HIP runtime already loaded in this process (torch's or the system's)."""
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    return ctypes.CDLL(path or "libamdhip64.so")


class KernelTimer:
    """Times every kernel the library launches while active: each dispatch
    stamps its own start and stop event (hipExtLaunchKernel)."""

    def __init__(self, capacity: int = 4096):
        _load()
        self.hip = _hip_runtime()
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.start = (ctypes.c_void_p * capacity)()
        self.stop = (ctypes.c_void_p * capacity)()
        self.kernel = (ctypes.c_int32 * capacity)()
        for arr in (self.start, self.stop):
            for i in range(capacity):
                ev = ctypes.c_void_p()
                if self.hip.hipEventCreate(ctypes.byref(ev)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                arr[i] = ev
        self.c = _TraceC(ctypes.cast(self.start, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(self.stop, ctypes.POINTER(ctypes.c_void_p)),
                         ctypes.cast(self.kernel, ctypes.POINTER(ctypes.c_int32)), capacity, 0)

    def __enter__(self):
        self.c.count = 0
        _check("coli_moe_set_trace", _load().coli_moe_set_trace(ctypes.byref(self.c)))
        return self

    def __exit__(self, *exc):
        _load().coli_moe_set_trace(None)
        return False

    def results(self):
        """[(kernel name, milliseconds)] of every timed kernel, in launch order."""
        out = []
        for i in range(self.c.count):
            self.hip.hipEventSynchronize(self.stop[i])
            ms = ctypes.c_float()
            if self.hip.hipEventElapsedTime(ctypes.byref(ms), self.start[i], self.stop[i]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append((KERNEL_NAMES[self.kernel[i]], ms.value))
        return out

    def close(self):
        for arr in (self.start, self.stop):
            for ev in arr:
                if ev:
                    self.hip.hipEventDestroy(ev)


def raw_library():
    """The loaded ctypes library (tests use it to check exported symbols)."""
    return _load()
