"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host (no GPU needed: every call here fails validation before
any HIP call, so nothing is launched)."""
import ctypes
import os
import re

import pytest

import int4_routed_expert_router_amd as coli
from int4_routed_expert_router_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli_moe.h")

FAKE = 0x100000  # a 256-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coli_moe_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("coli_moe_route", "coli_moe_route_hidden", "coli_moe_forward_decode",
              "coli_moe_forward_prefill", "coli_moe_workspace_bytes", "coli_moe_quantize_q8_0",
              "coli_moe_quantize_int4_gs64", "coli_moe_block_dots", "coli_moe_strerror", "coli_moe_version",
              "coli_moe_forward_decode_noalloc"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = binding.raw_library()
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert coli.coli_moe_version().count(".") == 2
    assert coli.coli_moe_strerror(-3) == "workspace too small"


def _layer(mxfp4=False, **kw):
    args = dict(hidden=2048, inter=512, n_experts=256, n_shared=1, top_k=8,
                flags=coli.COLI_ROUTE_SIGMOID | coli.COLI_ROUTE_RENORM, q4=FAKE, scales=FAKE)
    args.update(kw)
    return coli.Layer(args["hidden"], args["inter"], args["n_experts"], args["n_shared"],
                      args["top_k"], args["flags"], args["q4"], args["scales"], mxfp4=mxfp4)


class _FakeRoute:
    def __init__(self, null=False):
        self.c = binding._RouteC(*([0 if null else FAKE] * 8))


def test_workspace_sizes():
    L = _layer()
    T = 16
    rows = T * (8 + 1)
    dec = coli.coli_moe_workspace_bytes(L, T, coli.COLI_ENTRY_DECODE)
    assert dec == rows * 512 * 4 + rows * 2048 * 4  # h and o, fp32
    pre = coli.coli_moe_workspace_bytes(L, T, coli.COLI_ENTRY_PREFILL)
    assert pre > rows * 2048 * 4 + T * 2048
    assert coli.coli_moe_workspace_bytes(L, T, coli.COLI_ENTRY_ROUTE) == 0
    assert coli.coli_moe_workspace_bytes(L, 65, coli.COLI_ENTRY_DECODE) == 0  # T > 64
    assert coli.coli_moe_workspace_bytes(_layer(hidden=100), T, coli.COLI_ENTRY_DECODE) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=100), -1), (dict(inter=32), -1), (dict(hidden=16384 + 64), -1),
    (dict(n_experts=0), -1), (dict(n_experts=1025), -1), (dict(n_shared=2), -1),
    (dict(top_k=0), -1), (dict(top_k=257), -1), (dict(n_experts=64, top_k=33), -1),
    (dict(flags=2), -1), (dict(q4=0), -1), (dict(q4=FAKE + 8), -4), (dict(scales=FAKE + 2), -4),
])
def test_forward_rejects_bad_layers(kw, code):
    L = _layer(**kw)
    lib = binding.raw_library()
    rc = lib.coli_moe_forward_decode(ctypes.byref(L.c), ctypes.byref(_FakeRoute().c), FAKE, 1,
                                     FAKE, 0, FAKE, 1 << 40, None)
    assert rc == code


def test_forward_rejects_bad_calls():
    L = _layer()
    lib = binding.raw_library()
    r = ctypes.byref(_FakeRoute().c)
    big = 1 << 40
    dec = lib.coli_moe_forward_decode
    pre = lib.coli_moe_forward_prefill
    assert dec(ctypes.byref(L.c), r, FAKE, 0, FAKE, 0, FAKE, big, None) == -1      # T = 0
    assert dec(ctypes.byref(L.c), r, FAKE, 65, FAKE, 0, FAKE, big, None) == -1     # T > 64
    assert pre(ctypes.byref(L.c), r, FAKE, 65537, FAKE, 0, FAKE, big, None) == -1  # T too big
    assert dec(ctypes.byref(L.c), r, 0, 1, FAKE, 0, FAKE, big, None) == -1         # x NULL
    assert dec(ctypes.byref(L.c), r, FAKE, 1, FAKE, 7, FAKE, big, None) == -1      # y dtype
    assert dec(ctypes.byref(L.c), r, FAKE + 2, 1, FAKE, 0, FAKE, big, None) == -4  # x align
    assert dec(ctypes.byref(L.c), ctypes.byref(_FakeRoute(null=True).c), FAKE, 1, FAKE, 0,
               FAKE, big, None) == -1                                              # route
    need = coli.coli_moe_workspace_bytes(L, 4, coli.COLI_ENTRY_DECODE)
    assert dec(ctypes.byref(L.c), r, FAKE, 4, FAKE, 0, FAKE, need - 1, None) == -3
    assert dec(ctypes.byref(L.c), r, FAKE, 4, FAKE, 0, FAKE + 16, need, None) == -4
    need = coli.coli_moe_workspace_bytes(L, 300, coli.COLI_ENTRY_PREFILL)
    assert pre(ctypes.byref(L.c), r, FAKE, 300, FAKE, 0, FAKE, need - 1, None) == -3


def test_noalloc_decode_validates_before_any_hip_call():
    lib = binding.raw_library()
    na = lib.coli_moe_forward_decode_noalloc
    r = ctypes.byref(_FakeRoute().c)
    assert na(ctypes.byref(_layer(hidden=100).c), r, FAKE, 1, FAKE, 0, None) == -1  # layer
    assert na(ctypes.byref(_layer().c), r, FAKE, 65, FAKE, 0, None) == -1           # T > 64
    assert na(ctypes.byref(_layer().c), r, FAKE + 2, 1, FAKE, 0, None) == -4        # x align
    # past the 32 MiB scratch: 64 tokens x 33 rows of H + I = 16384 + 512 fp32 values
    big = _layer(hidden=16384, n_experts=64, top_k=32)
    assert coli.coli_moe_workspace_bytes(big, 64, coli.COLI_ENTRY_DECODE) > 32 << 20
    assert na(ctypes.byref(big.c), r, FAKE, 64, FAKE, 0, None) == -3
    # the largest GLM-shaped call fits
    glm = _layer(hidden=6144, inter=2048)
    assert coli.coli_moe_workspace_bytes(glm, 64, coli.COLI_ENTRY_DECODE) <= 32 << 20


def test_route_quantize_dots_reject_bad_calls():
    L = _layer()
    lib = binding.raw_library()
    r = ctypes.byref(_FakeRoute().c)
    assert lib.coli_moe_route(None, FAKE, None, 4, r, None, 0, None) == -1
    assert lib.coli_moe_route(ctypes.byref(L.c), 0, None, 4, r, None, 0, None) == -1
    assert lib.coli_moe_route(ctypes.byref(L.c), FAKE, None, 0, r, None, 0, None) == -1
    assert lib.coli_moe_route(ctypes.byref(L.c), FAKE + 1, None, 4, r, None, 0, None) == -4
    assert lib.coli_moe_route(ctypes.byref(L.c), FAKE, None, 65537, r, None, 0, None) == -1
    q = lib.coli_moe_quantize_q8_0
    assert q(FAKE, 0, 33, FAKE, FAKE, None) == -1
    assert q(FAKE, 2, 64, FAKE, FAKE, None) == -1
    assert q(FAKE + 2, 0, 64, FAKE, FAKE, None) == -4
    q4 = lib.coli_moe_quantize_int4_gs64
    assert q4(None, 0, 1, 64, FAKE, FAKE, None) == -1         # src NULL
    assert q4(FAKE, 2, 1, 64, FAKE, FAKE, None) == -1         # dtype
    assert q4(FAKE, 0, 0, 64, FAKE, FAKE, None) == -1         # rows = 0
    assert q4(FAKE, 0, 1, 96, FAKE, FAKE, None) == -1         # K % 64
    assert q4(FAKE, 0, 1 << 30, 128, FAKE, FAKE, None) == -1  # rows * K > 2^34
    # rows * K just past 2^34: one work-item per 8 values would pass 2^31
    assert q4(FAKE, 0, (1 << 28) + 1, 64, FAKE, FAKE, None) == -1
    assert lib.coli_moe_quantize_int8_gs64(FAKE, 0, (1 << 28) + 1, 64, FAKE, FAKE, None) == -1
    assert lib.coli_moe_quantize_mxfp4(FAKE, 0, (1 << 29) + 1, 32, FAKE, FAKE, None) == -1
    assert q4(FAKE + 8, 0, 1, 64, FAKE, FAKE, None) == -4     # src align
    assert q4(FAKE, 1, 1, 64, FAKE + 2, FAKE, None) == -4     # q4 align
    assert q4(FAKE, 1, 1, 64, FAKE, FAKE + 1, None) == -4     # scales align
    rp = lib.coli_moe_read_probe
    assert rp(None, 16, FAKE, None) == -1         # src NULL
    assert rp(FAKE, 24, FAKE, None) == -1         # bytes % 16
    assert rp(FAKE, 0, FAKE, None) == -1          # bytes = 0
    assert rp(FAKE, (1 << 36) + 16, FAKE, None) == -1   # past 2^36 bytes
    assert rp(FAKE, 16, None, None) == -1         # sink NULL
    assert rp(FAKE + 8, 16, FAKE, None) == -4     # src align
    assert rp(FAKE, 16, FAKE + 2, None) == -4     # sink align
    mp = lib.coli_moe_mfma_probe
    assert mp(3, 1, 1, FAKE, None) == -1          # kind
    assert mp(-1, 1, 1, FAKE, None) == -1
    assert mp(0, 0, 1, FAKE, None) == -1          # iters
    assert mp(0, (1 << 20) + 1, 1, FAKE, None) == -1
    assert mp(1, 1, 0, FAKE, None) == -1          # workgroups
    assert mp(2, 1, 1, None, None) == -1          # sink NULL
    assert mp(2, 1, 1, FAKE + 2, None) == -4      # sink align
    bd = lib.coli_moe_block_dots
    assert bd(ctypes.byref(L.c), 257, 0, FAKE, 4, FAKE, None) == -1   # expert out of range
    assert bd(ctypes.byref(L.c), 0, 3, FAKE, 4, FAKE, None) == -1     # matrix out of range
    assert bd(ctypes.byref(L.c), 0, 0, FAKE, 0, FAKE, None) == -1     # T = 0


def test_mx_path_rejects_bad_calls():
    """MXFP8 activations pair with MXFP4 weights only; the MX prefill needs H
    and I multiples of 256; the MX debug calls check their arguments."""
    lib = binding.raw_library()
    r = ctypes.byref(_FakeRoute().c)
    big = 1 << 40
    mx = coli.COLI_ROUTE_SIGMOID | coli.COLI_ACT_MXFP8
    pre = lib.coli_moe_forward_prefill
    assert pre(ctypes.byref(_layer(flags=mx).c), r, FAKE, 4, FAKE, 0, FAKE, big, None) == -1
    odd = _layer(mxfp4=True, flags=mx, hidden=192, inter=320)
    assert pre(ctypes.byref(odd.c), r, FAKE, 4, FAKE, 0, FAKE, big, None) == -2
    # decode ignores the flag: an int4-style argument error still comes first
    assert lib.coli_moe_forward_decode(ctypes.byref(odd.c), r, FAKE + 2, 1, FAKE, 0, FAKE, big,
                                       None) == -4
    q = lib.coli_moe_quantize_mxfp8
    assert q(FAKE, 0, 33, FAKE, FAKE, None) == -1            # n % 32
    assert q(FAKE, 2, 64, FAKE, FAKE, None) == -1            # dtype
    assert q(None, 0, 64, FAKE, FAKE, None) == -1            # src NULL
    assert q(FAKE + 2, 0, 64, FAKE, FAKE, None) == -4        # src align
    assert q(FAKE, 0, (1 << 34) + 32, FAKE, FAKE, None) == -1
    d = lib.coli_moe_mx_dots
    f4 = _layer(mxfp4=True)
    assert d(ctypes.byref(_layer().c), 0, 0, FAKE, FAKE, 4, FAKE, None) == -1   # not MXFP4
    assert d(ctypes.byref(f4.c), 257, 0, FAKE, FAKE, 4, FAKE, None) == -1       # expert
    assert d(ctypes.byref(f4.c), 0, 3, FAKE, FAKE, 4, FAKE, None) == -1         # matrix
    assert d(ctypes.byref(f4.c), 0, 0, FAKE, FAKE, 0, FAKE, None) == -1         # T
    assert d(ctypes.byref(f4.c), 0, 0, FAKE, FAKE, 4097, FAKE, None) == -1
    assert d(ctypes.byref(f4.c), 0, 0, FAKE + 8, FAKE, 4, FAKE, None) == -4     # q align
    assert d(ctypes.byref(f4.c), 0, 0, FAKE, FAKE + 2, 4, FAKE, None) == -4     # e align
    assert d(ctypes.byref(_layer(mxfp4=True, hidden=192).c), 0, 0, FAKE, FAKE, 4, FAKE,
             None) == -2                                                        # K % 256


def test_route_hidden_rejects_bad_calls():
    L = _layer()
    lib = binding.raw_library()
    r = ctypes.byref(_FakeRoute().c)
    rh = lib.coli_moe_route_hidden
    Lc = ctypes.byref(L.c)
    assert rh(None, FAKE, FAKE, None, 4, FAKE, r, None, 0, None) == -1
    assert rh(Lc, 0, FAKE, None, 4, FAKE, r, None, 0, None) == -1          # weights NULL
    assert rh(Lc, FAKE, 0, None, 4, FAKE, r, None, 0, None) == -1          # x NULL
    assert rh(Lc, FAKE, FAKE, None, 4, 0, r, None, 0, None) == -1          # logits NULL
    assert rh(Lc, FAKE, FAKE, None, 0, FAKE, r, None, 0, None) == -1       # T = 0
    assert rh(Lc, FAKE, FAKE, None, 65537, FAKE, r, None, 0, None) == -1   # T too big
    assert rh(Lc, FAKE + 8, FAKE, None, 4, FAKE, r, None, 0, None) == -4   # weights align
    assert rh(Lc, FAKE, FAKE + 2, None, 4, FAKE, r, None, 0, None) == -4   # x align
    assert rh(Lc, FAKE, FAKE, FAKE + 1, 4, FAKE, r, None, 0, None) == -4   # bias align
    assert rh(Lc, FAKE, FAKE, None, 4, FAKE,
              ctypes.byref(_FakeRoute(null=True).c), None, 0, None) == -1  # route buffers


def test_package_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        binding.raw_library()
