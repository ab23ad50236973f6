"""Routed-expert MoE layer for MI355X (gfx950): Python binding of libcoli_moe.

The work happens in the HIP library libcoli_moe.so (C ABI declared in
include/coli_moe.h); this package only marshals arguments.  PyTorch supplies
device memory and the current stream.  There is no fallback: importing
`native` fails loudly if the library has not been built
(`python -m int4_routed_expert_router_amd.build`).

Functions carry the C names:

    coli_moe_workspace_bytes, coli_moe_route, coli_moe_route_hidden,
    coli_moe_forward_decode, coli_moe_forward_prefill, coli_moe_quantize_q8_0,
    coli_moe_quantize_int4_gs64, coli_moe_quantize_int8_gs64, coli_moe_quantize_mxfp4,
    coli_moe_read_probe, coli_moe_mfma_probe, coli_moe_block_dots, coli_moe_strerror,
    coli_moe_version

plus two small holders that own the device buffers the C calls take:
`Layer` (the int4 gs64 container + shape) and `Route` (route outputs).
"""
from .binding import (  # noqa: F401
    COLI_ENTRY_DECODE, COLI_ENTRY_PREFILL, COLI_ENTRY_ROUTE, COLI_OUT_BF16, COLI_OUT_F32,
    COLI_ROUTE_RENORM, COLI_ROUTE_SIGMOID, COLI_ROUTE_SOFTMAX, COLI_SRC_BF16, COLI_SRC_F32,
    COLI_WEIGHTS_INT4, COLI_WEIGHTS_INT8, COLI_WEIGHTS_MXFP4, COLI_ACT_MXFP8,
    COLI_MFMA_BF16_K32, COLI_MFMA_I8_K32, COLI_MFMA_I8_K64,
    ColiError, KernelTimer, Layer, Route, coli_moe_block_dots, coli_moe_forward_decode,
    coli_moe_forward_decode_noalloc,
    coli_moe_forward_prefill, coli_moe_quantize_int4_gs64, coli_moe_quantize_int8_gs64,
    coli_moe_quantize_mxfp4, coli_moe_quantize_mxfp8, coli_moe_quantize_q8_0, coli_moe_read_probe,
    coli_moe_mfma_probe, coli_moe_mx_dots,
    coli_moe_route, coli_moe_route_hidden,
    coli_moe_strerror, coli_moe_version, coli_moe_workspace_bytes, library_path, workspace,
)
