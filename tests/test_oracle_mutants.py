"""Plant plausible mistakes in copies of the oracle and check the pins fail.

Each mutant is one textual change of oracle/coli_oracle.c (a dropped term, a
flipped sign, a wrong index or scale group, a swapped nibble order, a wrong
rounding rule, ...).  The copy is compiled to a temporary library on the CPU
and the pin checks of test_oracle_pins.py run against it; at least one check
must fail for every mutant.  The real oracle is never modified.
"""
import pytest

import oracle
import test_oracle_pins as pins

CHECKS = [
    pins.check_f16_rounding, pins.check_q8_0_golden, pins.check_q8_0_vs_bruteforce,
    pins.check_route_golden, pins.check_route_vs_bruteforce, pins.check_route_invariants,
    pins.check_decode_vs_bruteforce, pins.check_decode_mean_invariant,
    pins.check_decode_zero_scales, pins.check_decode_swiglu_mlp, pins.check_decode_closed_form,
    pins.check_block_dots_vs_bruteforce, pins.check_prefill_vs_bruteforce,
    pins.check_prefill_zero_scales, pins.check_router_logits_closed_form,
    pins.check_router_logits_vs_bruteforce, pins.check_int4_quant_vs_bruteforce,
    pins.check_int4_quant_closed_form, pins.check_int4_quant_properties,
    pins.check_int8_decode_prefill_vs_bruteforce, pins.check_int8_block_dots,
    pins.check_mxfp4_decode_prefill_vs_bruteforce, pins.check_mxfp4_block_dots,
    pins.check_int8_quant, pins.check_mxfp4_quant, pins.check_mxfp8_quant, pins.check_mx_dots,
    pins.check_prefill_mx_vs_bruteforce,
]

# (name, text in the oracle, replacement)
MUTANTS = [
    ("nibble order swapped", "int v = high ? (byte >> 4) : (byte & 15);",
     "int v = high ? (byte & 15) : (byte >> 4);"),
    ("nibble read unsigned", "return v >= 8 ? v - 16 : v;", "return v;"),
    ("nibble sign off by one", "return v >= 8 ? v - 16 : v;", "return v > 8 ? v - 16 : v;"),
    ("scale group of 32", "return or_f16(((const uint16_t *)sc)[n * (K / 64) + k / 64]);",
     "return or_f16(((const uint16_t *)sc)[n * (K / 64) + (k / 32) % (K / 64)]);"),
    ("matrix stride wrong",
     "return L->q4 + e * 3 * or_mat_bytes(L) + (int64_t)m * or_mat_bytes(L);",
     "return L->q4 + e * 3 * or_mat_bytes(L) + (int64_t)m * or_mat_bytes(L) / 2;"),
    ("int8 code read unsigned", "if (fmt == OR_INT8) return (int)(int8_t)mat[n * K + k];",
     "if (fmt == OR_INT8) return (int)mat[n * K + k];"),
    ("int8 rows read as nibble rows", "if (fmt == OR_INT8) return (int)(int8_t)mat[n * K + k];",
     "if (fmt == OR_INT8) return (int)(int8_t)mat[n * (K / 2) + k];"),
    ("int8 matrix sized as nibbles", "return L->fmt == OR_INT8 ? L->I * L->H : L->I * L->H / 2;",
     "return L->I * L->H / 2;"),
    ("e2m1 subnormals read as normal", "const double v = e ? ldexp(1.0 + 0.5 * m, e - 1) : 0.5 * m;",
     "const double v = ldexp(1.0 + 0.5 * m, e - 1);"),
    ("e2m1 exponent bias 0", "const double v = e ? ldexp(1.0 + 0.5 * m, e - 1) : 0.5 * m;",
     "const double v = e ? ldexp(1.0 + 0.5 * m, e) : 0.5 * m;"),
    ("e8m0 scale not halved", "return ldexp(1.0, (int)sc[n * (K / 32) + k / 32] - 128);",
     "return ldexp(1.0, (int)sc[n * (K / 32) + k / 32] - 127);"),
    ("fp4 scale per 64", "return ldexp(1.0, (int)sc[n * (K / 32) + k / 32] - 128);",
     "return ldexp(1.0, (int)sc[n * (K / 32) + k / 64] - 128);"),
    ("fp4 nibbles high first", "or_e2m1((k & 1) ? byte >> 4 : byte & 15)",
     "or_e2m1((k & 1) ? byte & 15 : byte >> 4)"),
    ("up uses gate scales", "*su = or_sc(L, e, 1), *sd = or_sc(L, e, 2);\n  const int f = L->fmt;\n  OR_ROWS_PARALLEL\n  for (int64_t n = 0; n < I; ++n) {\n    double g = 0.0, u = 0.0;\n    for (int64_t k = 0; k < H; ++k) {",
     "*su = or_sc(L, e, 0), *sd = or_sc(L, e, 2);\n  const int f = L->fmt;\n  OR_ROWS_PARALLEL\n  for (int64_t n = 0; n < I; ++n) {\n    double g = 0.0, u = 0.0;\n    for (int64_t k = 0; k < H; ++k) {"),
    ("silu sign flipped", "return g / (1.0 + exp(-g));", "return g / (1.0 + exp(g));"),
    ("gate and up swapped in swiglu", "h[n] = or_silu(g) * u;", "h[n] = or_silu(u) * g;"),
    ("down transposed", "acc += (double)or_q(qd, I, m, n, f) * or_s(sd, I, m, n, f) * h[n];",
     "acc += (double)or_q(qd, I, n % I, m % I, f) * or_s(sd, I, m, n, f) * h[n];"),
    ("shared expert dropped", "      if (S) {\n        or_ffn_f64(&L, E, x, h, o);", "      if (0) {\n        or_ffn_f64(&L, E, x, h, o);"),
    ("routing weight ignored", "for (int64_t i = 0; i < H; ++i) yt[i] += w * o[i];\n      }\n      if (S)",
     "for (int64_t i = 0; i < H; ++i) yt[i] += o[i];\n      }\n      if (S)"),
    ("tie to higher index", "if (best < 0 || s > best_s) {", "if (best < 0 || s >= best_s) {"),
    ("selection bias ignored", "float s = sel_bias ? (float)(l[e] + sel_bias[e]) : l[e];", "float s = l[e];"),
    ("softmax without max shift and wrong sum", "for (int32_t e = 0; e < E; ++e) z += exp((double)l[e] - mx);",
     "for (int32_t e = 1; e < E; ++e) z += exp((double)l[e] - mx);"),
    ("renorm skipped", "for (int32_t j = 0; j < k; ++j) w[j] /= sum;", "(void)sum;"),
    ("routed scale dropped", "(float)(w[j] * (double)routed_scale)", "(float)(w[j])"),
    ("group order unstable", "for (int64_t p = 0; p < P; ++p) pairs[fill[topk_idx[p]]++] = (int32_t)p;",
     "for (int64_t p = P - 1; p >= 0; --p) pairs[fill[topk_idx[p]]++] = (int32_t)p;"),
    ("q8_0 rounds half to even", "r = (int)roundf(ratio);", "r = (int)nearbyintf(ratio);"),
    ("q8_0 divides by 128", "volatile float d = a / 127.0f;", "volatile float d = a / 128.0f;"),
    ("q8_0 truncates", "r = (int)roundf(ratio);", "r = (int)ratio;"),
    ("block dot off by one block", "for (int64_t k = 32 * b; k < 32 * b + 32; ++k)",
     "for (int64_t k = 32 * b; k < 32 * b + 31; ++k)"),
    ("prefill weight scale group", "g += or_s(sg, H, n, 32 * b, f) * d",
     "g += or_s(sg, H, n, b, f) * d"),
    ("prefill h not requantised", "acc += or_s(sd, I, m, 32 * b, f) * or_f16(dh[b]) *",
     "acc += or_s(sd, I, m, 32 * b, f) * or_f16(dh[0]) *"),
    ("f16 rounding truncates", "double m = nearbyint(ldexp(a, 10 - E));", "double m = floor(ldexp(a, 10 - E));"),
    ("int4 scale from max / 8", "volatile float s = a / 7.0f;", "volatile float s = a / 8.0f;"),
    ("int4 quantised with the fp32 scale", "const float sf = (float)or_f16(s16);",
     "const float sf = s;"),
    ("int4 rounds half to even",
     "r = (int)roundf(u);", "r = (int)nearbyintf(u);"),
    ("int4 clamps at -7", "if (r < -8) r = -8;", "if (r < -7) r = -7;"),
    ("int4 nibbles packed high first",
     "*byte = (k & 1) ? (uint8_t)((*byte & 0x0f) | (nib << 4)) : (uint8_t)((*byte & 0xf0) | nib);",
     "*byte = (k & 1) ? (uint8_t)((*byte & 0xf0) | nib) : (uint8_t)((*byte & 0x0f) | (nib << 4));"),
    ("int8 scale from max / 128", "volatile float t = a / 127.0f;",
     "volatile float t = a / 128.0f;"),
    ("int8 clamps at -127", "if (r < -128) r = -128;", "if (r < -127) r = -127;"),
    ("mxfp4 shared exponent off by one", "E = (ex - 1) - 2 + 127;", "E = (ex - 1) - 1 + 127;"),
    ("mxfp4 ties away from zero", "if (m < mid || (m == mid && (j & 1) == 0)) {", "if (m < mid) {"),
    ("mxfp4 codes packed high first",
     "*dst = (k & 1) ? (uint8_t)((*dst & 0x0f) | (nib << 4)) : (uint8_t)((*dst & 0xf0) | nib);",
     "*dst = (k & 1) ? (uint8_t)((*dst & 0xf0) | nib) : (uint8_t)((*dst & 0x0f) | (nib << 4));"),
    ("mxfp4 drops the sign of zero", "(wb[i] < 0.0f || (wb[i] == 0.0f && signbit(wb[i])))",
     "(wb[i] < 0.0f)"),
    ("router weight transposed", "acc += or_bf16(x[t * H + k]) * or_bf16(w[e * H + k]);",
     "acc += or_bf16(x[t * H + k]) * or_bf16(w[k * E + e]);"),
    ("router drops the last column", "for (int64_t k = 0; k < H; ++k) acc += or_bf16(x[t * H + k])",
     "for (int64_t k = 0; k < H - 1; ++k) acc += or_bf16(x[t * H + k])"),
    ("mxfp8 shared exponent off by one", "E = (ex - 1) - 8 + 127;", "E = (ex - 1) - 7 + 127;"),
    ("mxfp8 ties away from zero", "if (m < mid || (m == mid && !(j & 1))) {", "if (m < mid) {"),
    ("mxfp8 overflows to NaN", "int c = 0x7e; /* saturate at 448 */", "int c = 0x7f;"),
    ("mxfp8 drops the sign of zero",
     "const int neg = vb[i] < 0.0f || (vb[i] == 0.0f && signbit(vb[i]));",
     "const int neg = vb[i] < 0.0f;"),
    ("e4m3 exponent bias 8", "const double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);",
     "const double v = e ? ldexp(1.0 + m / 8.0, e - 8) : ldexp(m / 8.0, -6);"),
    ("e4m3 subnormals read as normal",
     "const double v = e ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);",
     "const double v = ldexp(1.0 + m / 8.0, e - 7);"),
    ("mx block drops the activation scale",
     "return ldexp(acc, ((int)sc[n * (K / 32) + b] - 127) + ((int)ea[b] - 127));",
     "return ldexp(acc, ((int)sc[n * (K / 32) + b] - 127));"),
    ("mx weight scale per 64",
     "return ldexp(acc, ((int)sc[n * (K / 32) + b] - 127) + ((int)ea[b] - 127));",
     "return ldexp(acc, ((int)sc[n * (K / 32) + b / 2] - 127) + ((int)ea[b] - 127));"),
    ("mx fp4 nibbles high first", "or_e2m1((k & 1) ? (byte >> 4) : (byte & 15))",
     "or_e2m1((k & 1) ? (byte & 15) : (byte >> 4))"),
    ("mx activations paired wrongly", "* or_e4m3(qa[k]);", "* or_e4m3(qa[k ^ 1]);"),
    ("mx up uses gate weights", "u += or_mx_block(qu, su, H, n, qx, ex, b);",
     "u += or_mx_block(qg, su, H, n, qx, ex, b);"),
    ("mx down repeats block 0",
     "for (int64_t b = 0; b < I / 32; ++b) acc += or_mx_block(qd, sd, I, m, qh, eh, b);",
     "for (int64_t b = 0; b < I / 32; ++b) acc += or_mx_block(qd, sd, I, m, qh, eh + b - b, 0);"),
    ("router accumulates in fp32",
     "double acc = 0.0;\n      for (int64_t k = 0; k < H; ++k) acc += or_bf16(x[t * H + k])",
     "float acc = 0.0f;\n      for (int64_t k = 0; k < H; ++k) acc += or_bf16(x[t * H + k])"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation anchor not found once: " + name
    lib = oracle.compile_variant(src.replace(old, new), str(tmp_path / "mutant.so"))
    failed = []
    with oracle.use_library(lib):
        for check in CHECKS:
            try:
                check()
            except (AssertionError, ValueError, IndexError):
                failed.append(check.__name__)
    assert failed, "no pin caught mutant: " + name
