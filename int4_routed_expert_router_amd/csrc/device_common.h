// device_common.h -- small gfx950 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define COLI_DEV __device__ __forceinline__

typedef __bf16 coli_bf16x2 __attribute__((ext_vector_type(2)));
typedef int coli_i32x4 __attribute__((ext_vector_type(4)));

namespace coli {

constexpr int kWave = 64;

COLI_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

COLI_DEV float f16_to_f32(uint16_t bits) {
  return (float)__builtin_bit_cast(_Float16, bits);
}

// fp32 -> fp16 bits, round to nearest even (hardware conversion, default mode).
COLI_DEV uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
COLI_DEV uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs (v_dot2c_f32_bf16).
COLI_DEV float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(coli_bf16x2, a),
                                         __builtin_bit_cast(coli_bf16x2, b), acc, false);
}

// Four bf16 pairs from one dword of eight nibbles.  Nibble i (bits 4i..4i+3)
// is the weight of reduction index 8*dw + i.  The output pairs are
// (nibble 0, nibble 4), (1, 5), (2, 6), (3, 7); each element is the bf16
// value 128 + (q + 8) = 136 + q, exact, so a dot with activations carries a
// bias of 136 * sum(x) that the caller removes.
constexpr uint32_t kNibBias = 136;
// (a & b) ^ c as a v_bitop3_b32 truth table (a = 0xF0, b = 0xCC, c = 0xAA).
constexpr uint32_t kAndXor = 0x6Au;
COLI_DEV void nib8_to_bf16x4(uint32_t w, uint32_t &p0, uint32_t &p1, uint32_t &p2,
                             uint32_t &p3) {
  // (nibble & 15) ^ 8 turns two's complement into offset binary q + 8; the
  // upper bits 0x4300 make the bf16 value 128 + (q + 8).  Both in one
  // bitop3: ((w >> s) & 0x000f000f) ^ 0x43084308.
  constexpr uint32_t M = 0x000f000fu, K = 0x43084308u;
  p0 = __builtin_amdgcn_bitop3_b32(w, M, K, kAndXor);
  p1 = __builtin_amdgcn_bitop3_b32(w >> 4, M, K, kAndXor);
  p2 = __builtin_amdgcn_bitop3_b32(w >> 8, M, K, kAndXor);
  p3 = __builtin_amdgcn_bitop3_b32(w >> 12, M, K, kAndXor);
}

// Eight consecutive bf16 activations (x0..x7 packed in four dwords, low half
// first) rearranged into the pair order of nib8_to_bf16x4.
COLI_DEV void x8_to_pairs(const uint32_t d[4], uint32_t out[4]) {
  // out0 = (x0, x4), out1 = (x1, x5), out2 = (x2, x6), out3 = (x3, x7)
  out[0] = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);
  out[1] = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);
  out[2] = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);
  out[3] = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);
}

// -136 * (sum of a chunk's 32 activations), from its 16 paired dwords, in one
// fixed order.  Every dot2 decode kernel that removes the nibble bias uses
// these, so a token's result is the same whichever of them handled it.
constexpr uint32_t kBf16Ones = 0x3f803f80u;  // bf16 (1.0, 1.0)
COLI_DEV float chunk_bias(const uint32_t p[16]) {
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) s = dot2_bf16(p[q], kBf16Ones, s);
  return -(float)kNibBias * s;
}
// the same for an activation split into bf16 hi + lo halves
COLI_DEV float chunk_bias2(const uint32_t hp[16], const uint32_t lp[16]) {
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    s = dot2_bf16(hp[q], kBf16Ones, s);
    s = dot2_bf16(lp[q], kBf16Ones, s);
  }
  return -(float)kNibBias * s;
}

template <int W>
COLI_DEV float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

COLI_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

COLI_DEV float wave_sum(float v) { return group_sum<64>(v); }

COLI_DEV float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

}  // namespace coli
