// codec.h -- the weight codecs of the decode GEMVs (device code, shared by
// the streaming kernels and the general decode kernels).
#pragma once

#include "device_common.h"

namespace coli {
namespace {

// Weight codecs.  A chunk is 32 consecutive weights of a row (half of a
// 64-weight scale group): Q 16-byte quads of codes.  Activations are staged
// as 16 bf16 pairs per chunk in the pair order the codec's unpacking
// produces; every pair value is an exact bf16 integer (bias + q), and a
// codec with a bias removes the chunk's bias * sum(x) before its fp16 scale.
//
// int4 (one nibble per weight): one quad per chunk; pairs (k, k+4) within
// each 8 weights; bf16 136 + q from one v_bitop3 per pair.
struct CodecI4 {
  static constexpr int Q = 1;
  static constexpr int kChunksPerScale = 2;
  static constexpr float kBias = (float)kNibBias;
  static constexpr int64_t bytes(int64_t codes) { return codes / 2; }
  // fp16 scale of 32-value chunk c of row n of a K-wide matrix, whose
  // scales start at byte base (one per 64 weights)
  COLI_DEV static uint16_t scale_raw(const uint8_t *base, int64_t n, int K, int c) {
    return reinterpret_cast<const uint16_t *>(base)[n * (K / 64) + c / 2];
  }
  COLI_DEV static float scale(uint16_t raw) { return f16_to_f32(raw); }

  COLI_DEV static void pairs(const uint32_t d[4], uint32_t out[4]) { x8_to_pairs(d, out); }
  // chunk dotted with pairs xp (and, when lp is given, with a second set of
  // pairs lp: the low half of a split activation), from accumulator a
  template <bool TWO>
  COLI_DEV static float dot(const uint4 *w, const uint32_t *xp, const uint32_t *lp, float a) {
    const uint32_t wv[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      uint32_t p[4];
      nib8_to_bf16x4(wv[dw], p[0], p[1], p[2], p[3]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a = dot2_bf16(p[q], xp[4 * dw + q], a);
        if (TWO) a = dot2_bf16(p[q], lp[4 * dw + q], a);
      }
    }
    return a;
  }
  // bf16 slot of value w (0..31) in a chunk half: dword 4o + q pairs values
  // 8o + q (low 16 bits) and 8o + q + 4 (high 16 bits)
  COLI_DEV static int half_index(int w) {
    const int o = w >> 3, k = w & 7;
    return 2 * (4 * o + (k & 3)) + (k >> 2);
  }
  // eight weights (one dword) as four bf16 pairs in the activation pair order
  COLI_DEV static void kgroup(const uint32_t *dw, uint32_t out[4]) {
    nib8_to_bf16x4(dw[0], out[0], out[1], out[2], out[3]);
  }
  // raw scale of chunk cw of a run of chunks whose fp16 group scales (one
  // per two chunks) are packed in d
  COLI_DEV static uint16_t scale_at(const uint32_t *d, int cw) {
    return (uint16_t)(d[cw >> 2] >> (16 * ((cw >> 1) & 1)));
  }
};

// int8 (one byte per weight): two quads per chunk; natural pairs (k, k+1).
// Each signed byte converts to fp32 exactly (one sign-extending byte select
// per value) and two of them pack into a bf16 pair (their low halves are
// zero), so the pairs hold q itself: no bias, no cancellation.
struct CodecI8 {
  static constexpr int Q = 2;
  static constexpr int kChunksPerScale = 2;
  static constexpr float kBias = 0.0f;
  static constexpr int64_t bytes(int64_t codes) { return codes; }
  // fp16 scale of 32-value chunk c of row n of a K-wide matrix, whose
  // scales start at byte base (one per 64 weights)
  COLI_DEV static uint16_t scale_raw(const uint8_t *base, int64_t n, int K, int c) {
    return reinterpret_cast<const uint16_t *>(base)[n * (K / 64) + c / 2];
  }
  COLI_DEV static float scale(uint16_t raw) { return f16_to_f32(raw); }

  COLI_DEV static void pairs(const uint32_t d[4], uint32_t out[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = d[i];
  }
  COLI_DEV static uint32_t bf16_pair(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
  template <bool TWO>
  COLI_DEV static float dot(const uint4 *w, const uint32_t *xp, const uint32_t *lp, float a) {
    const uint32_t wv[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
    for (int dw = 0; dw < 8; ++dw) {
      const uint32_t v = wv[dw];
      const uint32_t p01 = bf16_pair((float)(int8_t)v, (float)(int8_t)(v >> 8));
      const uint32_t p23 = bf16_pair((float)(int8_t)(v >> 16), (float)(int8_t)(v >> 24));
      a = dot2_bf16(p01, xp[2 * dw], a);
      if (TWO) a = dot2_bf16(p01, lp[2 * dw], a);
      a = dot2_bf16(p23, xp[2 * dw + 1], a);
      if (TWO) a = dot2_bf16(p23, lp[2 * dw + 1], a);
    }
    return a;
  }
  COLI_DEV static int half_index(int w) { return w; }
  // eight weights (two dwords) as four bf16 pairs, natural order
  COLI_DEV static void kgroup(const uint32_t *dw, uint32_t out[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t v = dw[i];
      out[2 * i] = bf16_pair((float)(int8_t)v, (float)(int8_t)(v >> 8));
      out[2 * i + 1] = bf16_pair((float)(int8_t)(v >> 16), (float)(int8_t)(v >> 24));
    }
  }
  COLI_DEV static uint16_t scale_at(const uint32_t *d, int cw) {
    return (uint16_t)(d[cw >> 2] >> (16 * ((cw >> 1) & 1)));
  }
};

// MXFP4 (E2M1 nibbles, one E8M0 scale byte per 32 weights): one quad per
// chunk and one scale per chunk.  v_cvt_scalef32_pk_bf16_fp4 turns the two
// E2M1 codes of a byte (low nibble first) into an exact bf16 pair (scale 1;
// the chunk's power of two is applied after the dot); natural pairs.
struct CodecF4 {
  static constexpr int Q = 1;
  static constexpr int kChunksPerScale = 1;
  static constexpr float kBias = 0.0f;
  static constexpr int64_t bytes(int64_t codes) { return codes / 2; }
  COLI_DEV static uint16_t scale_raw(const uint8_t *base, int64_t n, int K, int c) {
    return base[n * (K / 32) + c];
  }
  // 2^(E - 127); E = 0 is the fp32 subnormal 2^-127
  COLI_DEV static float scale(uint16_t e) {
    return __uint_as_float(e ? (uint32_t)e << 23 : 0x00400000u);
  }
  COLI_DEV static void pairs(const uint32_t d[4], uint32_t out[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = d[i];
  }
  template <int B>  // byte B of v (the byte select is an instruction field)
  COLI_DEV static uint32_t pair(uint32_t v) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, B));
  }
  template <bool TWO>
  COLI_DEV static float dot(const uint4 *w, const uint32_t *xp, const uint32_t *lp, float a) {
    const uint32_t wv[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const uint32_t p[4] = {pair<0>(wv[dw]), pair<1>(wv[dw]), pair<2>(wv[dw]), pair<3>(wv[dw])};
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        a = dot2_bf16(p[b], xp[4 * dw + b], a);
        if (TWO) a = dot2_bf16(p[b], lp[4 * dw + b], a);
      }
    }
    return a;
  }
  COLI_DEV static int half_index(int w) { return w; }
  COLI_DEV static void kgroup(const uint32_t *dw, uint32_t out[4]) {
    out[0] = pair<0>(dw[0]);
    out[1] = pair<1>(dw[0]);
    out[2] = pair<2>(dw[0]);
    out[3] = pair<3>(dw[0]);
  }
  // E8M0 bytes, one per chunk
  COLI_DEV static uint16_t scale_at(const uint32_t *d, int cw) {
    return (uint16_t)((d[cw >> 2] >> (8 * (cw & 3))) & 0xffu);
  }
};

template <class C>
COLI_DEV float codec_bias(const uint32_t p[16]) {
  if (C::kBias == 0.0f) return 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) s = dot2_bf16(p[q], kBf16Ones, s);
  return -C::kBias * s;
}
template <class C>
COLI_DEV float codec_bias2(const uint32_t hp[16], const uint32_t lp[16]) {
  if (C::kBias == 0.0f) return 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    s = dot2_bf16(hp[q], kBf16Ones, s);
    s = dot2_bf16(lp[q], kBf16Ones, s);
  }
  return -C::kBias * s;
}

}  // namespace
}  // namespace coli
