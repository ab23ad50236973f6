// convert.hip -- float weights -> the int4 gs64 expert container.
//
// The container (tantan.ink post, section "我看到的几个坑": int4, symmetric,
// one fp16 scale per 64 weights) is made offline from the float checkpoint,
// one shard at a time (tantan.ink post, section "几个关键工程动作"; siami.tw
// article, section "技術核心").  The pages do not give the quantiser.  The
// rule implemented, per group of 64 consecutive weights of a row:
//   a = max |w|;  s = a / 7 in fp32 (IEEE division);  s16 = s rounded to
//   fp16 (nearest-even);  q = round half away from zero of fp32(w / s16),
//   clamped to [-8, 7];  a group with s16 == 0 gives q = 0.
// Weights are quantised against the scale the decoders multiply by, so the
// rounding error of each weight is at most half of s16.
//
// Layout: K % 64 == 0, so a row-major [rows][K] matrix is a flat sequence of
// groups -- group g is source values [64g, 64g+64), nibble bytes
// [32g, 32g+32) and scale g -- and one launch covers any number of
// matrices stored back to back (a whole expert, gate | up | down).
//
// One group is handled by 8 lanes, 8 values each: a 16-byte load per lane
// (two for fp32), max across the 8 lanes by three DPP moves, and one 4-byte
// store of 8 nibbles per lane, so loads and stores of a wavefront are
// contiguous.  Both divisions give the IEEE fp32 quotient.
#include "device_common.h"
#include "internal.h"

namespace coli {
namespace {

constexpr int kThreads = 256;  // 32 groups per workgroup

// DPP lane patterns (all lanes of each row and bank take part)
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1, 0, 3, 2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2, 3, 0, 1]
constexpr int kHalfRowMirror = 0x141;  // reverse within each group of 8 lanes
template <int CTRL>
COLI_DEV uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// 8-lane maximum of a >= 0 (non-negative floats order as their bit
// patterns do); the 8 lanes are consecutive and aligned.
COLI_DEV float max8(float a) {
  uint32_t ab = __float_as_uint(a);
  ab = max(ab, dpp_u32<kQuadXor1>(ab));
  ab = max(ab, dpp_u32<kQuadXor2>(ab));
  ab = max(ab, dpp_u32<kHalfRowMirror>(ab));  // lane i <-> 7 - i: the other quad
  return __uint_as_float(ab);
}

// One lane's share of a group: its 8 values in, its 8 nibbles and the
// group's scale out.  The 8 lanes of a group are consecutive and aligned.
COLI_DEV void quantize_chunk(const float v[8], uint32_t &packed, uint16_t &s16_out) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  a = max8(a);
  const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(a, 7.0f));
  const float sf = f16_to_f32(s16);
  packed = 0;
  if (sf != 0.0f) {
    // q2 = fl(w / h) with h = sf / 2 (exact) is 2 fl(w / sf), exactly:
    // scaling by 2 commutes with rounding away from the subnormal range, and
    // a quotient that small is code 0 either way.
    // The division is IEEE division by the group's one divisor with the
    // divisor-only part done once: the hardware reciprocal refined by one
    // Newton step, then per value a product and two exact-residual
    // corrections, each fma rounding to nearest.  These are the steps of
    // gfx9's correctly rounded fp32 division (v_div_scale / v_div_fmas /
    // v_div_fixup) with its range scaling and special-case fix-up left out.
    // Neither can change a code here: h is a normal fp32 number in
    // [2^-25, 32752], the inputs are finite, and scaling only occurs for a
    // numerator below about 2^-100, whose quotient rounds to code 0 anyway.
    const float h = 0.5f * sf;
    const float y0 = __builtin_amdgcn_rcpf(h);
    const float y = fmaf(fmaf(-h, y0, 1.0f), y0, y0);
    //
    // Rounding half away from zero, in integers: with t = trunc(2q),
    // q >= 0 gives r = floor(q + 1/2) = floor((t + 1) / 2) and q < 0 gives
    // r = -floor(|q| + 1/2) = floor(t / 2), i.e. r = (t + 1 + [t < 0]*-1)
    // >> 1 with an arithmetic shift.  r is nondecreasing in t, so clamping t
    // to [-16, 14] clamps r to [-8, 7].  u = r + 8 in [0, 15] is the offset
    // code; u ^ 8 is r's two's-complement nibble, applied to all eight
    // nibbles at once.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q2 = v[i] * y;
      q2 = fmaf(fmaf(-h, q2, v[i]), y, q2);
      q2 = fmaf(fmaf(-h, q2, v[i]), y, q2);
      int t = (int)q2;
      t = max(-16, min(14, t));
      const uint32_t u = (uint32_t)(t + 17 + (t >> 31)) >> 1;
      packed |= u << (4 * i);  // even k in the low nibble
    }
    packed ^= 0x88888888u;
  }
  s16_out = s16;
}

// int8 gs64: the same rule with 127 and byte codes.  Division and rounding
// as in quantize_chunk (round half away from zero from t = trunc(2q), where
// clamping t to [-256, 254] clamps the code to [-128, 127]).
COLI_DEV void quantize_chunk8(const float v[8], uint32_t &lo, uint32_t &hi,
                              uint16_t &s16_out) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
  a = max8(a);
  const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(a, 127.0f));
  const float sf = f16_to_f32(s16);
  uint32_t b[2] = {0u, 0u};
  if (sf != 0.0f) {
    const float h = 0.5f * sf;
    const float y0 = __builtin_amdgcn_rcpf(h);
    const float y = fmaf(fmaf(-h, y0, 1.0f), y0, y0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q2 = v[i] * y;
      q2 = fmaf(fmaf(-h, q2, v[i]), y, q2);
      q2 = fmaf(fmaf(-h, q2, v[i]), y, q2);
      int t = (int)q2;
      t = max(-256, min(254, t));
      const int r = (t + 1 + (t >> 31)) >> 1;
      b[i >> 2] |= (uint32_t)(r & 0xff) << (8 * (i & 3));
    }
  }
  lo = b[0];
  hi = b[1];
  s16_out = s16;
}

// MXFP4 (OCP MX conversion): a block of 32 is 4 consecutive lanes.  The
// shared exponent floor(log2 max|w|) - 2 is read from the maximum's fp32
// exponent field e: E8M0 byte E = max(e - 2, 0) (a subnormal or zero maximum
// gives 0).  Each value is scaled by 2^(127 - E) and becomes the nearest
// E2M1 code, ties to the even code, saturating at code 7 (6.0); the sign bit
// is the value's own, zero included.
COLI_DEV void quantize_chunk_fp4(const float v[8], uint32_t &packed, uint8_t &e_out) {
  uint32_t ab = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) ab = max(ab, __float_as_uint(v[i]) & 0x7fffffffu);
  ab = max(ab, dpp_u32<kQuadXor1>(ab));
  ab = max(ab, dpp_u32<kQuadXor2>(ab));
  const int e = (int)(ab >> 23);
  const uint32_t E = (uint32_t)max(e - 2, 0);
  const float f = __uint_as_float((254u - E) << 23);  // 2^(127 - E)
  // f is a power of two, so v * f is exact except far below the least nonzero
  // code, where only the sign survives either way.  The hardware conversion
  // (scale 1) applies exactly the rounding above to two values at a time,
  // element 2j going to the low nibble of byte j.
  uint32_t p = 0;
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[0] * f, v[1] * f, 1.0f, 0);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[2] * f, v[3] * f, 1.0f, 1);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[4] * f, v[5] * f, 1.0f, 2);
  p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(p, v[6] * f, v[7] * f, 1.0f, 3);
  packed = p;
  e_out = (uint8_t)E;
}

// Every source byte is read once and every code byte written once: both go
// through non-temporal accesses.
typedef unsigned int cv_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int cv_u32x2 __attribute__((ext_vector_type(2)));
typedef float cv_f32x4 __attribute__((ext_vector_type(4)));

COLI_DEV void load_chunk(const void *src, int src_dtype, int64_t t, float v[8]) {
  if (src_dtype == COLI_SRC_BF16) {
    const cv_u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const cv_u32x4 *>(src) + t);
    const uint32_t d[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_to_f32(d[j] & 0xffffu);
      v[2 * j + 1] = bf16_to_f32(d[j] >> 16);
    }
  } else {
    const cv_f32x4 *p = reinterpret_cast<const cv_f32x4 *>(src) + 2 * t;
    const cv_f32x4 f0 = __builtin_nontemporal_load(p), f1 = __builtin_nontemporal_load(p + 1);
    v[0] = f0.x, v[1] = f0.y, v[2] = f0.z, v[3] = f0.w;
    v[4] = f1.x, v[5] = f1.y, v[6] = f1.z, v[7] = f1.w;
  }
}

// A thread converts cpt<SRC>() chunks, kThreads apart (each step of a
// workgroup covers kThreads consecutive chunks, so the 8- or 4-lane groups
// stay whole and aligned), and requests all of their loads first: four
// 16-byte reads per lane in flight for either source type (measured: one or
// eight bf16 chunks per thread, and four fp32 chunks, were slower).
template <int SRC>
constexpr int cpt() { return SRC == COLI_SRC_BF16 ? 4 : 2; }

template <int SRC>
COLI_DEV int64_t chunk_of(int i) {
  return ((int64_t)blockIdx.x * cpt<SRC>() + i) * kThreads + threadIdx.x;
}

template <int SRC>
__global__ void __launch_bounds__(kThreads) quantize_int4_kernel(const void *__restrict__ src,
                                                                 int64_t ngroups,
                                                                 uint32_t *__restrict__ q4,
                                                                 uint16_t *__restrict__ scales) {
  float v[cpt<SRC>()][8];
#pragma unroll
  for (int i = 0; i < cpt<SRC>(); ++i)  // whole 8-lane groups are in or out together
    if ((chunk_of<SRC>(i) >> 3) < ngroups) load_chunk(src, SRC, chunk_of<SRC>(i), v[i]);
#pragma unroll
  for (int i = 0; i < cpt<SRC>(); ++i) {
    const int64_t t = chunk_of<SRC>(i);
    if ((t >> 3) >= ngroups) continue;
    uint32_t packed;
    uint16_t s16;
    quantize_chunk(v[i], packed, s16);
    __builtin_nontemporal_store(packed, q4 + t);
    if ((t & 7) == 0) scales[t >> 3] = s16;
  }
}

template <int SRC>
__global__ void __launch_bounds__(kThreads) quantize_int8_kernel(const void *__restrict__ src,
                                                                 int64_t ngroups,
                                                                 uint2 *__restrict__ q,
                                                                 uint16_t *__restrict__ scales) {
  float v[cpt<SRC>()][8];
#pragma unroll
  for (int i = 0; i < cpt<SRC>(); ++i)
    if ((chunk_of<SRC>(i) >> 3) < ngroups) load_chunk(src, SRC, chunk_of<SRC>(i), v[i]);
#pragma unroll
  for (int i = 0; i < cpt<SRC>(); ++i) {
    const int64_t t = chunk_of<SRC>(i);
    if ((t >> 3) >= ngroups) continue;
    uint32_t lo, hi;
    uint16_t s16;
    quantize_chunk8(v[i], lo, hi, s16);
    __builtin_nontemporal_store(cv_u32x2{lo, hi}, reinterpret_cast<cv_u32x2 *>(q) + t);
    if ((t & 7) == 0) scales[t >> 3] = s16;
  }
}

template <int SRC>
__global__ void __launch_bounds__(kThreads) quantize_mxfp4_kernel(const void *__restrict__ src,
                                                                  int64_t nblocks,
                                                                  uint32_t *__restrict__ q4,
                                                                  uint8_t *__restrict__ e8) {
  float v[cpt<SRC>()][8];
#pragma unroll
  for (int i = 0; i < cpt<SRC>(); ++i)  // whole 4-lane blocks are in or out together
    if ((chunk_of<SRC>(i) >> 2) < nblocks) load_chunk(src, SRC, chunk_of<SRC>(i), v[i]);
#pragma unroll
  for (int i = 0; i < cpt<SRC>(); ++i) {
    const int64_t t = chunk_of<SRC>(i);
    if ((t >> 2) >= nblocks) continue;
    uint32_t packed;
    uint8_t E;
    quantize_chunk_fp4(v[i], packed, E);
    __builtin_nontemporal_store(packed, q4 + t);
    if ((t & 3) == 0) e8[t >> 2] = E;
  }
}

}  // namespace

int launch_quantize_int4(const void *src, int src_dtype, int64_t n, uint8_t *q4,
                         uint16_t *scales, hipStream_t s) {
  const int64_t chunks = n / 8;
  const int c = src_dtype == COLI_SRC_BF16 ? cpt<COLI_SRC_BF16>() : cpt<COLI_SRC_F32>();
  const dim3 grid((unsigned)((chunks + kThreads * c - 1) / (kThreads * c)));
  uint32_t *q = reinterpret_cast<uint32_t *>(q4);
  if (src_dtype == COLI_SRC_BF16)
    launch_k(COLI_K_QUANTIZE_INT4, quantize_int4_kernel<COLI_SRC_BF16>, grid, dim3(kThreads),
             0, s, src, n / 64, q, scales);
  else
    launch_k(COLI_K_QUANTIZE_INT4, quantize_int4_kernel<COLI_SRC_F32>, grid, dim3(kThreads),
             0, s, src, n / 64, q, scales);
  return hip_status(hipGetLastError());
}

int launch_quantize_int8(const void *src, int src_dtype, int64_t n, int8_t *q, uint16_t *scales,
                         hipStream_t s) {
  const int64_t chunks = n / 8;
  const int c = src_dtype == COLI_SRC_BF16 ? cpt<COLI_SRC_BF16>() : cpt<COLI_SRC_F32>();
  const dim3 grid((unsigned)((chunks + kThreads * c - 1) / (kThreads * c)));
  uint2 *qq = reinterpret_cast<uint2 *>(q);
  if (src_dtype == COLI_SRC_BF16)
    launch_k(COLI_K_QUANTIZE_INT8, quantize_int8_kernel<COLI_SRC_BF16>, grid, dim3(kThreads), 0,
             s, src, n / 64, qq, scales);
  else
    launch_k(COLI_K_QUANTIZE_INT8, quantize_int8_kernel<COLI_SRC_F32>, grid, dim3(kThreads), 0,
             s, src, n / 64, qq, scales);
  return hip_status(hipGetLastError());
}

int launch_quantize_mxfp4(const void *src, int src_dtype, int64_t n, uint8_t *q4, uint8_t *e8,
                          hipStream_t s) {
  const int64_t chunks = n / 8;
  const int c = src_dtype == COLI_SRC_BF16 ? cpt<COLI_SRC_BF16>() : cpt<COLI_SRC_F32>();
  const dim3 grid((unsigned)((chunks + kThreads * c - 1) / (kThreads * c)));
  uint32_t *q = reinterpret_cast<uint32_t *>(q4);
  if (src_dtype == COLI_SRC_BF16)
    launch_k(COLI_K_QUANTIZE_MXFP4, quantize_mxfp4_kernel<COLI_SRC_BF16>, grid, dim3(kThreads),
             0, s, src, n / 32, q, e8);
  else
    launch_k(COLI_K_QUANTIZE_MXFP4, quantize_mxfp4_kernel<COLI_SRC_F32>, grid, dim3(kThreads),
             0, s, src, n / 32, q, e8);
  return hip_status(hipGetLastError());
}

}  // namespace coli
