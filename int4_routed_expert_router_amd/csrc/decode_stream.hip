// decode_stream.hip -- decode GEMVs for small batches (T <= 16).
//
// Work is cut into union slots: one expert of the batch union (or the
// shared expert) together with the tokens routed to it, whose pair-major
// h / o rows are consecutive.  A slot's rows are split into short runs (2
// gate/up row pairs or about 8 KB of down rows), one per wavefront.  A
// wavefront requests all of its weights at once, then fetches activation
// chunks and computes for each of the slot's tokens in turn, so an expert's
// weights cross HBM once per batch however many tokens chose it: many short
// independent wavefronts keep the most bytes in flight.  Gate/up stages the
// slot's activations per workgroup in LDS, up to four tokens at a time; down
// reads its chunks of each token's h directly, as gate/up wrote them.
// int4 codes become exact bf16 values 136 + q (one v_bitop3 per pair after
// a shift) and meet the activations in v_dot2_f32_bf16; each 32-chunk's bias
// 136 * sum(x) is removed before its fp16 group scale.  int8 codes (same
// container, one byte per weight) become exact bf16 values q through an
// fp32 conversion of each sign-extended byte (the codecs are in codec.h).
// Lane partials of several rows are combined with a reduce-scatter (each
// shuffle step halves the values a lane carries).  A token's arithmetic
// does not depend on the other tokens of the batch.  With I = 512, 1024 or
// 2048, down runs on the bf16 matrix cores instead (down_mfma_kernel): the
// weights dequantised the same way are the B operand and the tokens' h
// halves the A operand.  A batch of several tokens makes one launch per
// GEMV, in which each workgroup runs its slot's one-token or general code.
#include "device_common.h"
#include "codec.h"
#include "internal.h"

namespace coli {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kWaves = kThreads / 64;

// Sum NV values over groups of W lanes (W, NV powers of two, NV <= W).
// Every lane ends with the total of value value_index<NV, W>(lane).
template <int NV, int W>
COLI_DEV float reduce_scatter(float (&v)[NV], int lane) {
  int stride = W / 2;
#pragma unroll
  for (int nv = NV; nv > 1; nv >>= 1, stride >>= 1) {
    const bool upper = (lane & stride) != 0;
#pragma unroll
    for (int i = 0; i < nv / 2; ++i) {
      const float keep = upper ? v[i + nv / 2] : v[i];
      const float send = upper ? v[i] : v[i + nv / 2];
      v[i] = keep + __shfl_xor(send, stride, 64);
    }
  }
#pragma unroll
  for (; stride > 0; stride >>= 1) v[0] += __shfl_xor(v[0], stride, 64);
  return v[0];
}

template <int NV, int W>
COLI_DEV int value_index(int lane) {
  int idx = 0, stride = W / 2;
#pragma unroll
  for (int nv = NV; nv > 1; nv >>= 1, stride >>= 1)
    if (lane & stride) idx += nv / 2;
  return idx;
}

// Which slots a kernel's code computes: every slot of a one-token batch
// (kAll1); in a larger batch, the slots holding exactly one token, with the
// same single-token code (kSingles), or the others with the general code
// (kMulti).  A slot's tokens get the same arithmetic whichever launch
// computes them.
enum { kAll1 = 0, kSingles = 1, kMulti = 2 };

// Union slot `slot`: slots 0 .. S-1 are the shared expert (all T tokens, rows
// T*k + t), then one slot per routed expert of the union (counts[e] tokens,
// rows offsets[e] + i).  Token i of a slot has pair-major row pos0 + i.
// A gate/up weight quad, read once per call: a non-temporal load, so the
// stream does not displace cached lines.  (The same hint on the down
// weights made the down kernel slower, so it loads them plainly.)
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
COLI_DEV uint4 load_stream(const uint8_t *p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

struct Slot {
  int e, cnt, pos0;
  bool shared;
};
// ONE: a single-token batch, where every slot holds token 0 and the routed
// slots' rows are their offsets (no counts or pair lists to read).
template <bool ONE>
COLI_DEV Slot slot_of(const coli_moe_route_t &r, const Layer &L, int T, int slot) {
  Slot s;
  if (ONE) {
    s.shared = slot < L.S;
    s.e = s.shared ? L.E : r.union_ids[slot - L.S];
    s.cnt = 1;
    s.pos0 = s.shared ? L.k : r.offsets[s.e];
    return s;
  }
  if (slot < L.S) {
    s.e = L.E;
    s.cnt = T;
    s.pos0 = T * L.k;
    s.shared = true;
  } else {
    s.e = r.union_ids[slot - L.S];
    s.cnt = r.counts[s.e];
    s.pos0 = r.offsets[s.e];
    s.shared = false;
  }
  return s;
}
template <bool ONE>
COLI_DEV int token_of(const coli_moe_route_t &r, const Layer &L, const Slot &s, int i) {
  if (ONE) return 0;
  return s.shared ? i : r.pairs[s.pos0 + i] / L.k;
}

// Paired activations of chunk c in LDS: four 16-byte quads, stored
// quad-major so that consecutive lanes (consecutive chunks) read
// consecutive 16 bytes.
struct XChunk {
  uint32_t p[16];
};
COLI_DEV void lds_chunk(const uint4 *xs, int nch, int c, XChunk &out) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 v = xs[q * nch + c];
    out.p[4 * q] = v.x;
    out.p[4 * q + 1] = v.y;
    out.p[4 * q + 2] = v.z;
    out.p[4 * q + 3] = v.w;
  }
}

// Makes a packed weight quad opaque to the optimiser at this point.  Called
// once per token inside the token loops: otherwise the (loop-invariant)
// nibble unpacking is hoisted out of the loop, or above the activation
// staging, and the unpacked values (four times the registers of the packed
// ones) stay live across it.
COLI_DEV void opaque(uint4 &w) {
  asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
}

// The down GEMV consumes h as bf16 hi + lo halves (16 significant bits),
// already paired in the codec's order.  Row layout (I values, 4 bytes each):
// chunk c of 32 values holds 16 hi dwords then 16 lo dwords.
template <class C>
COLI_DEV void store_h_pair(float *row, int n, float h) {
  const uint32_t hi = f32_to_bf16_bits(h);
  const uint32_t lo = f32_to_bf16_bits(h - bf16_to_f32(hi));
  const int c = n >> 5;
  uint16_t *base = reinterpret_cast<uint16_t *>(row + 32 * c);
  const int half = C::half_index(n & 31);
  base[half] = (uint16_t)hi;
  base[32 + half] = (uint16_t)lo;
}

// ----------------------------------------------------------- gate / up

// H = 2048 * CPL: lane owns chunks lane + 64 i (i < CPL) of every row.  A
// wavefront computes RPW rows n of one slot for each of the slot's tokens;
// all their weights are requested at once, before the workgroup's activation
// staging, so the loads of every resident wavefront overlap.  The four
// wavefronts of a workgroup share the slot (I / RPW is a multiple of 4), so
// the staging loop and its barriers are uniform over the workgroup.  Dynamic
// LDS holds tg tokens: tg x 4 x NCH quads of paired bf16, then tg x NCH
// chunk biases.
template <int CPL, int RPW, int MODE, class C>
COLI_DEV void gateup_body(Layer L, coli_moe_route_t r, const uint16_t *__restrict__ x, int T,
                          int tg, float *__restrict__ h_out) {
  constexpr bool ONE = MODE == kAll1 || MODE == kSingles;  // one token in the slot
  constexpr int NCH = 64 * CPL;
  extern __shared__ uint4 smem[];
  float *xbias = reinterpret_cast<float *>(smem + tg * 4 * NCH);
  const int lane = threadIdx.x & 63;
  const int H = L.H, I = L.I;
  // wave-uniform: the slot lookups become scalar loads, weight bases scalar
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
  const int waves_per_slot = I / RPW;
  const int slot = wave / waves_per_slot;
  // (one token always has exactly k distinct experts: every slot is live)
  if (MODE != kAll1 && slot >= L.S + r.n_union[0]) return;  // the whole workgroup
  const Slot sl = slot_of<MODE == kAll1>(r, L, T, slot);
  if (MODE == kSingles && sl.cnt != 1) return;
  if (MODE == kMulti && sl.cnt == 1) return;
  // the slot's one token (a larger batch's single-token slot is routed: the
  // shared slot holds every token)
  const int tok1 = MODE == kSingles ? r.pairs[sl.pos0] / L.k : 0;
  const int n0 = (wave % waves_per_slot) * RPW;
  const int64_t row_bytes = C::bytes(H);
  const uint8_t *qg = L.q4 + (int64_t)sl.e * L.expert_bytes + (int64_t)n0 * row_bytes +
                      16 * C::Q * lane;
  const uint8_t *qu = qg + (int64_t)I * row_bytes;
  const uint8_t *sgb = reinterpret_cast<const uint8_t *>(L.scales + (int64_t)sl.e * L.expert_scales);
  const uint8_t *sub = reinterpret_cast<const uint8_t *>(L.scales + (int64_t)sl.e * L.expert_scales +
                                                         (int64_t)I * H / 64);
  // One token: this thread's activation chunk (c = threadIdx.x < NCH) is
  // requested before the weights, so that staging it waits for it alone
  // (the memory counter retires loads in issue order).
  uint4 xpre[4];
  if (ONE && threadIdx.x < NCH) {
    const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)tok1 * H) + 4 * threadIdx.x;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) xpre[dw] = src[dw];
  }
  uint4 wg[RPW][CPL][C::Q], wu[RPW][CPL][C::Q];
  uint16_t sg[RPW][CPL], su[RPW][CPL];
#pragma unroll
  for (int j = 0; j < RPW; ++j)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t ob = (int64_t)j * row_bytes + 1024 * C::Q * i;
#pragma unroll
      for (int q = 0; q < C::Q; ++q) {
        wg[j][i][q] = load_stream(qg + ob + 16 * q);
        wu[j][i][q] = load_stream(qu + ob + 16 * q);
      }
      sg[j][i] = C::scale_raw(sgb, n0 + j, H, lane + 64 * i);
      su[j][i] = C::scale_raw(sub, n0 + j, H, lane + 64 * i);
    }
    // a single token collapses to straight-line code, so the staging loads
  // below are issued while the weight loads are still in flight
  const int cnt = ONE ? 1 : sl.cnt;
  const int step = ONE ? 1 : tg;
#pragma unroll 1
  for (int g0 = 0; g0 < cnt; g0 += step) {
    const int nt = ONE ? 1 : min(tg, cnt - g0);
    if (g0) __syncthreads();  // the previous group's activations are consumed
    // stage x: chunk c of token g0 + ti -> four quads of paired bf16 + bias
    for (int idx = threadIdx.x; idx < nt * NCH; idx += kThreads) {
      const int ti = idx / NCH, c = idx - ti * NCH;
      const int t = token_of<ONE>(r, L, sl, g0 + ti);
      const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)t * H) + 4 * c;
      uint4 *xs = smem + ti * 4 * NCH;
      uint32_t p[16];
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        const uint4 v = ONE ? xpre[dw] : src[dw];
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        C::pairs(d, &p[4 * dw]);
        xs[dw * NCH + c] = make_uint4(p[4 * dw], p[4 * dw + 1], p[4 * dw + 2], p[4 * dw + 3]);
      }
      xbias[ti * NCH + c] = codec_bias<C>(p);
    }
    __syncthreads();
    #pragma unroll 1
    for (int ti = 0; ti < nt; ++ti) {
      // (one token: a single pass, nothing to hoist; and pinning the weight
      // registers there made the compiler copy them all, waiting for every
      // load, before the first dot product)
      if (!ONE) {
#pragma unroll
        for (int j = 0; j < RPW; ++j)
#pragma unroll
          for (int i = 0; i < CPL; ++i)
#pragma unroll
            for (int q = 0; q < C::Q; ++q) {
              opaque(wg[j][i][q]);
              opaque(wu[j][i][q]);
            }
      }
      const uint4 *xs = smem + ti * 4 * NCH;
      float v[2 * RPW];
#pragma unroll
      for (int j = 0; j < 2 * RPW; ++j) v[j] = 0.0f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        XChunk xc;
        lds_chunk(xs, NCH, lane + 64 * i, xc);
        const float nb = xbias[ti * NCH + lane + 64 * i];
#pragma unroll
        for (int j = 0; j < RPW; ++j) {
          v[2 * j] = fmaf(C::scale(sg[j][i]), C::template dot<false>(wg[j][i], xc.p, xc.p, nb),
                          v[2 * j]);
          v[2 * j + 1] = fmaf(C::scale(su[j][i]),
                              C::template dot<false>(wu[j][i], xc.p, xc.p, nb), v[2 * j + 1]);
        }
      }
      // value 2j is the gate of row j, 2j+1 its up; bring them to one lane
      const float tot = reduce_scatter<2 * RPW, 64>(v, lane);
      const int vi = value_index<2 * RPW, 64>(lane);
      constexpr int kSpan = 64 / (2 * RPW);  // lanes holding one value
      const float up = __shfl_down(tot, kSpan, 64);
      if ((lane % kSpan) == 0 && (vi & 1) == 0)
        store_h_pair<C>(h_out + (int64_t)(sl.pos0 + g0 + ti) * I, n0 + vi / 2, silu_mul(tot, up));
    }
  }
}

template <int CPL, int RPW, int MODE, class C>
__global__ void __launch_bounds__(kThreads) gateup_stream_kernel(
    Layer L, coli_moe_route_t r, const uint16_t *__restrict__ x, int T, int tg,
    float *__restrict__ h_out) {
  gateup_body<CPL, RPW, MODE, C>(L, r, x, T, tg, h_out);
}

// Every slot of a batch of several tokens in one launch: a workgroup whose
// slot holds one token runs the one-token code, the others the general code
// (each slot's arithmetic is that of the launch mode of its own code).
template <int CPL, int RPW, class C>
__global__ void __launch_bounds__(kThreads) gateup_mixed_kernel(
    Layer L, coli_moe_route_t r, const uint16_t *__restrict__ x, int T, int tg,
    float *__restrict__ h_out) {
  const int slot = blockIdx.x * kWaves / (L.I / RPW);  // the workgroup's slot
  if (slot >= L.S + r.n_union[0]) return;
  if (slot >= L.S && r.counts[r.union_ids[slot - L.S]] == 1)
    gateup_body<CPL, RPW, kSingles, C>(L, r, x, T, tg, h_out);
  else
    gateup_body<CPL, RPW, kMulti, C>(L, r, x, T, tg, h_out);
}

// ------------------------------------------------------------------ down

// K = I: LPR lanes per row (LPR = I/32 when I < 2048, else 64 with CPL
// chunks each); RPI = 64/LPR rows share a wave instruction; a wavefront
// computes RG such row groups (RPI * RG rows m) of one slot, for each of the
// slot's tokens with the same weights in registers.  Each lane reads its
// chunks of the token's h (hi + lo pairs, written by gate/up).  The four
// wavefronts of a workgroup share the slot (H / RPW is a multiple of 4).
// One token: the workgroup requests the token's h row before the weights,
// stages it in LDS quad-major (quad q of chunk c at q * I/32 + c, so a
// wavefront's reads are consecutive), and its wavefronts read it from there.
template <int LPR, int CPL, int RG, bool ONE, class C>
__global__ void __launch_bounds__(kThreads) down_stream_kernel(
    Layer L, coli_moe_route_t r, int T, const float *__restrict__ h_in,
    float *__restrict__ o_out) {
  constexpr int RPI = 64 / LPR;
  constexpr int RPW = RPI * RG;
  constexpr int NCHK = LPR * CPL;               // 32-value chunks of an h row (I / 32)
  constexpr int NQ = 8 * NCHK;                  // 16-byte quads of an h row
  constexpr int HPT = (NQ + kThreads - 1) / kThreads;
  __shared__ uint4 hsm[ONE ? NQ : 1];
  const int lane = threadIdx.x & 63;
  const int lr = lane / LPR, lc = lane % LPR;
  const int H = L.H, I = L.I;
  const int wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6));
  const int waves_per_slot = H / RPW;
  const int slot = wave / waves_per_slot;
  if (!ONE && slot >= L.S + r.n_union[0]) return;
  const Slot sl = slot_of<ONE>(r, L, T, slot);
  const int m0 = (wave % waves_per_slot) * RPW;
  uint4 hpre[HPT];
  if (ONE) {
    const uint4 *src = reinterpret_cast<const uint4 *>(h_in + (int64_t)sl.pos0 * I);
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
      const int qi = threadIdx.x + kThreads * j;
      if (NQ % kThreads == 0 || qi < NQ) hpre[j] = src[qi];
    }
  }
  const int64_t row_bytes = C::bytes(I);
  const uint8_t *qd = L.q4 + (int64_t)sl.e * L.expert_bytes + C::bytes((int64_t)2 * I * H) +
                      (int64_t)(m0 + lr) * row_bytes + 16 * C::Q * lc;
  const uint8_t *sdb = reinterpret_cast<const uint8_t *>(
      L.scales + (int64_t)sl.e * L.expert_scales + (int64_t)2 * I * H / 64);
  uint4 w[RG][CPL][C::Q];
  uint16_t sc[RG][CPL];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t row = RPI * j;
#pragma unroll
      for (int q = 0; q < C::Q; ++q)
        w[j][i][q] = *reinterpret_cast<const uint4 *>(qd + row * row_bytes + 16 * C::Q * LPR * i +
                                                      16 * q);
      sc[j][i] = C::scale_raw(sdb, m0 + lr + row, I, lc + LPR * i);
    }
  if (ONE) {
#pragma unroll
    for (int j = 0; j < HPT; ++j) {
      const int qi = threadIdx.x + kThreads * j;
      if (NQ % kThreads == 0 || qi < NQ) hsm[(qi & 7) * NCHK + (qi >> 3)] = hpre[j];
    }
    __syncthreads();
  }
  const int cnt = ONE ? 1 : sl.cnt;
#pragma unroll 1
  for (int ti = 0; ti < cnt; ++ti) {
    if (!ONE) {
#pragma unroll
      for (int j = 0; j < RG; ++j)
#pragma unroll
        for (int i = 0; i < CPL; ++i)
#pragma unroll
          for (int q = 0; q < C::Q; ++q) opaque(w[j][i][q]);
    }
    const int64_t pos = sl.pos0 + ti;
    float v[RG];
#pragma unroll
    for (int j = 0; j < RG; ++j) v[j] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lc + LPR * i;
      const uint4 *src = reinterpret_cast<const uint4 *>(h_in + pos * I + 32 * c);
      XChunk hi, lo;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 a = ONE ? hsm[q * NCHK + c] : src[q];
        const uint4 b = ONE ? hsm[(4 + q) * NCHK + c] : src[4 + q];
        hi.p[4 * q] = a.x, hi.p[4 * q + 1] = a.y, hi.p[4 * q + 2] = a.z, hi.p[4 * q + 3] = a.w;
        lo.p[4 * q] = b.x, lo.p[4 * q + 1] = b.y, lo.p[4 * q + 2] = b.z, lo.p[4 * q + 3] = b.w;
      }
      const float nb = codec_bias2<C>(hi.p, lo.p);
#pragma unroll
      for (int j = 0; j < RG; ++j)
        v[j] = fmaf(C::scale(sc[j][i]), C::template dot<true>(w[j][i], hi.p, lo.p, nb), v[j]);
    }
    const float tot = reduce_scatter<RG, LPR>(v, lc);
    constexpr int kSpan = LPR / RG;
    if ((lc % kSpan) == 0)
      o_out[pos * H + m0 + lr + RPI * value_index<RG, LPR>(lc)] = tot;
  }
}

// ------------------------------------------------- down on the matrix cores

// I = 2048.  The down GEMV as v_mfma_f32_16x16x32_bf16 products: the weights
// are the B operand (its 16 columns are 16 output rows m), the slot's tokens
// the A operand, token t's h as two rows -- 2t its high bf16 half, 2t + 1 its
// low half -- so one instruction covers both halves of up to 8 tokens (NA =
// 2 operand tiles for 9..16).  Lane l supplies the eight k values 8 (l / 16)
// .. + 7 of a 32-value chunk for row / column l % 16 of each operand.
//
// A workgroup computes TPW tiles of 16 rows of one slot; wavefront w takes
// k in [512 w, 512 w + 512).  A lane's 16-byte load holds 32 nibbles of one
// row (int4, MXFP4: one chunk; int8: half of one), so lane groups g = 0..3
// load consecutive 16-byte pieces and four permlane swaps transpose them into
// per-chunk operands.  Per 64-weight group (int4, int8; per 32 for MXFP4)
// the accumulator starts from the nibble bias -136 sum(a) (int4) and is
// scaled into the running sums; the four wavefronts' sums are added in LDS
// in a fixed order.  A token's arithmetic is the same in any batch.
typedef __bf16 coli_bf16x8 __attribute__((ext_vector_type(8)));
typedef float coli_f32x4 __attribute__((ext_vector_type(4)));

COLI_DEV void swap32(uint32_t &x, uint32_t &y) {
  const auto p = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = p[0];
  y = p[1];
}
COLI_DEV void swap16(uint32_t &x, uint32_t &y) {
  const auto p = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = p[0];
  y = p[1];
}
COLI_DEV coli_bf16x8 as_bf16x8(const uint32_t p[4]) {
  const uint4 v = make_uint4(p[0], p[1], p[2], p[3]);
  return __builtin_bit_cast(coli_bf16x8, v);
}

// k per wavefront: I / 4 (I = 512, 1024 or 2048)
template <int KW>
constexpr bool mfma_kw_ok() { return KW == 128 || KW == 256 || KW == 512; }

// Activation quad q (0..3 high half, 4..7 low half) of chunk c of A row a:
// from the LDS copy of the token's h row (one token) or from h itself (A row
// a is slot token min(a / 2, cnt - 1); rows past the slot's tokens repeat
// the last one, and their products are not used).
template <bool ONE, int NCHK>
COLI_DEV uint4 mfma_a_quad(const uint4 *hsm, const float *__restrict__ h_in, int pos0, int cnt,
                           int I, int a, int c, int q) {
  if (ONE) return hsm[q * NCHK + c];
  const int tok = min(a >> 1, cnt - 1);
  return reinterpret_cast<const uint4 *>(h_in + (int64_t)(pos0 + tok) * I + 32 * c)[q];
}

// 16-row tiles per wavefront: about eight 16-byte weight loads per lane
// (two tiles of 512 k with int4 codes, four of 256 or 128 k; half with int8)
template <class C, int KW>
constexpr int mfma_tpw() { return (KW == 512 ? 2 : 4) / C::Q; }

template <int NA, int MODE, class C, int KW>
COLI_DEV void down_mfma_body(Layer L, coli_moe_route_t r, int T, const float *__restrict__ h_in,
                             float *__restrict__ o_out) {
  static_assert(mfma_kw_ok<KW>(), "k per wavefront");
  constexpr bool ONE = MODE == kAll1 || MODE == kSingles;  // one token in the slot
  constexpr int TPW = mfma_tpw<C, KW>();
  constexpr int NCHK = KW / 8;                 // chunks of an h row (I / 32)
  constexpr int CPW = KW / 32;                 // chunks per wavefront
  constexpr int LPT = CPW * C::Q / 4;          // 16-byte loads per tile (int8: 8, else 4)
  constexpr int CPL = 4 / C::Q;                // chunks per load
  constexpr int CPS = C::kChunksPerScale;      // chunks sharing one scale
  constexpr int ROWS = 16 * NA;                // A rows
  constexpr bool kHasBias = C::kBias != 0.0f;
  constexpr int UNITS = kHasBias ? NCHK / 2 : 1;  // 64-value bias groups of a row
  // bias table: per group, the A rows (one token: [hi, lo, hi, lo], which is
  // what every lane group reads, since its A rows all repeat the token)
  constexpr int BROWS = ONE ? 4 : ROWS;
  __shared__ uint4 hsm[ONE ? 8 * NCHK : 1];
  __shared__ __align__(16) float bias_sm[UNITS * BROWS];
  __shared__ float red[kWaves * TPW * NA * 64 * 2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int g = lane >> 4, rr = lane & 15;
  const int H = L.H, I = L.I;
  const int wg_per_slot = H / (16 * TPW);
  const int slot = blockIdx.x / wg_per_slot;
  if (MODE != kAll1 && slot >= L.S + r.n_union[0]) return;  // the whole workgroup
  const Slot sl = slot_of<MODE == kAll1>(r, L, T, slot);
  if (MODE == kSingles && sl.cnt != 1) return;
  if (MODE == kMulti && sl.cnt == 1) return;
  const int cnt = ONE ? 1 : sl.cnt;
  const int m0 = (blockIdx.x % wg_per_slot) * (16 * TPW);
  const int k0 = wv * KW;
  // one token: the h row (I / 4 quads: 2 per thread at I = 2048), requested
  // before the weights
  constexpr int HQ = KW;  // 16-byte quads of an h row (hi + lo bf16 pairs)
  constexpr int HPT = (HQ + kThreads - 1) / kThreads;
  uint4 hp[HPT];
  if (ONE) {
    const uint4 *src = reinterpret_cast<const uint4 *>(h_in + (int64_t)sl.pos0 * I);
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int q = threadIdx.x + i * kThreads;
      hp[i] = q < HQ ? src[q] : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  // weights: tile t, load j holds bytes 64 j + 16 g of row m0 + 16 t + rr
  // within the wavefront's k range
  const int64_t row_bytes = C::bytes(I);
  const uint8_t *qd = L.q4 + (int64_t)sl.e * L.expert_bytes + C::bytes((int64_t)2 * I * H) +
                      (int64_t)(m0 + rr) * row_bytes + C::bytes(k0) + 16 * g;
  uint4 w[TPW][LPT];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int j = 0; j < LPT; ++j)
      w[t][j] = *reinterpret_cast<const uint4 *>(qd + (int64_t)16 * t * row_bytes + 64 * j);
  // the scales of the wavefront's CPW chunks of the row: KW / 32 bytes (one
  // fp16 per two chunks, or one E8M0 per chunk), exactly what is needed
  const uint8_t *sdb = reinterpret_cast<const uint8_t *>(
      L.scales + (int64_t)sl.e * L.expert_scales + (int64_t)2 * I * H / 64);
  uint4 sc[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int64_t row = m0 + 16 * t + rr;
    const int64_t off = CPS == 2 ? 2 * (row * (I / 64) + k0 / 64) : row * (I / 32) + k0 / 32;
    if (KW == 512) {
      sc[t] = *reinterpret_cast<const uint4 *>(sdb + off);
    } else if (KW == 256) {
      const uint2 v = *reinterpret_cast<const uint2 *>(sdb + off);
      sc[t] = make_uint4(v.x, v.y, 0u, 0u);
    } else {
      sc[t] = make_uint4(*reinterpret_cast<const uint32_t *>(sdb + off), 0u, 0u, 0u);
    }
  }
  if (ONE) {
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      const int q = threadIdx.x + i * kThreads;
      if (q < HQ) hsm[(q & 7) * NCHK + (q >> 3)] = hp[i];
    }
    __syncthreads();
  }
  if (kHasBias) {
    // -136 * (sum of A row a over group u), chunk 2u then 2u + 1, in order;
    // rows past the slot's tokens are not used and get 0
    for (int idx = threadIdx.x; idx < UNITS * BROWS; idx += kThreads) {
      const int u = idx / BROWS, a = idx - u * BROWS;
      if (ONE ? a >= 2 : a >= 2 * cnt) {
        if (!ONE) bias_sm[idx] = 0.0f;
        continue;
      }
      float sum = 0.0f;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = mfma_a_quad<ONE, NCHK>(hsm, h_in, sl.pos0, cnt, I, a, 2 * u + h, 4 * (a & 1) + q);
          sum = dot2_bf16(v.x, kBf16Ones, sum);
          sum = dot2_bf16(v.y, kBf16Ones, sum);
          sum = dot2_bf16(v.z, kBf16Ones, sum);
          sum = dot2_bf16(v.w, kBf16Ones, sum);
        }
      bias_sm[idx] = -(float)kNibBias * sum;
      if (ONE) bias_sm[idx + 2] = -(float)kNibBias * sum;
    }
    __syncthreads();
  }
  coli_f32x4 acc[TPW][NA], d[TPW][NA];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[t][a] = coli_f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    uint32_t dw[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      dw[t][0] = w[t][j].x, dw[t][1] = w[t][j].y, dw[t][2] = w[t][j].z, dw[t][3] = w[t][j].w;
      if (C::Q == 1) {  // lane group g held chunk g: now dword b holds chunk b
        swap32(dw[t][0], dw[t][2]);
        swap32(dw[t][1], dw[t][3]);
        swap16(dw[t][0], dw[t][1]);
        swap16(dw[t][2], dw[t][3]);
      } else {  // group g held half g & 1 of chunk g >> 1: now dwords 2b, 2b + 1
        swap16(dw[t][0], dw[t][2]);  // hold k group g of chunk b
        swap16(dw[t][1], dw[t][3]);
        swap32(dw[t][0], dw[t][2]);
        swap32(dw[t][1], dw[t][3]);
      }
    }
#pragma unroll
    for (int b = 0; b < CPL; ++b) {
      const int cw = j * CPL + b;  // chunk within the wavefront's range
      const int c = k0 / 32 + cw;  // chunk within the row
#pragma unroll
      for (int a = 0; a < NA; ++a) {
        // the chunk's activations (and its group's bias) serve every tile
        const int arow = 16 * a + rr;
        const uint4 av = mfma_a_quad<ONE, NCHK>(hsm, h_in, sl.pos0, cnt, I, arow, c,
                                                4 * (arow & 1) + g);
        const uint32_t ap[4] = {av.x, av.y, av.z, av.w};
        const coli_bf16x8 aop = as_bf16x8(ap);
        coli_f32x4 cin = coli_f32x4{0.f, 0.f, 0.f, 0.f};
        if (kHasBias && cw % CPS == 0) {
          const float4 bv = *reinterpret_cast<const float4 *>(
              &bias_sm[(c >> 1) * BROWS + (ONE ? 0 : 16 * a + 4 * g)]);
          cin = coli_f32x4{bv.x, bv.y, bv.z, bv.w};
        }
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
          uint32_t bp[4];
          C::kgroup(dw[t] + C::Q * b, bp);
          if (cw % CPS == 0) d[t][a] = cin;
          d[t][a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aop, as_bf16x8(bp), d[t][a], 0, 0, 0);
          if (cw % CPS == CPS - 1) {
            const uint32_t sd[4] = {sc[t].x, sc[t].y, sc[t].z, sc[t].w};
            const float sv = C::scale(C::scale_at(sd, cw));
#pragma unroll
            for (int v = 0; v < (ONE ? 2 : 4); ++v)  // one token: rows 0, 1 are used
              acc[t][a][v] = fmaf(sv, d[t][a][v], acc[t][a][v]);
          }
        }
      }
    }
    // keeps each load's operand reads (LDS) next to its products, so the
    // scheduler does not hold every chunk's operands in registers at once
    asm volatile("" ::: "memory");
  }
  // lane (g, rr), value v: A row 16 a + 4 g + v, output row m0 + 16 t + rr;
  // rows 2i and 2i + 1 are the halves of slot token i = 8 a + 2 g + v / 2
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int a = 0; a < NA; ++a) {
      float *dst = red + ((wv * TPW + t) * NA + a) * 128 + 2 * lane;
      dst[0] = acc[t][a][0] + acc[t][a][1];
      if (!ONE) dst[1] = acc[t][a][2] + acc[t][a][3];  // one token: not read
    }
  __syncthreads();
  // the four wavefronts' sums, in wavefront order
  for (int idx = threadIdx.x; idx < TPW * 16 * cnt; idx += kThreads) {
    const int i = idx / (TPW * 16), rem = idx - i * (TPW * 16);
    const int t = rem >> 4, row = rem & 15;
    const int a = i >> 3, gi = (i & 7) >> 1, vi = i & 1;
    const int off = (t * NA + a) * 128 + 2 * (16 * gi + row) + vi;
    float v = red[off];
#pragma unroll
    for (int w2 = 1; w2 < kWaves; ++w2) v += red[w2 * TPW * NA * 128 + off];
    o_out[(int64_t)(sl.pos0 + i) * H + m0 + 16 * t + row] = v;
  }
}

template <int NA, int MODE, class C, int KW>
__global__ void __launch_bounds__(kThreads) down_mfma_kernel(
    Layer L, coli_moe_route_t r, int T, const float *__restrict__ h_in,
    float *__restrict__ o_out) {
  down_mfma_body<NA, MODE, C, KW>(L, r, T, h_in, o_out);
}

// Every slot of a batch of several tokens in one launch, as for gate/up
template <int NA, class C, int KW>
__global__ void __launch_bounds__(kThreads) down_mfma_mixed_kernel(
    Layer L, coli_moe_route_t r, int T, const float *__restrict__ h_in,
    float *__restrict__ o_out) {
  const int slot = blockIdx.x / (L.H / (16 * mfma_tpw<C, KW>()));  // the workgroup's slot
  if (slot >= L.S + r.n_union[0]) return;
  if (slot >= L.S && r.counts[r.union_ids[slot - L.S]] == 1)
    down_mfma_body<1, kSingles, C, KW>(L, r, T, h_in, o_out);
  else
    down_mfma_body<NA, kMulti, C, KW>(L, r, T, h_in, o_out);
}

constexpr int kMaxStage = 4;  // tokens of one slot staged in LDS at once

// gate/up rows per wavefront: two with int4 codes, one with int8 codes
// (the same weight registers either way)
template <class C>
constexpr int gateup_rpw() { return C::Q == 1 ? 2 : 1; }

template <int CPL, class C>
hipError_t gateup_cpl(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                      float *h, int nslots, hipStream_t s) {
  constexpr int RPW = gateup_rpw<C>();
  const int waves = nslots * (L.I / RPW);
  // up to kMaxStage tokens per LDS stage, within 64 KB
  const size_t per_token = (size_t)64 * CPL * (4 * sizeof(uint4) + sizeof(float));
  int tg = T < kMaxStage ? T : kMaxStage;
  while (tg > 1 && tg * per_token > 65536) --tg;
  const size_t lds = tg * per_token;
  const dim3 grid((waves + kWaves - 1) / kWaves);
  if (T == 1)
    launch_k(COLI_K_DECODE_GATEUP, gateup_stream_kernel<CPL, RPW, kAll1, C>, grid,
             dim3(kThreads), lds, s, L, r, x, T, tg, h);
  else  // one launch, each workgroup with its slot's code
    launch_k(COLI_K_DECODE_GATEUP, gateup_mixed_kernel<CPL, RPW, C>, grid, dim3(kThreads), lds, s,
             L, r, x, T, tg, h);
  return hipGetLastError();
}

// row groups per wavefront of the down GEMV: about eight 16-byte loads per
// lane (8 rows of 1 KB of int4 codes when I = 2048; half the rows for int8)
template <int LPR, int CPL, class C>
constexpr int down_rg() {
  return (CPL == 1 ? 8 : (CPL == 2 ? 4 : 2)) / C::Q;
}
template <int LPR, int CPL, class C>
constexpr int down_rows_wave() { return (64 / LPR) * down_rg<LPR, CPL, C>(); }

template <int LPR, int CPL, class C>
hipError_t down_shape(const Layer &L, const coli_moe_route_t &r, int T, const float *h,
                      float *o, int nslots, hipStream_t s) {
  const int waves = nslots * (L.H / down_rows_wave<LPR, CPL, C>());
  const dim3 grid((waves + kWaves - 1) / kWaves);
  constexpr int RG = down_rg<LPR, CPL, C>();
  if (T == 1)
    launch_k(COLI_K_DECODE_DOWN, down_stream_kernel<LPR, CPL, RG, true, C>, grid, dim3(kThreads),
             0, s, L, r, T, h, o);
  else
    launch_k(COLI_K_DECODE_DOWN, down_stream_kernel<LPR, CPL, RG, false, C>, grid,
             dim3(kThreads), 0, s, L, r, T, h, o);
  return hipGetLastError();
}

// I = 4 * KW (512, 1024, 2048): the down GEMV on the matrix cores, NA
// operand tiles of 8 tokens
template <class C, int KW>
hipError_t down_mfma(const Layer &L, const coli_moe_route_t &r, int T, const float *h, float *o,
                     int nslots, hipStream_t s) {
  const dim3 grid(nslots * (L.H / (16 * mfma_tpw<C, KW>())));
  if (T == 1) {
    launch_k(COLI_K_DECODE_DOWN, down_mfma_kernel<1, kAll1, C, KW>, grid, dim3(kThreads), 0, s,
             L, r, T, h, o);
    return hipGetLastError();
  }
  // one launch, each workgroup with its slot's code
  if (T <= 8)
    launch_k(COLI_K_DECODE_DOWN, down_mfma_mixed_kernel<1, C, KW>, grid, dim3(kThreads), 0, s, L,
             r, T, h, o);
  else
    launch_k(COLI_K_DECODE_DOWN, down_mfma_mixed_kernel<2, C, KW>, grid, dim3(kThreads), 0, s, L,
             r, T, h, o);
  return hipGetLastError();
}

// Shape of the streaming path for this layer, or false if it has none.
template <class C>
bool stream_shape(const Layer &L, int &lpr, int &cpl) {
  const int hc = L.H / 2048;
  if (L.H % 2048 || hc < 1 || hc > 4) return false;
  int rows_wave;
  if (L.I == 512) {
    lpr = 16, cpl = 1, rows_wave = down_rows_wave<16, 1, C>();
  } else if (L.I == 1024) {
    lpr = 32, cpl = 1, rows_wave = down_rows_wave<32, 1, C>();
  } else if (L.I % 2048 == 0 && L.I / 2048 <= 4) {
    lpr = 64, cpl = L.I / 2048;
    rows_wave = cpl == 1 ? down_rows_wave<64, 1, C>() : cpl == 2 ? down_rows_wave<64, 2, C>()
                : cpl == 3 ? down_rows_wave<64, 3, C>() : down_rows_wave<64, 4, C>();
  } else {
    return false;
  }
  return L.I % 8 == 0 && L.H % rows_wave == 0;
}

template <class C>
bool launch_stream(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                   float *h, float *o, hipStream_t s, hipError_t *err) {
  int lpr, cpl;
  if (T > kMaxStreamT || !stream_shape<C>(L, lpr, cpl)) return false;
  const int nslots = max_union(L, T) + L.S;
  hipError_t e = hipSuccess;
  switch (L.H / 2048) {
    case 1: e = gateup_cpl<1, C>(L, r, x, T, h, nslots, s); break;
    case 2: e = gateup_cpl<2, C>(L, r, x, T, h, nslots, s); break;
    case 3: e = gateup_cpl<3, C>(L, r, x, T, h, nslots, s); break;
    default: e = gateup_cpl<4, C>(L, r, x, T, h, nslots, s); break;
  }
  if (e == hipSuccess) {
    if (lpr == 16) e = down_mfma<C, 128>(L, r, T, h, o, nslots, s);
    else if (lpr == 32) e = down_mfma<C, 256>(L, r, T, h, o, nslots, s);
    else if (cpl == 1) e = down_mfma<C, 512>(L, r, T, h, o, nslots, s);
    else if (cpl == 2) e = down_shape<64, 2, C>(L, r, T, h, o, nslots, s);
    else if (cpl == 3) e = down_shape<64, 3, C>(L, r, T, h, o, nslots, s);
    else e = down_shape<64, 4, C>(L, r, T, h, o, nslots, s);
  }
  *err = e;
  return true;
}

}  // namespace

// Launches gate/up and down for T <= kMaxStreamT tokens when the shape has a
// streaming path (H a multiple of 2048 up to 8192; I in {512, 1024} or a
// multiple of 2048 up to 8192; H a multiple of a down wavefront's rows).
// Returns false, launching nothing, otherwise.
bool launch_decode_stream(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                          float *h, float *o, hipStream_t s, hipError_t *err) {
  if (L.f4) return launch_stream<CodecF4>(L, r, x, T, h, o, s, err);
  return L.w8 ? launch_stream<CodecI8>(L, r, x, T, h, o, s, err)
              : launch_stream<CodecI4>(L, r, x, T, h, o, s, err);
}

}  // namespace coli
