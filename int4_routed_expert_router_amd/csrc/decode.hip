// decode.hip -- decode / verify forward (T <= 64): int4-dequant GEMVs.
//
// Each distinct expert of the batch union is streamed from HBM once per call
// (tantan.ink post on colibri, section "几个关键工程动作": the batch reads a
// deduplicated expert once; gate/up/down adjacent).  The three steps:
//
//  gateup : work item = (union slot, block of rows n).  Every lane streams
//           16-byte chunks (32 nibbles) of gate row n and up row n with
//           coalesced dwordx4 loads, turns nibbles into exact bf16 values
//           (136 + q) with three bit operations per pair, and accumulates
//           v_dot2_f32_bf16 products against the token's bf16 activations,
//           which sit in LDS pre-paired to the nibble order.  The 136*sum(x)
//           bias of each 32-chunk is removed before the fp16 group scale is
//           applied.  Lane partials are reduced across the row's lanes and
//           h = silu(g) * u is written as fp32 [pair row][I].
//  down   : the same stream over W_down rows m; the fp32 h of each token is
//           split into bf16 hi + lo halves (16 significant bits) so the bf16
//           dot keeps fp32-level accuracy.  Writes o fp32 [pair row][H].
//  combine: y[t] = sum_j w[t,j] * o[row of pair (t,j)] + o[shared row t], in
//           a fixed order, rounded to bf16 (or stored fp32).
// A token's output depends only on its own rows, so results are independent
// of the other tokens in the batch, and there are no atomics.
#include "device_common.h"
#include "codec.h"
#include "internal.h"

namespace coli {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kMaxDecodeT = 64;

// Work description of one union slot: expert id and its token rows.
struct SlotInfo {
  int expert;
  int ntok;
  int pos[kMaxDecodeT];  // pair-major row of each token's h / o
  int tok[kMaxDecodeT];  // token index
};

// Fill `si` for slot `slot` (slot 0 is the shared expert when S == 1).
// Returns false when the slot is past the batch union.
__device__ bool load_slot(const coli_moe_route_t &r, int slot, int T, int k, int E, int S,
                          SlotInfo &si) {
  const int P = T * k;
  if (S && slot == 0) {
    if (threadIdx.x == 0) {
      si.expert = E;
      si.ntok = T;
    }
    for (int i = threadIdx.x; i < T; i += kThreads) {
      si.pos[i] = P + i;
      si.tok[i] = i;
    }
    return true;
  }
  const int u = slot - S;
  if (u >= r.n_union[0]) return false;
  const int e = r.union_ids[u];
  const int beg = r.offsets[e], cnt = r.counts[e];
  if (threadIdx.x == 0) {
    si.expert = e;
    si.ntok = cnt;
  }
  for (int i = threadIdx.x; i < cnt; i += kThreads) {
    si.pos[i] = beg + i;
    si.tok[i] = r.pairs[beg + i] / k;
  }
  return true;
}

// ------------------------------------------------------------- gate / up

// LPR lanes share one row; CPL = chunks per lane (0: runtime loop);
// TG tokens per pass.  Rows per work item: 4 waves * 2 * (64/LPR) * 2.
template <int LPR, int CPL, int TG, class C>
__global__ void __launch_bounds__(kThreads) gateup_kernel(Layer L, coli_moe_route_t r,
                                                          const uint16_t *__restrict__ x,
                                                          int T, float *__restrict__ h_out,
                                                          int nrb, int items) {
  constexpr int RPW = 64 / LPR;          // rows in flight per wave per row slot
  constexpr int ROWS_WAVE = 2 * RPW * 2; // two row slots per lane, two iterations
  constexpr int ROWS_ITEM = 4 * ROWS_WAVE;
  const int H = L.H, I = L.I, NCH = H / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SlotInfo si;
  uint4 *xs = reinterpret_cast<uint4 *>(smem);               // [TG][4][NCH]
  float *corr = reinterpret_cast<float *>(xs + TG * 4 * NCH);  // [TG][NCH]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int lr = lane / LPR, lc = lane % LPR;
  const int cpl = CPL ? CPL : (NCH + LPR - 1) / LPR;
  const int nslots = (items / nrb);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int slot = item % nslots, rb = item / nslots;
    __syncthreads();
    if (!load_slot(r, slot, T, L.k, L.E, L.S, si)) continue;
    __syncthreads();
    const int e = si.expert, ntok = si.ntok;
    const uint8_t *qg = L.q4 + (int64_t)e * L.expert_bytes;
    const uint8_t *qu = qg + C::bytes((int64_t)I * H);
    const uint8_t *sg = reinterpret_cast<const uint8_t *>(L.scales + (int64_t)e * L.expert_scales);
    const uint8_t *su =
        reinterpret_cast<const uint8_t *>(L.scales + (int64_t)e * L.expert_scales + (int64_t)I * H / 64);
    const int64_t rowb = C::bytes(H);  // bytes per weight row
    const int row_base = rb * ROWS_ITEM + wid * ROWS_WAVE;

    for (int t0 = 0; t0 < ntok; t0 += TG) {
      const int nt = min(TG, ntok - t0);
      // stage the token group's activations, paired to the nibble order
      __syncthreads();
      for (int i = threadIdx.x; i < TG * NCH; i += kThreads) {
        const int tt = i / NCH, c = i % NCH;
        float nb = 0.0f;
        if (tt < nt) {
          const uint4 *src = reinterpret_cast<const uint4 *>(x + (int64_t)si.tok[t0 + tt] * H) + 4 * c;
          uint32_t p[16];
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const uint4 v = src[dw];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            C::pairs(d, &p[4 * dw]);
            xs[(tt * 4 + dw) * NCH + c] = make_uint4(p[4 * dw], p[4 * dw + 1], p[4 * dw + 2], p[4 * dw + 3]);
          }
          nb = codec_bias<C>(p);
        }
        corr[tt * NCH + c] = -nb;
      }
      __syncthreads();

#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int ra = row_base + it * 2 * RPW + lr, rb2 = ra + RPW;
        float ga[TG], ua[TG], gb[TG], ub[TG];
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) ga[tt] = ua[tt] = gb[tt] = ub[tt] = 0.0f;
        const bool va = ra < I, vb = rb2 < I;
#pragma unroll
        for (int i = 0; i < (CPL ? CPL : 1); ++i) {
          for (int ii = i; ii < cpl; ii += (CPL ? CPL : 1)) {
            const int c = lc + LPR * ii;
            if (c >= NCH) break;
            uint4 wga[C::Q], wua[C::Q], wgb[C::Q], wub[C::Q];
#pragma unroll
            for (int q = 0; q < C::Q; ++q)
              wga[q] = wua[q] = wgb[q] = wub[q] = make_uint4(0, 0, 0, 0);
            float sga = 0.f, sua = 0.f, sgb = 0.f, sub = 0.f;
            if (va) {
#pragma unroll
              for (int q = 0; q < C::Q; ++q) {
                wga[q] = *reinterpret_cast<const uint4 *>(qg + ra * rowb + 16 * (C::Q * c + q));
                wua[q] = *reinterpret_cast<const uint4 *>(qu + ra * rowb + 16 * (C::Q * c + q));
              }
              sga = C::scale(C::scale_raw(sg, ra, H, c));
              sua = C::scale(C::scale_raw(su, ra, H, c));
            }
            if (vb) {
#pragma unroll
              for (int q = 0; q < C::Q; ++q) {
                wgb[q] = *reinterpret_cast<const uint4 *>(qg + rb2 * rowb + 16 * (C::Q * c + q));
                wub[q] = *reinterpret_cast<const uint4 *>(qu + rb2 * rowb + 16 * (C::Q * c + q));
              }
              sgb = C::scale(C::scale_raw(sg, rb2, H, c));
              sub = C::scale(C::scale_raw(su, rb2, H, c));
            }
            float aga[TG], aua[TG], agb[TG], aub[TG];
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
              const float cr = -corr[tt * NCH + c];
              aga[tt] = aua[tt] = agb[tt] = aub[tt] = cr;
            }
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
              if (TG > 1 && tt >= nt) break;
              uint32_t xp[16];
#pragma unroll
              for (int dw = 0; dw < 4; ++dw) {
                const uint4 xv = xs[(tt * 4 + dw) * NCH + c];
                xp[4 * dw] = xv.x;
                xp[4 * dw + 1] = xv.y;
                xp[4 * dw + 2] = xv.z;
                xp[4 * dw + 3] = xv.w;
              }
              aga[tt] = C::template dot<false>(wga, xp, nullptr, aga[tt]);
              aua[tt] = C::template dot<false>(wua, xp, nullptr, aua[tt]);
              agb[tt] = C::template dot<false>(wgb, xp, nullptr, agb[tt]);
              aub[tt] = C::template dot<false>(wub, xp, nullptr, aub[tt]);
            }
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
              ga[tt] = fmaf(sga, aga[tt], ga[tt]);
              ua[tt] = fmaf(sua, aua[tt], ua[tt]);
              gb[tt] = fmaf(sgb, agb[tt], gb[tt]);
              ub[tt] = fmaf(sub, aub[tt], ub[tt]);
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          if (TG > 1 && tt >= nt) break;
          const float g0 = group_sum<LPR>(ga[tt]), u0 = group_sum<LPR>(ua[tt]);
          const float g1 = group_sum<LPR>(gb[tt]), u1 = group_sum<LPR>(ub[tt]);
          if (lc == 0) {
            float *hrow = h_out + (int64_t)si.pos[t0 + tt] * I;
            if (va) hrow[ra] = silu_mul(g0, u0);
            if (vb) hrow[rb2] = silu_mul(g1, u1);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down

template <int LPR, int CPL, int TG, class C>
__global__ void __launch_bounds__(kThreads) down_kernel(Layer L, coli_moe_route_t r, int T,
                                                        const float *__restrict__ h_in,
                                                        float *__restrict__ o_out, int nrb,
                                                        int items) {
  constexpr int RPW = 64 / LPR;
  constexpr int ROWS_WAVE = 2 * RPW * 2;
  constexpr int ROWS_ITEM = 4 * ROWS_WAVE;
  const int H = L.H, I = L.I, NCH = I / 32;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ SlotInfo si;
  uint4 *xs = reinterpret_cast<uint4 *>(smem);               // [TG][8][NCH]: hi dw0..3, lo dw0..3
  float *corr = reinterpret_cast<float *>(xs + TG * 8 * NCH);  // [TG][NCH]
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int lr = lane / LPR, lc = lane % LPR;
  const int cpl = CPL ? CPL : (NCH + LPR - 1) / LPR;
  const int nslots = (items / nrb);

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int slot = item % nslots, rb = item / nslots;
    __syncthreads();
    if (!load_slot(r, slot, T, L.k, L.E, L.S, si)) continue;
    __syncthreads();
    const int e = si.expert, ntok = si.ntok;
    const uint8_t *qd = L.q4 + (int64_t)e * L.expert_bytes + C::bytes((int64_t)2 * I * H);
    const uint8_t *sd = reinterpret_cast<const uint8_t *>(L.scales + (int64_t)e * L.expert_scales +
                                                          (int64_t)2 * I * H / 64);
    const int64_t rowb = C::bytes(I);
    const int row_base = rb * ROWS_ITEM + wid * ROWS_WAVE;

    for (int t0 = 0; t0 < ntok; t0 += TG) {
      const int nt = min(TG, ntok - t0);
      __syncthreads();
      for (int i = threadIdx.x; i < TG * NCH; i += kThreads) {
        const int tt = i / NCH, c = i % NCH;
        float nb = 0.0f;
        if (tt < nt) {
          const float4 *src = reinterpret_cast<const float4 *>(h_in + (int64_t)si.pos[t0 + tt] * I) + 8 * c;
          uint32_t ph[16], pl[16];
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            const float4 a = src[2 * dw], b = src[2 * dw + 1];
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t h0 = f32_to_bf16_bits(v[2 * q]), h1 = f32_to_bf16_bits(v[2 * q + 1]);
              const float r0 = v[2 * q] - bf16_to_f32(h0), r1 = v[2 * q + 1] - bf16_to_f32(h1);
              const uint32_t l0 = f32_to_bf16_bits(r0), l1 = f32_to_bf16_bits(r1);
              hi[q] = h0 | (h1 << 16);
              lo[q] = l0 | (l1 << 16);
            }
            C::pairs(hi, &ph[4 * dw]);
            C::pairs(lo, &pl[4 * dw]);
            xs[(tt * 8 + dw) * NCH + c] = make_uint4(ph[4 * dw], ph[4 * dw + 1], ph[4 * dw + 2], ph[4 * dw + 3]);
            xs[(tt * 8 + 4 + dw) * NCH + c] = make_uint4(pl[4 * dw], pl[4 * dw + 1], pl[4 * dw + 2], pl[4 * dw + 3]);
          }
          nb = codec_bias2<C>(ph, pl);
        }
        corr[tt * NCH + c] = -nb;
      }
      __syncthreads();

#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int ma = row_base + it * 2 * RPW + lr, mb = ma + RPW;
        float oa[TG], ob[TG];
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) oa[tt] = ob[tt] = 0.0f;
        const bool va = ma < H, vb = mb < H;
#pragma unroll
        for (int i = 0; i < (CPL ? CPL : 1); ++i) {
          for (int ii = i; ii < cpl; ii += (CPL ? CPL : 1)) {
            const int c = lc + LPR * ii;
            if (c >= NCH) break;
            uint4 wa[C::Q], wb[C::Q];
#pragma unroll
            for (int q = 0; q < C::Q; ++q) wa[q] = wb[q] = make_uint4(0, 0, 0, 0);
            float sa = 0.f, sb = 0.f;
            if (va) {
#pragma unroll
              for (int q = 0; q < C::Q; ++q)
                wa[q] = *reinterpret_cast<const uint4 *>(qd + ma * rowb + 16 * (C::Q * c + q));
              sa = C::scale(C::scale_raw(sd, ma, I, c));
            }
            if (vb) {
#pragma unroll
              for (int q = 0; q < C::Q; ++q)
                wb[q] = *reinterpret_cast<const uint4 *>(qd + mb * rowb + 16 * (C::Q * c + q));
              sb = C::scale(C::scale_raw(sd, mb, I, c));
            }
            float aa[TG], ab[TG];
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) aa[tt] = ab[tt] = -corr[tt * NCH + c];
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
              if (TG > 1 && tt >= nt) break;
              uint32_t hp[16], lp[16];
#pragma unroll
              for (int dw = 0; dw < 4; ++dw) {
                const uint4 xh = xs[(tt * 8 + dw) * NCH + c];
                const uint4 xl = xs[(tt * 8 + 4 + dw) * NCH + c];
                hp[4 * dw] = xh.x;
                hp[4 * dw + 1] = xh.y;
                hp[4 * dw + 2] = xh.z;
                hp[4 * dw + 3] = xh.w;
                lp[4 * dw] = xl.x;
                lp[4 * dw + 1] = xl.y;
                lp[4 * dw + 2] = xl.z;
                lp[4 * dw + 3] = xl.w;
              }
              aa[tt] = C::template dot<true>(wa, hp, lp, aa[tt]);
              ab[tt] = C::template dot<true>(wb, hp, lp, ab[tt]);
            }
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
              oa[tt] = fmaf(sa, aa[tt], oa[tt]);
              ob[tt] = fmaf(sb, ab[tt], ob[tt]);
            }
          }
        }
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          if (TG > 1 && tt >= nt) break;
          const float s0 = group_sum<LPR>(oa[tt]), s1 = group_sum<LPR>(ob[tt]);
          if (lc == 0) {
            float *orow = o_out + (int64_t)si.pos[t0 + tt] * H;
            if (va) orow[ma] = s0;
            if (vb) orow[mb] = s1;
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------- combine

__global__ void __launch_bounds__(kThreads) combine_kernel(const float *__restrict__ o,
                                                           const int32_t *__restrict__ pair_pos,
                                                           const float *__restrict__ w, int T,
                                                           int H, int k, int S, void *y,
                                                           int y_dtype) {
  const int t = blockIdx.y;
  const int m = (blockIdx.x * kThreads + threadIdx.x) * 4;
  if (m >= H) return;
  // The row positions and weights are uniform over the workgroup.  They are
  // read in batches of kBatch, then all o rows of a batch are requested
  // before the first is used, so a token costs about two memory round trips
  // per batch instead of two per routed expert.  The sum order stays
  // j = 0 .. k-1, then the shared expert.
  constexpr int kBatch = 8;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // the shared expert's row (row 0 when there is none: read, not used)
  const float4 sh = *reinterpret_cast<const float4 *>(o + (S ? (int64_t)T * k + t : 0) * H + m);
  for (int j0 = 0; j0 < k; j0 += kBatch) {
    int64_t pos[kBatch];
    float wj[kBatch];
    float4 v[kBatch];
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      const int j = min(j0 + jj, k - 1);  // past k: a valid row, not used
      pos[jj] = pair_pos[(int64_t)t * k + j];
      wj[jj] = w[(int64_t)t * k + j];
    }
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj)
      v[jj] = *reinterpret_cast<const float4 *>(o + pos[jj] * H + m);
#pragma unroll
    for (int jj = 0; jj < kBatch; ++jj) {
      if (j0 + jj < k) {
        acc.x = fmaf(wj[jj], v[jj].x, acc.x);
        acc.y = fmaf(wj[jj], v[jj].y, acc.y);
        acc.z = fmaf(wj[jj], v[jj].z, acc.z);
        acc.w = fmaf(wj[jj], v[jj].w, acc.w);
      }
    }
  }
  if (S) {
    acc.x += sh.x;
    acc.y += sh.y;
    acc.z += sh.z;
    acc.w += sh.w;
  }
  if (y_dtype == COLI_OUT_F32) {
    *reinterpret_cast<float4 *>(reinterpret_cast<float *>(y) + (int64_t)t * H + m) = acc;
  } else {
    const uint32_t lo = f32_to_bf16_bits(acc.x) | (f32_to_bf16_bits(acc.y) << 16);
    const uint32_t hi = f32_to_bf16_bits(acc.z) | (f32_to_bf16_bits(acc.w) << 16);
    *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(y) + (int64_t)t * H + m) = make_uint2(lo, hi);
  }
}

// --------------------------------------------------------------- launch

struct Shape {
  int lpr, cpl;
};

Shape pick_shape(int K) {
  const int nch = K / 32;
  if (nch <= 8) return {8, 1};
  if (nch <= 16) return {16, 1};
  if (nch <= 32) return {32, 1};
  if (nch <= 64) return {64, 1};
  const int cpl = (nch + 63) / 64;
  return {64, cpl <= 4 ? cpl : 0};
}

int rows_per_item(int lpr) { return 4 * 2 * (64 / lpr) * 2; }

template <int TG, class C>
hipError_t launch_gateup(Shape sh, dim3 grid, size_t lds, hipStream_t s, const Layer &L,
                         const coli_moe_route_t &r, const uint16_t *x, int T, float *h,
                         int nrb, int items) {
#define COLI_GU(LPR, CPL)                                                                \
  launch_k(COLI_K_DECODE_GATEUP, gateup_kernel<LPR, CPL, TG, C>, grid, dim3(kThreads), lds, s, L, \
           r, x, T, h, nrb, items)
  switch (sh.lpr * 10 + sh.cpl) {
    case 81: COLI_GU(8, 1); break;
    case 161: COLI_GU(16, 1); break;
    case 321: COLI_GU(32, 1); break;
    case 641: COLI_GU(64, 1); break;
    case 642: COLI_GU(64, 2); break;
    case 643: COLI_GU(64, 3); break;
    case 644: COLI_GU(64, 4); break;
    default: COLI_GU(64, 0); break;
  }
#undef COLI_GU
  return hipGetLastError();
}

template <int TG, class C>
hipError_t launch_down(Shape sh, dim3 grid, size_t lds, hipStream_t s, const Layer &L,
                       const coli_moe_route_t &r, int T, const float *h, float *o, int nrb,
                       int items) {
#define COLI_DN(LPR, CPL)                                                                 \
  launch_k(COLI_K_DECODE_DOWN, down_kernel<LPR, CPL, TG, C>, grid, dim3(kThreads), lds, s, L, r, \
           T, h, o, nrb, items)
  switch (sh.lpr * 10 + sh.cpl) {
    case 81: COLI_DN(8, 1); break;
    case 161: COLI_DN(16, 1); break;
    case 321: COLI_DN(32, 1); break;
    case 641: COLI_DN(64, 1); break;
    case 642: COLI_DN(64, 2); break;
    case 643: COLI_DN(64, 3); break;
    case 644: COLI_DN(64, 4); break;
    default: COLI_DN(64, 0); break;
  }
#undef COLI_DN
  return hipGetLastError();
}

// tokens per pass: 1 for single-token decode, else as many as LDS allows
int pick_tg(int T, int K, int bytes_per_value) {
  if (T == 1) return 1;
  const size_t per_tok = (size_t)K * bytes_per_value + (size_t)(K / 32) * 4;
  return per_tok * 4 <= 60 * 1024 ? 4 : 1;
}

// Gate/up and down over (union slot, row block) work items, any shape and
// up to 64 tokens, for weight codec C.
template <class C>
hipError_t decode_general(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                          float *h, float *o, int nslots, hipStream_t s) {
  hipError_t err;
  {  // gate / up
    const Shape sh = pick_shape(L.H);
    const int nrb = (L.I + rows_per_item(sh.lpr) - 1) / rows_per_item(sh.lpr);
    const int items = nslots * nrb;
    const dim3 grid(items < 8192 ? items : 8192);
    const int tg = pick_tg(T, L.H, 2);
    const size_t lds = (size_t)tg * (L.H / 32) * (64 + 4);
    err = tg == 1 ? launch_gateup<1, C>(sh, grid, lds, s, L, r, x, T, h, nrb, items)
                  : launch_gateup<4, C>(sh, grid, lds, s, L, r, x, T, h, nrb, items);
    if (err != hipSuccess) return err;
  }
  {  // down
    const Shape sh = pick_shape(L.I);
    const int nrb = (L.H + rows_per_item(sh.lpr) - 1) / rows_per_item(sh.lpr);
    const int items = nslots * nrb;
    const dim3 grid(items < 8192 ? items : 8192);
    const int tg = pick_tg(T, L.I, 4);
    const size_t lds = (size_t)tg * (L.I / 32) * (128 + 4);
    err = tg == 1 ? launch_down<1, C>(sh, grid, lds, s, L, r, T, h, o, nrb, items)
                  : launch_down<4, C>(sh, grid, lds, s, L, r, T, h, o, nrb, items);
  }
  return err;
}

}  // namespace

void launch_combine(const float *o, const coli_moe_route_t &r, int T, int H, int k, int S,
                    void *y, int y_dtype, hipStream_t s) {
  const dim3 grid((H / 4 + kThreads - 1) / kThreads, T);
  launch_k(COLI_K_COMBINE, combine_kernel, grid, dim3(kThreads), 0, s, o, r.pair_pos, r.topk_w, T,
           H, k, S, y, y_dtype);
}

size_t decode_workspace(const Layer &L, int T) {
  const int64_t rows = pair_rows(L, T);
  return align_up((size_t)rows * L.I * 4) + align_up((size_t)rows * L.H * 4);
}

int launch_decode(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T, void *y,
                  int y_dtype, void *ws, hipStream_t s) {
  const int64_t rows = pair_rows(L, T);
  float *h = reinterpret_cast<float *>(ws);
  float *o = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + align_up((size_t)rows * L.I * 4));
  const int nslots = max_union(L, T) + L.S;
  hipError_t err = hipSuccess;

  if (launch_decode_stream(L, r, x, T, h, o, s, &err)) {
    if (err != hipSuccess) return COLI_E_HIP;
    launch_combine(o, r, T, L.H, L.k, L.S, y, y_dtype, s);
    return hip_status(hipGetLastError());
  }

  err = L.f4 ? decode_general<CodecF4>(L, r, x, T, h, o, nslots, s)
      : L.w8  ? decode_general<CodecI8>(L, r, x, T, h, o, nslots, s)
              : decode_general<CodecI4>(L, r, x, T, h, o, nslots, s);
  if (err != hipSuccess) return COLI_E_HIP;
  launch_combine(o, r, T, L.H, L.k, L.S, y, y_dtype, s);
  err = hipGetLastError();
  return hip_status(err);
}

}  // namespace coli
