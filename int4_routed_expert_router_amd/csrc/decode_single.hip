// decode_single.hip -- single-token decode (T = 1): streaming GEMVs.
//
// The union's rows are split into short runs (2 gate/up row pairs or about
// 8 KB of down rows), one per wavefront, each inside one union slot.  A
// wavefront requests all of its weights at once, then fetches its
// activation chunks, computes and exits: many short independent wavefronts
// keep the most bytes in flight.  Gate/up stages x once per workgroup in LDS
// (the same vector for every slot when T = 1); down reads its chunks of the
// slot's h directly, as gate/up wrote them.  Nibbles become exact
// bf16 values 136 + q (one v_bitop3 per pair after a shift) and meet the
// activations in v_dot2_f32_bf16; each 32-chunk's bias 136 * sum(x) is
// removed before its fp16 group scale.  Lane partials of several rows are
// combined with a reduce-scatter (each shuffle step halves the values a lane
// carries).
#include "device_common.h"
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

// Expert and pair-major row of union slot `slot` for a single token.
COLI_DEV void slot_of(const coli_moe_route_t &r, const Layer &L, int slot, int &e, int &pos) {
  if (L.S && slot == 0) {
    e = L.E;
    pos = L.k;  // row T*k + t with T = 1, t = 0
  } else {
    e = r.union_ids[slot - L.S];
    pos = r.offsets[e];
  }
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

// 32 weights of one chunk (a 16-byte load) dotted with paired activations;
// the accumulator starts at -bias.
COLI_DEV float chunk_dot(const uint4 w, const uint32_t *xp, float neg_bias) {
  const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
  float a = neg_bias;
#pragma unroll
  for (int dw = 0; dw < 4; ++dw) {
    uint32_t p[4];
    nib8_to_bf16x4(wv[dw], p[0], p[1], p[2], p[3]);
#pragma unroll
    for (int q = 0; q < 4; ++q) a = dot2_bf16(p[q], xp[4 * dw + q], a);
  }
  return a;
}

// The down GEMV consumes h as bf16 hi + lo halves (16 significant bits),
// already paired to the nibble order.  Row layout (I values, 4 bytes each):
// chunk c of 32 values holds 16 hi dwords then 16 lo dwords; dword 4*o + q
// of a half pairs values 8o + q (low 16 bits) and 8o + q + 4 (high 16 bits).
COLI_DEV void store_h_pair(float *row, int n, float h) {
  const uint32_t hi = f32_to_bf16_bits(h);
  const uint32_t lo = f32_to_bf16_bits(h - bf16_to_f32(hi));
  const int c = n >> 5, w = n & 31, o = w >> 3, k = w & 7;
  uint16_t *base = reinterpret_cast<uint16_t *>(row + 32 * c);
  const int half = 2 * (4 * o + (k & 3)) + (k >> 2);
  base[half] = (uint16_t)hi;
  base[32 + half] = (uint16_t)lo;
}

// ----------------------------------------------------------- gate / up

// H = 2048 * CPL: lane owns chunks lane + 64 i (i < CPL) of every row.  A
// wavefront computes RPW rows n of one slot; all their weights are requested
// at once, before the workgroup's activation staging, so the loads of every
// resident wavefront overlap.
template <int CPL, int RPW>
__global__ void __launch_bounds__(kThreads) gateup_single_kernel(
    Layer L, coli_moe_route_t r, const uint16_t *__restrict__ x, float *__restrict__ h_out) {
  constexpr int NCH = 64 * CPL;
  __shared__ uint4 xs[4 * NCH];
  __shared__ float xb[NCH];
  const int lane = threadIdx.x & 63;
  const int H = L.H, I = L.I;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int waves_per_slot = I / RPW;
  const int slot = wave / waves_per_slot;
  const bool active = slot < L.S + r.n_union[0];
  int e = 0, pos = 0;
  if (active) slot_of(r, L, slot, e, pos);
  const int n0 = (wave % waves_per_slot) * RPW;
  const uint8_t *qg = L.q4 + (int64_t)e * L.expert_bytes + (int64_t)n0 * (H / 2) + 16 * lane;
  const uint8_t *qu = qg + (int64_t)I * H / 2;
  const uint16_t *sgp = L.scales + (int64_t)e * L.expert_scales + (int64_t)n0 * (H / 64) + lane / 2;
  const uint16_t *sup = sgp + (int64_t)I * H / 64;
  uint4 wg[RPW][CPL], wu[RPW][CPL];
  uint16_t sg[RPW][CPL], su[RPW][CPL];
  if (active) {
#pragma unroll
    for (int j = 0; j < RPW; ++j)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const int64_t ob = (int64_t)j * (H / 2) + 1024 * i;
        const int64_t os = (int64_t)j * (H / 64) + 32 * i;
        wg[j][i] = *reinterpret_cast<const uint4 *>(qg + ob);
        wu[j][i] = *reinterpret_cast<const uint4 *>(qu + ob);
        sg[j][i] = sgp[os];
        su[j][i] = sup[os];
      }
  }
  // stage x: chunk c -> four quads of paired bf16 and its bias
  for (int c = threadIdx.x; c < NCH; c += kThreads) {
    const uint4 *src = reinterpret_cast<const uint4 *>(x) + 4 * c;
    uint32_t p[16];
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const uint4 v = src[dw];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
      x8_to_pairs(d, &p[4 * dw]);
      xs[dw * NCH + c] = make_uint4(p[4 * dw], p[4 * dw + 1], p[4 * dw + 2], p[4 * dw + 3]);
    }
    xb[c] = chunk_bias(p);
  }
  __syncthreads();
  if (!active) return;

  float v[2 * RPW];
#pragma unroll
  for (int j = 0; j < 2 * RPW; ++j) v[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    XChunk xc;
    lds_chunk(xs, NCH, lane + 64 * i, xc);
    const float nb = xb[lane + 64 * i];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      v[2 * j] = fmaf(f16_to_f32(sg[j][i]), chunk_dot(wg[j][i], xc.p, nb), v[2 * j]);
      v[2 * j + 1] = fmaf(f16_to_f32(su[j][i]), chunk_dot(wu[j][i], xc.p, nb), v[2 * j + 1]);
    }
  }
  // value 2j is the gate of row j, 2j+1 its up; bring them to one lane
  const float tot = reduce_scatter<2 * RPW, 64>(v, lane);
  const int vi = value_index<2 * RPW, 64>(lane);
  constexpr int kSpan = 64 / (2 * RPW);  // lanes holding one value
  const float up = __shfl_down(tot, kSpan, 64);
  if ((lane % kSpan) == 0 && (vi & 1) == 0)
    store_h_pair(h_out + (int64_t)pos * I, n0 + vi / 2, silu_mul(tot, up));
}

// ------------------------------------------------------------------ down

// K = I: LPR lanes per row (LPR = I/32 when I < 2048, else 64 with CPL
// chunks each); RPI = 64/LPR rows share a wave instruction; a wavefront
// computes RG such row groups (RPI * RG rows m) of one slot.  Each lane
// reads its chunks of the slot's h (hi + lo pairs, written by gate/up) once.
template <int LPR, int CPL, int RG>
__global__ void __launch_bounds__(kThreads) down_single_kernel(
    Layer L, coli_moe_route_t r, const float *__restrict__ h_in, float *__restrict__ o_out) {
  constexpr int RPI = 64 / LPR;
  constexpr int RPW = RPI * RG;
  const int lane = threadIdx.x & 63;
  const int lr = lane / LPR, lc = lane % LPR;
  const int H = L.H, I = L.I;
  const int wave = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int waves_per_slot = H / RPW;
  const int slot = wave / waves_per_slot;
  if (slot >= L.S + r.n_union[0]) return;
  int e, pos;
  slot_of(r, L, slot, e, pos);
  const int m0 = (wave % waves_per_slot) * RPW;
  const uint8_t *qd = L.q4 + (int64_t)e * L.expert_bytes + (int64_t)I * H +
                      (int64_t)(m0 + lr) * (I / 2) + 16 * lc;
  const uint16_t *sdp = L.scales + (int64_t)e * L.expert_scales + (int64_t)2 * I * H / 64 +
                        (int64_t)(m0 + lr) * (I / 64) + lc / 2;
  uint4 w[RG][CPL];
  uint16_t sc[RG][CPL];
#pragma unroll
  for (int j = 0; j < RG; ++j)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int64_t row = RPI * j;
      w[j][i] = *reinterpret_cast<const uint4 *>(qd + row * (I / 2) + 16 * LPR * i);
      sc[j][i] = sdp[row * (I / 64) + LPR / 2 * i];
    }
  float v[RG];
#pragma unroll
  for (int j = 0; j < RG; ++j) v[j] = 0.0f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const uint4 *src = reinterpret_cast<const uint4 *>(h_in + (int64_t)pos * I + 32 * (lc + LPR * i));
    XChunk hi, lo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 a = src[q], b = src[4 + q];
      hi.p[4 * q] = a.x, hi.p[4 * q + 1] = a.y, hi.p[4 * q + 2] = a.z, hi.p[4 * q + 3] = a.w;
      lo.p[4 * q] = b.x, lo.p[4 * q + 1] = b.y, lo.p[4 * q + 2] = b.z, lo.p[4 * q + 3] = b.w;
    }
    const float nb = chunk_bias2(hi.p, lo.p);
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      const uint32_t wv[4] = {w[j][i].x, w[j][i].y, w[j][i].z, w[j][i].w};
      float a = nb;
#pragma unroll
      for (int dw = 0; dw < 4; ++dw) {
        uint32_t p[4];
        nib8_to_bf16x4(wv[dw], p[0], p[1], p[2], p[3]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a = dot2_bf16(p[q], hi.p[4 * dw + q], a);
          a = dot2_bf16(p[q], lo.p[4 * dw + q], a);
        }
      }
      v[j] = fmaf(f16_to_f32(sc[j][i]), a, v[j]);
    }
  }
  const float tot = reduce_scatter<RG, LPR>(v, lc);
  constexpr int kSpan = LPR / RG;
  if ((lc % kSpan) == 0)
    o_out[(int64_t)pos * H + m0 + lr + RPI * value_index<RG, LPR>(lc)] = tot;
}

template <int CPL>
hipError_t gateup_cpl(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, float *h,
                      int nslots, hipStream_t s) {
  constexpr int RPW = 2;
  const int waves = nslots * (L.I / RPW);
  launch_k(COLI_K_DECODE_GATEUP, gateup_single_kernel<CPL, RPW>,
           dim3((waves + kWaves - 1) / kWaves), dim3(kThreads), 0, s, L, r, x, h);
  return hipGetLastError();
}

// row groups per wavefront of the down GEMV: about eight 16-byte loads per
// lane (8 rows of 1 KB when I = 2048)
template <int LPR, int CPL>
constexpr int down_rg() { return CPL == 1 ? 8 : (CPL == 2 ? 4 : 2); }
template <int LPR, int CPL>
constexpr int down_rows_wave() { return (64 / LPR) * down_rg<LPR, CPL>(); }

template <int LPR, int CPL>
hipError_t down_shape(const Layer &L, const coli_moe_route_t &r, const float *h, float *o,
                      int nslots, hipStream_t s) {
  const int waves = nslots * (L.H / down_rows_wave<LPR, CPL>());
  launch_k(COLI_K_DECODE_DOWN, down_single_kernel<LPR, CPL, down_rg<LPR, CPL>()>,
           dim3((waves + kWaves - 1) / kWaves), dim3(kThreads), 0, s, L, r, h, o);
  return hipGetLastError();
}

}  // namespace

// Launches gate/up and down for T = 1 when the shape has a fast path
// (H a multiple of 2048 up to 8192; I in {512, 1024} or a multiple of 2048
// up to 8192; H a multiple of a down workgroup's rows).  Returns false,
// launching nothing, otherwise.
bool launch_decode_single(const Layer &L, const coli_moe_route_t &r, const uint16_t *x,
                          float *h, float *o, hipStream_t s, hipError_t *err) {
  const int nslots = max_union(L, 1) + L.S;
  const int hc = L.H / 2048;
  if (L.H % 2048 || hc < 1 || hc > 4) return false;
  int lpr, cpl, rows_wave;
  if (L.I == 512) {
    lpr = 16, cpl = 1, rows_wave = down_rows_wave<16, 1>();
  } else if (L.I == 1024) {
    lpr = 32, cpl = 1, rows_wave = down_rows_wave<32, 1>();
  } else if (L.I % 2048 == 0 && L.I / 2048 <= 4) {
    lpr = 64, cpl = L.I / 2048;
    rows_wave = cpl == 1 ? down_rows_wave<64, 1>() : cpl == 2 ? down_rows_wave<64, 2>()
                : cpl == 3 ? down_rows_wave<64, 3>() : down_rows_wave<64, 4>();
  } else {
    return false;
  }
  if (L.I % 2 || L.H % rows_wave) return false;
  hipError_t e = hipSuccess;
  switch (hc) {
    case 1: e = gateup_cpl<1>(L, r, x, h, nslots, s); break;
    case 2: e = gateup_cpl<2>(L, r, x, h, nslots, s); break;
    case 3: e = gateup_cpl<3>(L, r, x, h, nslots, s); break;
    default: e = gateup_cpl<4>(L, r, x, h, nslots, s); break;
  }
  if (e == hipSuccess) {
    if (lpr == 16) e = down_shape<16, 1>(L, r, h, o, nslots, s);
    else if (lpr == 32) e = down_shape<32, 1>(L, r, h, o, nslots, s);
    else if (cpl == 1) e = down_shape<64, 1>(L, r, h, o, nslots, s);
    else if (cpl == 2) e = down_shape<64, 2>(L, r, h, o, nslots, s);
    else if (cpl == 3) e = down_shape<64, 3>(L, r, h, o, nslots, s);
    else e = down_shape<64, 4>(L, r, h, o, nslots, s);
  }
  *err = e;
  return true;
}

}  // namespace coli
