// prefill.hip -- prefill / large-batch forward on the integer path.
//
// The integer kernel of the reference engine takes Q8_0-style int8
// activations (alphamatch.ai blog on colibri, section "優化整數核心"), and
// prefill runs the MoE as a batched union (same blog, section "技術卓越").
// Here that contraction runs on gfx950's int8 matrix cores:
//
//  quantize : x (bf16) -> Q8_0 int8 + fp16 scale per 32 values.
//  plan     : the batch union becomes a list of (expert, 64-token tile).
//  gemm     : one work item = (token tile, 64 output channels of gate AND
//             up, or 128 rows of down).  Per 64-deep K step the workgroup
//             stages 128 weight rows (int4 -> int8 x16, exact) and 64 token
//             rows of int8 activations in LDS in matrix-core operand order,
//             then every wavefront issues v_mfma_i32_16x16x32_i8, one per
//             32-value block so each block's exact int32 dot stays separate.
//             The accumulator input is the bit pattern of 1.5*2^23, so the
//             int32 result read as fp32 is 1.5*2^23 + 16*dot exactly; one FMA
//             with the activation scale removes the offset and scales the
//             block, a second applies the weight group's scale.
//             gate/up epilogue: h = silu(g)*u, then Q8_0 of h per 32
//             channels (one wavefront holds exactly one block per token).
//             down epilogue: fp32 o rows.
//  combine  : shared with decode (fixed-order weighted sum).
#include "device_common.h"
#include "internal.h"

namespace coli {

namespace {

constexpr int kThreads = 256;
constexpr int BM = 64;    // tokens per tile
constexpr int BR = 128;   // weight rows per tile
constexpr int BK = 64;    // reduction depth per step (one weight scale group)
constexpr int kDepth = 4; // K steps of global loads kept in flight per thread
constexpr uint32_t kMagic = 0x4B400000u;  // bits of 1.5 * 2^23
constexpr float kMagicF = 12582912.0f;

enum Mode { kGateUp = 0, kDown = 1, kDots = 2 };

// --------------------------------------------------------------- Q8_0

// Quantise 32 fp32 values held by one thread: q (natural order) and fp16 d.
// d = max|v| / 127 (correctly rounded division), q = round half away from
// zero of v / d, clamped to +-127; all-zero blocks give d = 0, q = 0.
COLI_DEV void q8_0_block(const float v[32], uint32_t qw[8], uint16_t &d16) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
  const float d = __fdiv_rn(a, 127.0f);
  d16 = f32_to_f16_bits(d);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t packed = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int q = 0;
      if (a != 0.0f) {
        q = (int)roundf(__fdiv_rn(v[4 * w + j], d));
        q = max(-127, min(127, q));
      }
      packed |= (uint32_t)(q & 0xff) << (8 * j);
    }
    qw[w] = packed;
  }
}

// PR (the int4 path of the DMA GEMM): the codes of every 8 values are
// stored as [k0 k2 k4 k6 k1 k3 k5 k7], the order of unpacked nibbles, and
// the block's record {-M*d16, d16} (fp32) replaces the fp16 scale.
template <bool PR>
__global__ void __launch_bounds__(kThreads) quantize_kernel(const void *__restrict__ src,
                                                            int src_dtype, int64_t nblocks,
                                                            int8_t *__restrict__ q,
                                                            uint16_t *__restrict__ d,
                                                            float2 *__restrict__ rec) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if (src_dtype == COLI_SRC_BF16) {
    const uint4 *p = reinterpret_cast<const uint4 *>(src) + 4 * b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = p[i];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = bf16_to_f32(w[j] & 0xffffu);
        v[8 * i + 2 * j + 1] = bf16_to_f32(w[j] >> 16);
      }
    }
  } else {
    const float4 *p = reinterpret_cast<const float4 *>(src) + 8 * b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4 f = p[i];
      v[4 * i] = f.x;
      v[4 * i + 1] = f.y;
      v[4 * i + 2] = f.z;
      v[4 * i + 3] = f.w;
    }
  }
  uint32_t qw[8];
  uint16_t d16;
  q8_0_block(v, qw, d16);
  if (PR) {
#pragma unroll
    for (int w = 0; w < 8; w += 2) {
      const uint32_t lo = qw[w], hi = qw[w + 1];
      qw[w] = __builtin_amdgcn_perm(hi, lo, 0x06040200u);
      qw[w + 1] = __builtin_amdgcn_perm(hi, lo, 0x07050301u);
    }
  }
  uint4 *qo = reinterpret_cast<uint4 *>(q) + 2 * b;
  qo[0] = make_uint4(qw[0], qw[1], qw[2], qw[3]);
  qo[1] = make_uint4(qw[4], qw[5], qw[6], qw[7]);
  if (PR) {
    const float df = f16_to_f32(d16);
    rec[b] = make_float2(-kMagicF * df, df);
  } else {
    d[b] = d16;
  }
}

// ---------------------------------------------------------------- plan

// A tile of up to BM tokens of one expert.  `row0` is the first pair-major
// row (h / o rows); routed tiles read token ids from route.pairs, shared
// tiles (expert == E) use tokens row0 - T*k onwards.
struct TileDesc {
  int expert, row0, ntok, pad;
};

__global__ void __launch_bounds__(1024) plan_kernel(coli_moe_route_t r, int T, int k, int E,
                                                    int S, int4 *__restrict__ tiles,
                                                    int *__restrict__ ntiles) {
  __shared__ int wsum[16];
  __shared__ int total;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int nu = r.n_union[0];
  const int shared_tiles = S ? (T + BM - 1) / BM : 0;
  int base_off = shared_tiles;
  for (int u0 = 0; u0 < nu; u0 += 1024) {
    const int u = u0 + tid;
    int e = 0, cnt = 0, off = 0;
    if (u < nu) {
      e = r.union_ids[u];
      cnt = r.counts[e];
      off = r.offsets[e];
    }
    const int nt = (cnt + BM - 1) / BM;
    int inc = nt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(inc, o, 64);
      if (lane >= o) inc += n;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    if (tid == 0) {
      int acc = 0;
      for (int i = 0; i < 16; ++i) {
        const int t = wsum[i];
        wsum[i] = acc;
        acc += t;
      }
      total = acc;
    }
    __syncthreads();
    const int first = base_off + wsum[wid] + inc - nt;
    for (int j = 0; j < nt; ++j)
      tiles[first + j] = make_int4(e, off + BM * j, min(BM, cnt - BM * j), 0);
    base_off += total;
    __syncthreads();
  }
  for (int j = tid; j < shared_tiles; j += 1024)
    tiles[j] = make_int4(E, T * k + BM * j, min(BM, T - BM * j), 0);
  if (tid == 0) ntiles[0] = base_off;
}

// ---------------------------------------------------------------- GEMM

// weight code formats: int4 nibbles, int8 bytes, MXFP4 E2M1 nibbles
constexpr int kFmtI4 = 0, kFmtI8 = 1, kFmtF4 = 2;

// MXFP4: 8 E2M1 codes (a dword, low nibble first) -> 8 int8 2 * E2M1 in k
// order, as two dwords.  Magnitudes index byte tables of 2|v| and -2|v|
// (v_perm), and each byte takes the negative entry where its code's sign bit
// is set: v_perm selectors 8-11 replicate bits 15 / 31 of its operands, so
// shifted copies of the codes give 0xff per negative code.
constexpr uint32_t kF4PosLo = 0x03020100u, kF4PosHi = 0x0C080604u;  // 0 1 2 3 | 4 6 8 12
constexpr uint32_t kF4NegLo = 0xFDFEFF00u, kF4NegHi = 0xF4F8FAFCu;  // negated
COLI_DEV void fp4x8_to_i8(uint32_t w, uint32_t &k0123, uint32_t &k4567) {
  const uint32_t me = w & 0x07070707u, mo = (w >> 4) & 0x07070707u;  // even / odd k
  // sign masks: even codes' sign bits 3, 11, 19, 27; odd codes' 7, 15, 23, 31
  const uint32_t se = __builtin_amdgcn_perm(w << 4, w << 12, 0x0B090A08u);
  const uint32_t so = __builtin_amdgcn_perm(w, w << 8, 0x0B090A08u);
  // v_bitop3 truth table 0xCA is a ? b : c, bit by bit
  const uint32_t ve = __builtin_amdgcn_bitop3_b32(
      se, __builtin_amdgcn_perm(kF4NegHi, kF4NegLo, me), __builtin_amdgcn_perm(kF4PosHi, kF4PosLo, me),
      0xCAu);  // se ? neg : pos
  const uint32_t vo = __builtin_amdgcn_bitop3_b32(
      so, __builtin_amdgcn_perm(kF4NegHi, kF4NegLo, mo), __builtin_amdgcn_perm(kF4PosHi, kF4PosLo, mo),
      0xCAu);
  // interleave: k0 k1 k2 k3 = ve.b0 vo.b0 ve.b1 vo.b1, k4..k7 = bytes 2, 3
  k0123 = __builtin_amdgcn_perm(vo, ve, 0x05010400u);
  k4567 = __builtin_amdgcn_perm(vo, ve, 0x07030602u);
}


// LDS stage: operands already in matrix-core lane order.  Each 16-row x
// 32-deep operand tile is 64 lanes x 8 bytes; consecutive tiles are kPad
// entries apart (64 + 16), which puts the two 32-blocks of a row tile (and
// of a token tile) in opposite halves of the 256-byte bank window, so the
// unpacking writes below hit distinct banks within each half-wavefront.
constexpr int kPad = 80;
// NB weight scales per row and step: 1 (a 64-weight group) or 2 (MXFP4,
// one per 32-block).
template <int NB>
struct Stage {
  uint2 w[BR / 16][2][kPad];  // [row tile][32-block][lane] 8 int8 weights (int4: x16)
  uint2 a[BM / 16][2][kPad];  // [token tile][32-block][lane] 8 int8 activations
  float sw[NB][BR];           // weight scales of each row (0 on padding steps)
  float4 sa[BM];              // per token: d0*f, -M*d0*f, d1*f, -M*d1*f (f: 1/16 for int4)
};

struct GemmArgs {
  const uint8_t *wq;       // code matrix base (rows x K >> rs bytes)
  int rs;                  // row bytes = K >> rs: 1 for int4 codes, 0 for int8
  const uint16_t *ws;      // its scales (rows x K/64)
  int rows;                // rows of this matrix (I or H)
  int K;                   // reduction length
  const int8_t *act;       // activation rows [*, K] (natural k order)
  const uint16_t *act_d;   // their fp16 scales [*, K/32]
  int64_t up_offset_q;     // gate/up: byte offset of the up matrix from gate
  int64_t up_offset_s;     // and of its scales
};

// Row source of weight row r (0..BR-1) of a tile starting at n0.  Rows past
// the matrix are clamped to row 0: they are computed and never stored.
template <int MODE>
COLI_DEV void weight_row(const GemmArgs &g, int n0, int r, const uint8_t *&q,
                         const uint16_t *&s) {
  int n;
  int64_t oq = 0, os = 0;
  if (MODE == kGateUp) {
    n = n0 + (r & 63);
    if (r >= 64) {
      oq = g.up_offset_q;
      os = g.up_offset_s;
    }
  } else {
    n = n0 + r;
  }
  const int nn = n < g.rows ? n : 0;
  q = g.wq + oq + (int64_t)nn * (g.K >> g.rs);
  s = g.ws + os + (int64_t)nn * (g.K / 64);
}

// What one thread moves from global memory per K step, and where from.
// Thread t: weights of row 16*(t>>5) + (t&15), 32-block (t>>4)&1; int8
// activations of token 16*(t>>6) + (t&15), 16-byte quarter 2*((t>>4)&1) +
// ((t>>5)&1); two fp16 scales: a weight row's group scale (t < 128, twice)
// or token (t-128)&63's two block scales.  Every thread issues the same
// four unconditional loads, so the compiler can count them in flight.
struct Src {
  const uint8_t *w;
  const int8_t *a;
  const uint16_t *s;
  int s_step;  // scale elements per K step (1 weight, 2 activation)
  int s_next;  // offset of the second scale
};

template <int WF>
struct Prefetch {
  uint4 w[WF == kFmtI8 ? 2 : 1];  // one 32-block of codes: 16 bytes of nibbles, or 32 of int8
  uint4 a;                        // 16 bytes of int8 activations
  uint32_t s;  // two 16-bit scale units, first in the low half (MXFP4: two E8M0 bytes in one)
};

template <int WF>
COLI_DEV void load_step(const Src &src, int ks, Prefetch<WF> &p) {
#pragma unroll
  for (int h = 0; h < (WF == kFmtI8 ? 2 : 1); ++h)
    p.w[h] = *reinterpret_cast<const uint4 *>(src.w + ks * (WF == kFmtI8 ? BK : BK / 2) + 16 * h);
  p.a = *reinterpret_cast<const uint4 *>(src.a + ks * BK);
  const uint16_t *s = src.s + ks * src.s_step;
  p.s = (uint32_t)s[0] | ((uint32_t)s[src.s_next] << 16);
}

// Registers -> LDS for one step.  `live` is false on the padding steps past
// the end of K: their weight scales become 0, so they add exactly nothing.
// 2^(E - 128) of an E8M0 byte: the MXFP4 scale halved for the doubled codes
COLI_DEV float e8m0_half(uint32_t E) {
  return __uint_as_float(E > 1 ? (E - 1) << 23 : (0x00400000u >> (1 - E)));
}

template <int MODE, int WF>
COLI_DEV void store_step(const Prefetch<WF> &p, Stage<WF == kFmtF4 ? 2 : 1> &st, int wid,
                         bool live) {
  const int t = threadIdx.x;
  {  // 32 codes -> 32 int8, natural k order, into 4 lanes' slots
    const int rt = t >> 5, blk = (t >> 4) & 1, rr = t & 15;
    if (WF == kFmtI8) {  // as they are: 8 bytes per lane
      const uint4 v0 = p.w[0], v1 = p.w[WF == kFmtI8 ? 1 : 0];
      st.w[rt][blk][rr] = make_uint2(v0.x, v0.y);
      st.w[rt][blk][rr + 16] = make_uint2(v0.z, v0.w);
      st.w[rt][blk][rr + 32] = make_uint2(v1.x, v1.y);
      st.w[rt][blk][rr + 48] = make_uint2(v1.z, v1.w);
    } else {
      const uint32_t w[4] = {p.w[0].x, p.w[0].y, p.w[0].z, p.w[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t lo, hi;
        if (WF == kFmtF4) {
          fp4x8_to_i8(w[i], lo, hi);  // 2 * E2M1
        } else {
          const uint32_t even = (w[i] << 4) & 0xf0f0f0f0u;  // k 0,2,4,6 (x16)
          const uint32_t odd = w[i] & 0xf0f0f0f0u;          // k 1,3,5,7 (x16)
          lo = __builtin_amdgcn_perm(odd, even, 0x05010400u);
          hi = __builtin_amdgcn_perm(odd, even, 0x07030602u);
        }
        st.w[rt][blk][rr + 16 * i] = make_uint2(lo, hi);
      }
    }
  }
  {  // activations: token tile wid, k [16*qq, 16*qq+16) of the step
    const int blk = (t >> 4) & 1, j0 = 2 * ((t >> 5) & 1), mm = t & 15;
    st.a[wid][blk][mm + 16 * j0] = make_uint2(p.a.x, p.a.y);
    st.a[wid][blk][mm + 16 * (j0 + 1)] = make_uint2(p.a.z, p.a.w);
  }
  if (MODE == kDots) return;
  if (wid < 2) {
    if (WF == kFmtF4) {  // the step's two E8M0 bytes, block 0 in the low byte
      st.sw[0][t] = live ? e8m0_half(p.s & 0xffu) : 0.0f;
      st.sw[WF == kFmtF4 ? 1 : 0][t] = live ? e8m0_half((p.s >> 8) & 0xffu) : 0.0f;
    } else {
      st.sw[0][t] = live ? f16_to_f32((uint16_t)p.s) : 0.0f;
    }
  } else if (wid == 2) {
    // int4 codes sit in the stage x16: their activation scales carry 1/16
    constexpr float f = WF == kFmtI4 ? 0.0625f : 1.0f;
    const float d0 = f16_to_f32((uint16_t)p.s) * f;
    const float d1 = f16_to_f32((uint16_t)(p.s >> 16)) * f;
    st.sa[t - BR] = make_float4(d0, -kMagicF * d0, d1, -kMagicF * d1);
  }
}

COLI_DEV coli_i32x4 mfma_i8(uint2 a, uint2 b, coli_i32x4 c) {
  const long la = (long)(((uint64_t)a.y << 32) | a.x);
  const long lb = (long)(((uint64_t)b.y << 32) | b.x);
  return __builtin_amdgcn_mfma_i32_16x16x32_i8(la, lb, c, 0, 0, 0);
}

// Row tiles of a wave: gate/up waves (wn) own gate tiles {2wn, 2wn+1} and up
// tiles {4+2wn, 4+2wn+1}; down/dots waves own tiles {4wn .. 4wn+3}.
template <int MODE>
COLI_DEV int wave_row_tile(int wn, int a) {
  return MODE == kGateUp ? (a < 2 ? 2 * wn + a : 4 + 2 * wn + (a - 2)) : 4 * wn + a;
}

// One work item of the grouped GEMM: a tile of up to BM token rows of one
// expert, times one block of output rows.  Fills the token row ids (input
// rows) and pair-major output rows of the tile in LDS; tokens past ntok read
// row 0 and are never stored.
struct Item {
  int expert, row0, ntok, n0;
};

// Work items are ordered in bands of kBand consecutive token tiles: within a
// band, the tiles at one block of output rows, then the next block.  Tiles of
// one expert are consecutive, so the tiles that share a weight slice run at
// about the same time and read it from L2, while a band's activations (at
// most kBand x 64 rows) stay in L2 across its row blocks.
constexpr int kBand = 4;
COLI_DEV int band_items(int ntiles, int n_ntiles) {
  return (ntiles + kBand - 1) / kBand * kBand * n_ntiles;
}
COLI_DEV void item_coords(int item, int n_ntiles, int &tile, int &ntile) {
  const int per_band = kBand * n_ntiles;
  const int band = item / per_band, rem = item - band * per_band;
  ntile = rem / kBand;
  tile = band * kBand + (rem - ntile * kBand);
}

template <int MODE>
COLI_DEV Item setup_item(int tile, int ntile, const int4 *tiles, int fixed_ntok,
                         int fixed_expert, const coli_moe_route_t &r, int T, int k,
                         int *rowid, int *outrow) {
  Item it;
  if (tiles) {
    const int4 td = tiles[tile];
    it.expert = td.x;
    it.row0 = td.y;
    it.ntok = td.z;
  } else {
    it.expert = fixed_expert;
    it.row0 = tile * BM;
    it.ntok = min(BM, fixed_ntok - it.row0);
  }
  it.n0 = ntile * (MODE == kGateUp ? 64 : BR);
  __syncthreads();  // the previous item's epilogue has read rowid / outrow
  if (threadIdx.x < BM) {
    const int m = threadIdx.x;
    int rid = 0, orow = 0;
    if (m < it.ntok) {
      orow = it.row0 + m;
      if (MODE == kGateUp) {
        rid = (it.row0 >= T * k) ? (it.row0 - T * k) + m : r.pairs[it.row0 + m] / k;
      } else {
        rid = it.row0 + m;
      }
    }
    rowid[m] = rid;
    outrow[m] = orow;
  }
  __syncthreads();
  return it;
}

// Epilogue of a work item from the per-wave accumulators (8 16x16 tiles:
// a*2+ms = row tile a of the wave, token tile ms).
//  gate/up: h = silu(g) * u, then Q8_0 of h per 32 channels -- one wave
//           holds exactly the 32 channels of one block for its 32 tokens.
//  down   : fp32 o rows.
template <int MODE>
COLI_DEV void epilogue(const float (&acc)[8][4], const GemmArgs &g, const Item &it,
                       const int *outrow, int wn, int wm, int lane, int8_t *qh_out,
                       uint16_t *dh_out, float *o_out) {
  if (MODE == kGateUp) {
    // acc[a*2+ms]: a in {0,1} gate row tiles, {2,3} the up tiles of the same
    // channels (row sub-tile ns = a & 1)
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const int m = 32 * wm + 16 * ms + (lane & 15);
      float hv[2][4];
      float amax = 0.0f;
#pragma unroll
      for (int ns = 0; ns < 2; ++ns)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hv[ns][i] = silu_mul(acc[ns * 2 + ms][i], acc[(2 + ns) * 2 + ms][i]);
          amax = fmaxf(amax, fabsf(hv[ns][i]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const float dq = __fdiv_rn(amax, 127.0f);
      uint32_t qw[2];
#pragma unroll
      for (int ns = 0; ns < 2; ++ns) {
        uint32_t packed = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int q = 0;
          if (amax != 0.0f) {
            q = (int)roundf(__fdiv_rn(hv[ns][i], dq));
            q = max(-127, min(127, q));
          }
          packed |= (uint32_t)(q & 0xff) << (8 * i);
        }
        qw[ns] = packed;
      }
      if (m < it.ntok) {
        const int I = g.rows;
        const int ch = it.n0 + 32 * wn;  // first channel of this wave's block
        if (ch < I) {
          int8_t *qrow = qh_out + (int64_t)outrow[m] * I + ch;
          *reinterpret_cast<uint32_t *>(qrow + 4 * (lane >> 4)) = qw[0];
          *reinterpret_cast<uint32_t *>(qrow + 16 + 4 * (lane >> 4)) = qw[1];
          if ((lane >> 4) == 0) dh_out[(int64_t)outrow[m] * (I / 32) + ch / 32] = f32_to_f16_bits(dq);
        }
      }
    }
  } else if (MODE == kDown) {
#pragma unroll
    for (int ms = 0; ms < 2; ++ms) {
      const int m = 32 * wm + 16 * ms + (lane & 15);
      if (m >= it.ntok) continue;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int n = it.n0 + 16 * wave_row_tile<MODE>(wn, a) + 4 * (lane >> 4);
        if (n < g.rows)
          *reinterpret_cast<float4 *>(o_out + (int64_t)outrow[m] * g.rows + n) =
              make_float4(acc[a * 2 + ms][0], acc[a * 2 + ms][1], acc[a * 2 + ms][2],
                          acc[a * 2 + ms][3]);
      }
    }
  }
}

template <int MODE, int WF>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_kernel(GemmArgs g, coli_moe_route_t r, const int4 *__restrict__ tiles,
            const int *__restrict__ ntiles_p, int fixed_ntok, int fixed_expert, int T, int k,
            int n_ntiles, int64_t expert_stride_q, int64_t expert_stride_s,
            int8_t *__restrict__ qh_out, uint16_t *__restrict__ dh_out,
            float *__restrict__ o_out, int32_t *__restrict__ dots_out) {
  constexpr int NB = WF == kFmtF4 ? 2 : 1;
  __shared__ Stage<NB> st[2];
  __shared__ int rowid[BM];
  __shared__ int outrow[BM];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wid >> 1, wm = wid & 1;
  const int ntiles = tiles ? ntiles_p[0] : (fixed_ntok + BM - 1) / BM;
  const int items = band_items(ntiles, n_ntiles);
  const int nsteps = g.K / BK;
  // K steps rounded up to the prefetch depth; the extra steps are padding
  const int nsteps_pad = (nsteps + kDepth - 1) / kDepth * kDepth;
  // XCD-aware order: consecutive virtual ids (same weights) on one XCD
  const int G = gridDim.x;
  const int vid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  for (int item = vid; item < items; item += G) {
    int tile, ntile;
    item_coords(item, n_ntiles, tile, ntile);
    if (tile >= ntiles) continue;  // past the last tile of the last band
    const Item it = setup_item<MODE>(tile, ntile, tiles, fixed_ntok, fixed_expert, r, T, k,
                                     rowid, outrow);
    const int expert = it.expert, row0 = it.row0, ntok = it.ntok, n0 = it.n0;
    GemmArgs ge = g;
    ge.wq = g.wq + (int64_t)expert * expert_stride_q;
    ge.ws = g.ws + (int64_t)expert * expert_stride_s;

    Src src;
    {
      const int t = threadIdx.x;
      const uint16_t *s_row;
      weight_row<MODE>(ge, n0, 16 * (t >> 5) + (t & 15), src.w, s_row);
      src.w += (WF == kFmtI8 ? 32 : 16) * ((t >> 4) & 1);
      const int m = 16 * wid + (t & 15);
      const int qq = 2 * ((t >> 4) & 1) + ((t >> 5) & 1);
      src.a = ge.act + (int64_t)rowid[m] * ge.K + 16 * qq;
      if (MODE == kDots || wid < 2) {
        const uint8_t *unused;
        weight_row<MODE>(ge, n0, (MODE == kDots ? t & 127 : t), unused, src.s);
        src.s_step = 1;
        src.s_next = 0;
      } else {
        src.s = ge.act_d + (int64_t)rowid[(t - BR) & 63] * (ge.K / 32);
        src.s_step = 2;
        src.s_next = 1;
      }
    }

    float acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[a][i] = 0.0f;
    const coli_i32x4 magic = {(int)kMagic, (int)kMagic, (int)kMagic, (int)kMagic};

    // One K step on LDS stage `cur`: for each 32-block, 4 row tiles x 2
    // token tiles of MFMAs, then per output (D - M) * d as one FMA (exact
    // product, one rounding) and acc += s_w * that.  Folding both blocks'
    // offsets into one constant would save an FMA but leaves the sum
    // rounded at the offset's magnitude (~1.3e7 * d), about 500x coarser.
    auto step = [&](const Stage<NB> &cur, int ks) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        coli_i32x4 d[8];
        uint2 bop[2];
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) bop[ms] = cur.a[2 * wm + ms][blk][lane];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const uint2 aop = cur.w[wave_row_tile<MODE>(wn, a)][blk][lane];
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) d[a * 2 + ms] = mfma_i8(aop, bop[ms], magic);
        }
        if (MODE == kDots) {
          if (ks >= nsteps) continue;
          // exact block dots: (bits - magic) / 16, written [token][row][block]
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int ms = 0; ms < 2; ++ms) {
              const int m = 32 * wm + 16 * ms + (lane & 15);
              if (m >= ntok) continue;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int n = n0 + 16 * wave_row_tile<MODE>(wn, a) + 4 * (lane >> 4) + i;
                if (n >= g.rows) continue;
                dots_out[((int64_t)(row0 + m) * g.rows + n) * (g.K / 32) + 2 * ks + blk] =
                    (d[a * 2 + ms][i] - (int)kMagic) >> (WF == kFmtI4 ? 4 : 0);
              }
            }
        } else {
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) {
            const float2 sa = reinterpret_cast<const float2 *>(
                &cur.sa[32 * wm + 16 * ms + (lane & 15)])[blk];
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const float4 sw = *reinterpret_cast<const float4 *>(
                  &cur.sw[NB == 2 ? blk : 0][16 * wave_row_tile<MODE>(wn, a) + 4 * (lane >> 4)]);
              const float swv[4] = {sw.x, sw.y, sw.z, sw.w};
#pragma unroll
              for (int i = 0; i < 4; ++i)
                acc[a * 2 + ms][i] = fmaf(
                    swv[i], fmaf(__int_as_float(d[a * 2 + ms][i]), sa.x, sa.y), acc[a * 2 + ms][i]);
            }
          }
          // The accumulators are final for this block: without this the
          // compiler sinks every step's epilogue to the end of the unrolled
          // loop and keeps all of their MFMA results live at once.
#pragma unroll
          for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(acc[a][i]));
        }
      }
    };

    // Pipeline: a register ring holds the raw global data of the next
    // kDepth steps (loads in flight), LDS holds two unpacked stages.  Step
    // ks computes on stage ks & 1, refills the ring slot it freed with step
    // ks + kDepth (clamped to the last step, so every load is in bounds and
    // unconditional), and unpacks step ks + 1 into the other stage.
    Prefetch<WF> pf[kDepth];
#pragma unroll
    for (int i = 0; i < kDepth; ++i) load_step<WF>(src, min(i, nsteps - 1), pf[i]);
    store_step<MODE, WF>(pf[0], st[0], wid, true);
    __syncthreads();
    for (int ks0 = 0; ks0 < nsteps_pad; ks0 += kDepth) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int ks = ks0 + u;
        load_step<WF>(src, min(ks + kDepth, nsteps - 1), pf[u]);
        step(st[u & 1], ks);
        store_step<MODE, WF>(pf[(u + 1) % kDepth], st[(u + 1) & 1], wid, ks + 1 < nsteps);
        __syncthreads();
      }
    }

    epilogue<MODE>(acc, g, it, outrow, wn, wm, lane, qh_out, dh_out, o_out);
  }
}

// ----------------------------------------------- GEMM, K a multiple of 256

// The same work items, epilogues and arithmetic as gemm_kernel, with one
// LDS stage holding four K steps (256 k).  Global loads then move whole
// 128-byte lines: per 16-byte load instruction a wavefront covers 8 weight
// rows x 128 bytes (4 steps of one row) or 4 token rows x 256 bytes, and the
// scales of 4 steps arrive in one 8-byte load per thread.  That keeps the
// number of distinct cache lines a wavefront touches per K step low, which
// is what the per-step loads of gemm_kernel are limited by.  One group of
// loads is in flight while the previous group is computed; two barriers per
// group.
constexpr int kGroup = 4;   // K steps per LDS stage
// NB: weight scales per step, 1 (a 64-weight group) or 2 (one per 32-block)
template <int NB>
struct Stage4 {
  uint2 w[BR / 16][kGroup][2][64];  // [row tile][step][32-block][lane ^ swz]
  uint2 a[BM / 16][kGroup][2][64];  // [token tile][step][32-block][lane ^ swz]
  float sw[kGroup * NB][BR];        // weight scales: [step] or [2 * step + block]
  float2 sa[kGroup][BM];            // d0/16, d1/16 of each token
};
// Operand entry e of the tile of (step s, block b) sits at e ^ swz(s, b).
// The XOR permutes each tile, so a wavefront reading all 64 entries still
// reads one contiguous 512-byte tile; the unpacking writes, where the lanes
// of a half-wavefront cover 8 (step, block) pairs x 4 consecutive entries,
// land on 32 distinct 8-byte bank pairs.  (52.5 KB per workgroup: three
// workgroups per compute unit.)
COLI_DEV int swz(int s, int b) { return 4 * (2 * s + b); }

// Per thread: four 16-byte weight loads (load j: row 32*wave + 8j +
// 4*(lane>>5) + (lane&3), 16-byte chunk (lane>>2)&7 of the row's 128 bytes),
// four 16-byte activation loads (load j: token 16*wave + 4j + (lane&3),
// chunk 4*step + quarter of the token's 256 bytes with step (lane>>2)&3 and
// quarter 2*((lane>>4)&1) + (lane>>5)), and one 8-byte scale load.
struct Src4 {
  const uint8_t *wbase;  // the expert's matrix (wave-uniform)
  const int8_t *abase;   // activation rows (wave-uniform)
  uint32_t w[4];         // byte offsets of the four weight loads from wbase
  uint32_t a[4];         // byte offsets of the four activation loads from abase
  const uint16_t *s;
  int s_group;  // scale elements per group: 4 (a weight row) or 8 (a token)
};
// W8: int8 codes, 256 bytes of a row per stage instead of 128, so each of
// the four weight loads is a pair of 16-byte loads (both halves of one
// 32-block); the stage holds the codes as they are.
template <bool W8>
struct Group4 {
  uint4 w[4][W8 ? 2 : 1], a[4];
  uint2 s;
};

template <bool W8>
COLI_DEV void load_group(const Src4 &src, int gi, Group4<W8> &G) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < (W8 ? 2 : 1); ++h)
      G.w[j][h] = *reinterpret_cast<const uint4 *>(src.wbase +
                                                   (src.w[j] + gi * (W8 ? 256 : 128) + 16 * h));
#pragma unroll
  for (int j = 0; j < 4; ++j)
    G.a[j] = *reinterpret_cast<const uint4 *>(src.abase + (src.a[j] + gi * 256));
  G.s = *reinterpret_cast<const uint2 *>(src.s + gi * src.s_group);
}

// Registers -> LDS.  Within each half-wavefront the 8-byte writes land on
// distinct banks: lane bits 0-1 pick consecutive entries and the (step,
// block) pair moves the address by a multiple of 4 entries (mod 32).
template <int MODE, int WF, int NB>
COLI_DEV void store_group(const Group4<WF == kFmtI8> &G, Stage4<NB> &st, int wid) {
  constexpr bool W8 = WF == kFmtI8;
  const int l = threadIdx.x & 63;
  {
    const int c = (l >> 2) & 7, s = c >> 1, b = c & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rt = 2 * wid + (j >> 1), rr = 8 * (j & 1) + 4 * (l >> 5) + (l & 3);
      if (W8) {  // k-quarters 2h and 2h + 1 of the 32-block
#pragma unroll
        for (int h = 0; h < (W8 ? 2 : 1); ++h) {
          const uint4 v = G.w[j][h];
          st.w[rt][s][b][(rr + 16 * (2 * h)) ^ swz(s, b)] = make_uint2(v.x, v.y);
          st.w[rt][s][b][(rr + 16 * (2 * h + 1)) ^ swz(s, b)] = make_uint2(v.z, v.w);
        }
        continue;
      }
      const uint32_t w[4] = {G.w[j][0].x, G.w[j][0].y, G.w[j][0].z, G.w[j][0].w};
      if (WF == kFmtF4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t lo, hi;
          fp4x8_to_i8(w[i], lo, hi);
          st.w[rt][s][b][(rr + 16 * i) ^ swz(s, b)] = make_uint2(lo, hi);
        }
        continue;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t even = (w[i] << 4) & 0xf0f0f0f0u;  // k 0,2,4,6 (x16)
        const uint32_t odd = w[i] & 0xf0f0f0f0u;          // k 1,3,5,7 (x16)
        st.w[rt][s][b][(rr + 16 * i) ^ swz(s, b)] =
            make_uint2(__builtin_amdgcn_perm(odd, even, 0x05010400u),
                       __builtin_amdgcn_perm(odd, even, 0x07030602u));
      }
    }
  }
  {
    const int s = (l >> 2) & 3, blk = (l >> 4) & 1, j0 = 2 * (l >> 5);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mm = 4 * j + (l & 3);
      st.a[wid][s][blk][(mm + 16 * j0) ^ swz(s, blk)] = make_uint2(G.a[j].x, G.a[j].y);
      st.a[wid][s][blk][(mm + 16 * (j0 + 1)) ^ swz(s, blk)] = make_uint2(G.a[j].z, G.a[j].w);
    }
  }
  if (MODE == kDots) return;
  const int t = threadIdx.x;
  const uint16_t h[4] = {(uint16_t)G.s.x, (uint16_t)(G.s.x >> 16), (uint16_t)G.s.y,
                         (uint16_t)(G.s.y >> 16)};
  if (wid < 2) {  // weight row t: the scales of steps 0..3
    if (WF == kFmtF4) {  // 8 E8M0 bytes, block 2s + b; 2^(E-128) for the doubled codes
      const uint32_t e[2] = {G.s.x, G.s.y};
#pragma unroll
      for (int q = 0; q < 2 * kGroup; ++q) {
        const uint32_t E = (e[q >> 2] >> (8 * (q & 3))) & 0xffu;
        st.sw[q][t] = __uint_as_float(E > 1 ? (E - 1) << 23 : (0x00400000u >> (1 - E)));
      }
    } else {
#pragma unroll
      for (int s = 0; s < kGroup; ++s) st.sw[s][t] = f16_to_f32(h[s]);
    }
  } else {  // token (t-128)/2: steps 2*(t&1) and 2*(t&1)+1, two blocks each
    // int4 codes sit in the stage x16: their activation scales carry 1/16
    constexpr float f = WF == kFmtI4 ? 0.0625f : 1.0f;
    const int m = (t - BR) >> 1, s0 = 2 * (t & 1);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      st.sa[s0 + u][m] = make_float2(f16_to_f32(h[2 * u]) * f, f16_to_f32(h[2 * u + 1]) * f);
  }
}

template <int MODE, int WF>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm4_kernel(GemmArgs g, coli_moe_route_t r, const int4 *__restrict__ tiles,
             const int *__restrict__ ntiles_p, int fixed_ntok, int fixed_expert, int T, int k,
             int n_ntiles, int64_t expert_stride_q, int64_t expert_stride_s,
             int8_t *__restrict__ qh_out, uint16_t *__restrict__ dh_out,
             float *__restrict__ o_out, int32_t *__restrict__ dots_out) {
  constexpr bool W8 = WF == kFmtI8;
  constexpr int NB = WF == kFmtF4 ? 2 : 1;
  __shared__ Stage4<NB> st;
  __shared__ int rowid[BM];
  __shared__ int outrow[BM];
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wid >> 1, wm = wid & 1;
  const int ntiles = tiles ? ntiles_p[0] : (fixed_ntok + BM - 1) / BM;
  const int items = band_items(ntiles, n_ntiles);
  const int ngroups = g.K / (kGroup * BK);
  const int G = gridDim.x;
  const int vid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;

  for (int item = vid; item < items; item += G) {
    int tile, ntile;
    item_coords(item, n_ntiles, tile, ntile);
    if (tile >= ntiles) continue;  // past the last tile of the last band
    const Item it = setup_item<MODE>(tile, ntile, tiles, fixed_ntok, fixed_expert, r, T, k,
                                     rowid, outrow);
    GemmArgs ge = g;
    ge.wq = g.wq + (int64_t)it.expert * expert_stride_q;
    ge.ws = g.ws + (int64_t)it.expert * expert_stride_s;

    Src4 src;
    {
      const int t = threadIdx.x;
      const uint16_t *unused;
      src.wbase = ge.wq;
      src.abase = ge.act;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint8_t *q;
        weight_row<MODE>(ge, it.n0, 32 * wid + 8 * j + 4 * (lane >> 5) + (lane & 3), q, unused);
        src.w[j] = (uint32_t)(q - ge.wq) + (W8 ? 32 : 16) * ((lane >> 2) & 7);
        const int m = 16 * wid + 4 * j + (lane & 3);
        const int c = 4 * ((lane >> 2) & 3) + 2 * ((lane >> 4) & 1) + (lane >> 5);
        src.a[j] = (uint32_t)rowid[m] * (uint32_t)ge.K + 16 * c;
      }
      if (MODE == kDots || wid < 2) {
        const uint8_t *unused_q;
        weight_row<MODE>(ge, it.n0, t & 127, unused_q, src.s);
        src.s_group = kGroup;
      } else {
        src.s = ge.act_d + (int64_t)rowid[(t - BR) >> 1] * (ge.K / 32) + 4 * (t & 1);
        src.s_group = 2 * kGroup;
      }
    }

    float acc[8][4];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[a][i] = 0.0f;
    coli_i32x4 magic = {(int)kMagic, (int)kMagic, (int)kMagic, (int)kMagic};
    // held in registers (not rebuilt from a constant before every MFMA)
    asm volatile("" : "+v"(magic));

    // The 8 (step, 32-block) blocks of a stage run as a software pipeline:
    // while block q's epilogue runs on the vector ALUs, block q+1's MFMAs run
    // on the matrix core and block q+2's operands are on their way from LDS.
    // Each step's scales are read with the operands of its first block.
    struct Ops {
      uint2 a[4], b[2];
    };
    struct Scl {
      float w[4][4];
      float d[2][2];
    };
    auto load_ops = [&](int q, Ops &o) {
      const int s = q >> 1, blk = q & 1;
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) o.b[ms] = st.a[2 * wm + ms][s][blk][lane ^ swz(s, blk)];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        o.a[a] = st.w[wave_row_tile<MODE>(wn, a)][s][blk][lane ^ swz(s, blk)];
    };
    // scales of block q (NB = 2) or of step q (NB = 1); activations by step
    auto load_scl = [&](int q, Scl &c) {
      if (MODE == kDots) return;
      const int s = NB == 2 ? q >> 1 : q;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float4 w4 = *reinterpret_cast<const float4 *>(
            &st.sw[q][16 * wave_row_tile<MODE>(wn, a) + 4 * (lane >> 4)]);
        c.w[a][0] = w4.x, c.w[a][1] = w4.y, c.w[a][2] = w4.z, c.w[a][3] = w4.w;
      }
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) {
        const float2 d2 = st.sa[s][32 * wm + 16 * ms + (lane & 15)];
        c.d[ms][0] = d2.x, c.d[ms][1] = d2.y;
      }
    };
    auto mfmas = [&](const Ops &o, coli_i32x4 (&d)[8]) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) d[a * 2 + ms] = mfma_i8(o.a[a], o.b[ms], magic);
    };
    // block q of group gi: epilogue (or, for the block-dot export, the dots)
    auto finish = [&](int gi, int q, const Scl &c, const coli_i32x4 (&d)[8]) {
      const int blk = q & 1, ks = kGroup * gi + (q >> 1);
      if (MODE == kDots) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int ms = 0; ms < 2; ++ms) {
            const int m = 32 * wm + 16 * ms + (lane & 15);
            if (m >= it.ntok) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int n = it.n0 + 16 * wave_row_tile<MODE>(wn, a) + 4 * (lane >> 4) + i;
              if (n >= g.rows) continue;
              dots_out[((int64_t)(it.row0 + m) * g.rows + n) * (g.K / 32) + 2 * ks + blk] =
                  (d[a * 2 + ms][i] - (int)kMagic) >> (WF == kFmtI4 ? 4 : 0);
            }
          }
      } else {
#pragma unroll
        for (int ms = 0; ms < 2; ++ms) {
          const float da = c.d[ms][blk], ca = -kMagicF * da;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[a * 2 + ms][i] = fmaf(c.w[a][i], fmaf(__int_as_float(d[a * 2 + ms][i]), da, ca),
                                        acc[a * 2 + ms][i]);
        }
        // keep this block's epilogue here (see gemm_kernel)
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(acc[a][i]));
      }
    };
    auto compute_stage = [&](int gi) {
      Ops o0, o1;
      Scl c0, c1;
      coli_i32x4 d0[8], d1[8];
      load_scl(0, c0);
      load_ops(0, o0);
      load_ops(1, o1);
      mfmas(o0, d0);
#pragma unroll
      for (int q = 0; q < 2 * kGroup; ++q) {
        // block q's results are in d[q & 1], block q+1's operands in o[(q+1) & 1]
        if (q + 1 < 2 * kGroup) mfmas((q & 1) ? o0 : o1, (q & 1) ? d0 : d1);
        if (q + 2 < 2 * kGroup) load_ops(q + 2, (q & 1) ? o1 : o0);
        if (NB == 2) {  // one scale set per block: block q + 1's next
          if (q + 1 < 2 * kGroup) load_scl(q + 1, (q & 1) ? c0 : c1);
          finish(gi, q, (q & 1) ? c1 : c0, (q & 1) ? d1 : d0);
        } else {        // one per step: step s + 1's during step s's first block
          if ((q & 1) == 0 && q + 2 < 2 * kGroup) load_scl((q >> 1) + 1, ((q >> 1) & 1) ? c0 : c1);
          finish(gi, q, ((q >> 1) & 1) ? c1 : c0, (q & 1) ? d1 : d0);
        }
      }
    };

    Group4<W8> grp;
    load_group(src, 0, grp);
    store_group<MODE, WF, NB>(grp, st, wid);
    __syncthreads();
    if (ngroups > 1) load_group(src, 1, grp);
    for (int gi = 0; gi < ngroups; ++gi) {
      compute_stage(gi);
      if (gi + 1 < ngroups) {
        __syncthreads();  // every wavefront is done with the stage
        store_group<MODE, WF, NB>(grp, st, wid);
        __syncthreads();
        if (gi + 2 < ngroups) load_group(src, gi + 2, grp);
      }
    }
    epilogue<MODE>(acc, g, it, outrow, wn, wm, lane, qh_out, dh_out, o_out);
  }
}

// ------------------------------------ GEMM from DMA-filled stages (int4)
//
// The same work items and arithmetic as gemm4_kernel, arranged for the
// vector ALUs, which bound this contraction: every output needs two fp32
// FMAs per 32-block (activation scale with the offset removed, then the
// weight scale), against 1/16 of a matrix-core instruction.
//  * Stages of 256 k are copied global -> LDS with global_load_lds (the
//    data never passes through registers): 128 weight rows of nibbles
//    (16 KB), the tile's 64 token rows of int8 activations (16 KB), the
//    rows' fp16 group scales and the tokens' block records {-M*d, d}.  Two
//    stages alternate, so one is loading while the other is computed.
//  * Wave w computes weight rows [16w, 16w+16) and [64+16w, 64+16w+16) (for
//    gate/up: gate and up of the same 16 channels) against each 16-token
//    subtile that holds a token; empty subtiles are skipped (templated on
//    their count), so a tile of n tokens costs ceil(n/16) subtiles.
//  * The nibbles are unpacked as each wave reads its operand: a dword of 8
//    codes gives (w << 4) & 0xf0f0f0f0 (k 0,2,4,6 times 16) and w &
//    0xf0f0f0f0 (k 1,3,5,7 times 16).  The activations are stored in that
//    order within every 8 values ([x0 x2 x4 x6 x1 x3 x5 x7]) by whoever
//    writes them (the Q8_0 kernel for x, the gate/up epilogue for h), so
//    the pairing of weights and activations, and every block dot, is exact.
//  * LDS layouts are XOR-swizzled at 16-byte granularity so that each DMA
//    instruction moves whole 128-byte lines and each operand read is free
//    of bank conflicts: weight row r keeps block c at chunk c ^ ((r>>1)&7),
//    token t keeps its 16-byte piece j at j ^ (t & 15).
constexpr int kSK = 256;            // k per stage
constexpr int kSB = kSK / 32;       // 32-blocks per stage
#define COLI_LDS __attribute__((address_space(3)))

struct DStage {
  uint4 w[BR * 8];   // [row][chunk]: 16 B of nibbles = one 32-block of one row
  uint4 a[BM * 16];  // [token][chunk]: 16 B of int8 = half a 32-block
  uint2 sw[BR];      // [row]: fp16 scales of the stage's four 64-groups
  uint4 sa[BM * 4];  // [token][pair]: records {c, d} of blocks 2p and 2p+1
};

// global -> LDS, 16 (or 4) bytes per lane; lane i lands at lds + 16*i (4*i).
COLI_DEV void dma16(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (COLI_LDS void *)lds, 16, 0, 0);
}
COLI_DEV void dma4(const void *g, void *lds) {
  __builtin_amdgcn_global_load_lds(g, (COLI_LDS void *)lds, 4, 0, 0);
}
COLI_DEV void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Per-lane DMA sources of a work item; a stage adds a fixed byte step.
struct DSrc {
  const uint8_t *w[4];  // weight chunk of instruction 4*wave + j (step 128 B)
  const int8_t *a[4];   // activation chunk of instruction 4*wave + j (step 256 B)
  const uint8_t *sw;    // 4 bytes of scales (step 8 B)
  const uint8_t *sa;    // 16 bytes of records (step 64 B)
};

// Natural-order 8 int8 values (lo = k0..3, hi = k4..7) -> the even/odd
// order of the unpacked nibbles: [k0 k2 k4 k6], [k1 k3 k5 k7].
COLI_DEV uint2 even_odd8(uint32_t lo, uint32_t hi) {
  return make_uint2(__builtin_amdgcn_perm(hi, lo, 0x06040200u),
                    __builtin_amdgcn_perm(hi, lo, 0x07050301u));
}

template <int MODE, int NTS>
COLI_DEV void dgemm_item(const GemmArgs &g, const Item &it, const int *rowid, const int *outrow,
                         const uint8_t *wq, const uint16_t *ws, const float2 *rec,
                         DStage &B0, DStage &B1, float (*xch)[4][16], int8_t *qh_out,
                         float2 *rech_out, float *o_out, int32_t *dots_out) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = lane >> 4, lr = lane & 15;
  const int nst = g.K / kSK;

  // ---- DMA sources of this lane
  DSrc src;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // weights: instruction q = 4*wave + j covers item rows 8q..8q+7
    const int row = 32 * wv + 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const uint8_t *q;
    const uint16_t *unused;
    weight_row<MODE == kDots ? kDown : MODE>(g, it.n0, row, q, unused);
    src.w[j] = q + 16 * chunk;
    // activations: instruction q covers tokens 4q..4q+3
    const int t = 16 * wv + 4 * j + (lane >> 4);
    src.a[j] = g.act + (int64_t)rowid[t] * g.K + 16 * ((lane & 15) ^ (t & 15));
  }
  {
    const int row = 32 * wv + (lane >> 1);
    const uint8_t *unused;
    const uint16_t *s;
    weight_row<MODE == kDots ? kDown : MODE>(g, it.n0, row, unused, s);
    src.sw = reinterpret_cast<const uint8_t *>(s) + 4 * (lane & 1);
    // record pairs are stored at position pair ^ ((t >> 2) & 3): the 16
    // tokens a read covers then fall on distinct 16-byte bank groups
    const int t = 16 * wv + (lane >> 2);
    src.sa = reinterpret_cast<const uint8_t *>(rec + (int64_t)rowid[t] * (g.K / 32)) +
             16 * ((lane & 3) ^ ((t >> 2) & 3));
  }
  (void)wq;
  (void)ws;
  // DMA instruction p (0..9) of a stage: 4 of weights, 4 of activations,
  // the scales and the records.  A stage's ten are spread over the blocks
  // of the previous stage's compute, so no wavefront stalls behind a burst
  // of them on the memory pipeline while it has arithmetic to issue.
  // Wave wv moves the activations and records of tokens 16wv..16wv+15, so
  // the waves past the tile's last 16-token subtile move none.
  const bool tok_live = wv < NTS;
  auto issue_part = [&](DStage &B, int st, int p) {
    if (p < 4) {
      dma16(src.w[p] + st * (kSK / 2), &B.w[(4 * wv + p) * 64]);
    } else if (p < 8) {
      if (tok_live) dma16(src.a[p - 4] + st * kSK, &B.a[(4 * wv + p - 4) * 64]);
    } else if (MODE != kDots) {
      if (p == 8) dma4(src.sw + st * 8, reinterpret_cast<uint8_t *>(B.sw) + 256 * wv);
      else if (tok_live) dma16(src.sa + st * 64, &B.sa[64 * wv]);
    }
  };
  auto issue = [&](DStage &B, int st) {
#pragma unroll
    for (int p = 0; p < 10; ++p) issue_part(B, st, p);
  };

  float acc[2][NTS][4];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rs][ts][i] = 0.0f;
  coli_i32x4 magic = {(int)kMagic, (int)kMagic, (int)kMagic, (int)kMagic};
  asm volatile("" : "+v"(magic));

  // per-lane LDS byte offsets of the operand reads (before the block XOR)
  const int rA = 16 * wv + lr;                               // row of subtile 0
  const uint32_t offA = rA * 128 + 16 * ((rA >> 1) & 7) + 4 * kq;  // ^ 16*b
  const uint32_t offB = lr * 256 + 16 * ((kq >> 1) ^ lr) + 8 * (kq & 1);  // ^ 32*b
  const int rS = 16 * wv + 4 * kq;                            // first row of the lane's scales

  struct Ops {
    long a[2], b[NTS];
  };
  // LDS reads of block b's operands (raw nibble words and activation
  // pairs), then their unpacking into MFMA operands: split so that the
  // previous block's scale FMAs can run while the reads are in flight
  struct Raw {
    uint32_t w[2];
    uint2 v[NTS];
  };
  auto load_ops = [&](const DStage &B, int b, Raw &rw) {
    const char *wb = reinterpret_cast<const char *>(B.w) + (offA ^ (16 * b));
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) rw.w[rs] = *reinterpret_cast<const uint32_t *>(wb + rs * 64 * 128);
    const char *ab = reinterpret_cast<const char *>(B.a) + (offB ^ (32 * b));
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) rw.v[ts] = *reinterpret_cast<const uint2 *>(ab + ts * 16 * 256);
  };
  auto unpack_ops = [&](const Raw &rw, Ops &o) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) {
      const uint32_t x = rw.w[rs];
      const uint32_t ev = (x << 4) & 0xf0f0f0f0u, od = x & 0xf0f0f0f0u;
      o.a[rs] = (long)(((uint64_t)od << 32) | ev);
    }
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      uint2 v = rw.v[ts];
      if (MODE == kDots) v = even_odd8(v.x, v.y);  // caller's codes are in natural order
      o.b[ts] = (long)(((uint64_t)v.y << 32) | v.x);
    }
  };
  auto mfmas = [&](const Ops &o, coli_i32x4 (&d)[2][NTS]) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int ts = 0; ts < NTS; ++ts)
        d[rs][ts] = __builtin_amdgcn_mfma_i32_16x16x32_i8(o.a[rs], o.b[ts], magic, 0, 0, 0);
  };
  // weight scales of group gq for the lane's 8 rows (from the stage's fp16
  // scales, read once per stage), and the token records of the group
  struct Scl {
    float w[2][4];
    float4 r[NTS];  // {c, d} of the group's two blocks
  };
  uint4 swh[2][2];  // [rs][rows 4kq+{0,1} | 4kq+{2,3}]: 4 fp16 each
  auto read_sw = [&](const DStage &B) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        swh[rs][h] = *reinterpret_cast<const uint4 *>(&B.sw[rS + 64 * rs + 2 * h]);
  };
  const int fsa = (lr >> 2) & 3;
  auto read_scl = [&](const DStage &B, int gq, Scl &c) {
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 q = swh[rs][i >> 1];
        const uint32_t hw = (i & 1) ? ((gq & 2) ? q.w : q.z) : ((gq & 2) ? q.y : q.x);
        c.w[rs][i] = f16_to_f32((uint16_t)((gq & 1) ? hw >> 16 : hw));
        // kept as fp32 values: folded into the FMAs as v_fma_mix_f32 (mixed
        // fp16 operand) the compiler would issue at a lower rate
        asm volatile("" : "+v"(c.w[rs][i]));
      }
    const uint4 *sa = &B.sa[lr * 4 + (gq ^ fsa)];
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const uint4 v = sa[ts * 64];
      c.r[ts] = make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
                            __uint_as_float(v.w));
    }
  };
  auto finish = [&](int st, int b, const Scl &c, const coli_i32x4 (&d)[2][NTS]) {
    if (MODE == kDots) {
#pragma unroll
      for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int ts = 0; ts < NTS; ++ts) {
          const int m = 16 * ts + lr;
          if (m >= it.ntok) continue;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int n = it.n0 + 16 * wv + 64 * rs + 4 * kq + i;
            if (n >= g.rows) continue;
            dots_out[((int64_t)(it.row0 + m) * g.rows + n) * (g.K / 32) + kSB * st + b] =
                (d[rs][ts][i] - (int)kMagic) >> 4;
          }
        }
      return;
    }
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const float cc = (b & 1) ? c.r[ts].z : c.r[ts].x;
      const float dd = (b & 1) ? c.r[ts].w : c.r[ts].y;
#pragma unroll
      for (int rs = 0; rs < 2; ++rs)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[rs][ts][i] =
              fmaf(c.w[rs][i], fmaf(__int_as_float(d[rs][ts][i]), dd, cc), acc[rs][ts][i]);
    }
#pragma unroll
    for (int rs = 0; rs < 2; ++rs)
#pragma unroll
      for (int ts = 0; ts < NTS; ++ts)
#pragma unroll
        for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(acc[rs][ts][i]));
  };
  // one stage: block b's MFMAs run while block b-1's epilogue runs; the
  // next stage's DMA (into `N`, if `nxt` >= 0) is issued along the way
  auto compute = [&](const DStage &B, int st, DStage &N, int nxt) {
    Ops o;
    Raw rw;
    Scl c0, c1;
    coli_i32x4 d0[2][NTS], d1[2][NTS];
    load_ops(B, 0, rw);
    unpack_ops(rw, o);
    if (MODE != kDots) {
      read_sw(B);
      read_scl(B, 0, c0);
    }
    mfmas(o, d0);
#pragma unroll
    for (int b = 0; b < kSB; ++b) {
      if (nxt >= 0) {
        issue_part(N, nxt, b);
        if (b < 2) issue_part(N, nxt, 8 + b);
      }
      // order within a block: next block's LDS reads, this block's scale
      // FMAs (which cover the read latency), then the next block's unpack
      // and MFMAs; the scheduling barriers keep the compiler from hoisting
      // the unpack (and with it the LDS wait) above the FMAs
      if (b + 1 < kSB) {
        load_ops(B, b + 1, rw);
        if (MODE != kDots && ((b + 1) & 1) == 0) read_scl(B, (b + 1) >> 1, ((b >> 1) & 1) ? c0 : c1);
      }
      __builtin_amdgcn_sched_barrier(0);
      finish(st, b, ((b >> 1) & 1) ? c1 : c0, (b & 1) ? d1 : d0);
      __builtin_amdgcn_sched_barrier(0);
      if (b + 1 < kSB) {
        unpack_ops(rw, o);
        mfmas(o, (b & 1) ? d0 : d1);
      }
    }
  };

  issue(B0, 0);
  wait_dma();
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    compute(B0, st, B1, st + 1 < nst ? st + 1 : -1);
    wait_dma();
    __syncthreads();
    if (st + 1 >= nst) break;
    compute(B1, st + 1, B0, st + 2 < nst ? st + 2 : -1);
    wait_dma();
    __syncthreads();
  }

  // ---- epilogue
  if (MODE == kGateUp) {
    // h = silu(g) * u for channels n0 + 16*wv + 4*kq + i; the codes are in
    // units of 16 (x16 nibbles), removed here exactly.  Q8_0 of h per 32
    // channels: waves 2p and 2p+1 hold the two halves of block p.
    float hv[NTS][4];
    float am[NTS];
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[ts][i] = silu_mul(acc[0][ts][i] * 0.0625f, acc[1][ts][i] * 0.0625f);
        a = fmaxf(a, fabsf(hv[ts][i]));
      }
      a = fmaxf(a, __shfl_xor(a, 16, 64));
      a = fmaxf(a, __shfl_xor(a, 32, 64));
      am[ts] = a;
      if (kq == 0) xch[wv][ts][lr] = a;
    }
    __syncthreads();
    const int I = g.rows;
    const int ch0 = it.n0 + 16 * wv;  // first channel of this wave
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const float amax = fmaxf(am[ts], xch[wv ^ 1][ts][lr]);
      const float dq = __fdiv_rn(amax, 127.0f);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int q = 0;
        if (amax != 0.0f) {
          q = (int)roundf(__fdiv_rn(hv[ts][i], dq));
          q = max(-127, min(127, q));
        }
        packed |= (uint32_t)(q & 0xff) << (8 * i);
      }
      // lanes kq = 2m, 2m+1 hold channels 8m..8m+3 and 8m+4..8m+7; write
      // them as [c0 c2 c4 c6] and [c1 c3 c5 c7]
      const uint32_t e = __builtin_amdgcn_perm(packed, packed, 0x03010200u);  // q0 q2 q1 q3
      const uint32_t p = (uint32_t)__shfl_xor((int)e, 16, 64);
      const uint32_t out = (kq & 1) ? ((p >> 16) | (e & 0xffff0000u)) : ((e & 0xffffu) | (p << 16));
      const int m = 16 * ts + lr;
      if (m < it.ntok && ch0 < I) {
        const int64_t orow = outrow[m];
        *reinterpret_cast<uint32_t *>(qh_out + orow * I + ch0 + 4 * kq) = out;
        if ((wv & 1) == 0 && kq == 0) {
          const float d16 = f16_to_f32(f32_to_f16_bits(dq));
          rech_out[orow * (I / 32) + ch0 / 32] = make_float2(-kMagicF * d16, d16);
        }
      }
    }
  } else if (MODE == kDown) {
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const int m = 16 * ts + lr;
      if (m >= it.ntok) continue;
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        const int n = it.n0 + 16 * wv + 64 * rs + 4 * kq;
        if (n < g.rows)
          *reinterpret_cast<float4 *>(o_out + (int64_t)outrow[m] * g.rows + n) =
              make_float4(acc[rs][ts][0] * 0.0625f, acc[rs][ts][1] * 0.0625f,
                          acc[rs][ts][2] * 0.0625f, acc[rs][ts][3] * 0.0625f);
      }
    }
  }
}

template <int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
dgemm_kernel(GemmArgs g, coli_moe_route_t r, const int4 *__restrict__ tiles,
             const int *__restrict__ ntiles_p, int fixed_ntok, int fixed_expert, int T, int k,
             int n_ntiles, int64_t expert_stride_q, int64_t expert_stride_s,
             const float2 *__restrict__ rec, int8_t *__restrict__ qh_out,
             float2 *__restrict__ rech_out, float *__restrict__ o_out,
             int32_t *__restrict__ dots_out) {
  __shared__ DStage B0;
  __shared__ DStage B1;
  __shared__ int rowid[BM];
  __shared__ int outrow[BM];
  __shared__ float xch[4][4][16];
  const int ntiles = tiles ? ntiles_p[0] : (fixed_ntok + BM - 1) / BM;
  const int items = band_items(ntiles, n_ntiles);
  const int G = gridDim.x;
  const int vid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int item = vid; item < items; item += G) {
    int tile, ntile;
    item_coords(item, n_ntiles, tile, ntile);
    if (tile >= ntiles) continue;
    const Item it = setup_item<MODE>(tile, ntile, tiles, fixed_ntok, fixed_expert, r, T, k,
                                     rowid, outrow);
    GemmArgs ge = g;
    ge.wq = g.wq + (int64_t)it.expert * expert_stride_q;
    ge.ws = g.ws + (int64_t)it.expert * expert_stride_s;
    const int nts = (it.ntok + 15) >> 4;
    switch (nts) {
      case 1:
        dgemm_item<MODE, 1>(ge, it, rowid, outrow, ge.wq, ge.ws, rec, B0, B1, xch, qh_out,
                            rech_out, o_out, dots_out);
        break;
      case 2:
        dgemm_item<MODE, 2>(ge, it, rowid, outrow, ge.wq, ge.ws, rec, B0, B1, xch, qh_out,
                            rech_out, o_out, dots_out);
        break;
      case 3:
        dgemm_item<MODE, 3>(ge, it, rowid, outrow, ge.wq, ge.ws, rec, B0, B1, xch, qh_out,
                            rech_out, o_out, dots_out);
        break;
      default:
        dgemm_item<MODE, 4>(ge, it, rowid, outrow, ge.wq, ge.ws, rec, B0, B1, xch, qh_out,
                            rech_out, o_out, dots_out);
        break;
    }
  }
}

// ------------------------------------------ MX path: MXFP4 x MXFP8 on the MX matrix cores
//
// Layers flagged COLI_ACT_MXFP8 (MXFP4 weights) quantise the activations to
// MXFP8 -- FP8 E4M3 codes with one E8M0 scale per 32 values, the OCP
// microscaling format of the weights -- and run both GEMMs on
// v_mfma_scale_f32_16x16x128_f8f6f4, which applies the two E8M0 scales of
// every 32-block itself: there is no per-block epilogue on the vector ALUs.
//
// Operand layout of the instruction (measured on the GPU with an in-bounds
// probe): lane l = r + 16 g holds row (or column) r.  An FP4 operand holds
// k in [32g, 32g + 32) as 16 bytes, low nibble first; an FP8 operand holds
// k in [16g, 16g + 16) in bytes 0..15 and k in [64 + 16g, 64 + 16g + 16) in
// bytes 16..31.  Lane l's scale byte belongs to row r and the 32-block g.
// The result tile is laid out as in the other 16x16 instructions; one
// instruction covers 128 k.
typedef int coli_i32x8 __attribute__((ext_vector_type(8)));
typedef float coli_f32x4v __attribute__((ext_vector_type(4)));

// E8M0 shared exponent of a 32-block with maximum magnitude amax:
// floor(log2 amax) - 8 (the largest E4M3 exponent) + 127, clamped to
// [0, 254]; 0 for an all-zero block.  floor(log2) comes from the fp32
// exponent field; a subnormal amax clamps to 0 anyway.
COLI_DEV uint32_t mx8_exponent(float amax) {
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xffu);  // biased; 0 for 0 / subnormal
  const int E = ex - 127 - 8 + 127;
  return amax > 0.0f ? (uint32_t)max(0, min(254, E)) : 0u;
}

// E4M3 code of v / 2^(E-127) (v fp32), nearest with ties to the even code,
// saturating at 448, sign kept (also for zero).  The scaled magnitude m is
// exact (a power-of-two scaling; only values far below the smallest code
// can lose bits, and they code 0 either way).
COLI_DEV uint32_t mx8_code(float v, uint32_t E) {
  // 2^(127 - E) is a normal fp32 number for E <= 253; fp32 inputs give E <= 246
  const float m = E <= 253 ? fabsf(v) * __uint_as_float((254u - E) << 23)
                           : fabsf(v) * 0x1p-126f * 0.5f;
  uint32_t c;
  if (m >= 448.0f) {
    c = 0x7e;
  } else if (m < 0x1p-6f) {            // subnormal codes: m / 2^-9, nearest even
    c = (uint32_t)rintf(m * 512.0f);   // 8 = 2^-6, the smallest normal code
  } else {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu) - 127;  // 2^e <= m
    uint32_t r = (uint32_t)rintf(m * __uint_as_float((uint32_t)(127 + 3 - e) << 23));  // 8..16
    int ee = e;
    if (r == 16) {
      r = 8;
      ++ee;
    }
    c = ((uint32_t)(ee + 7) << 3) | (r - 8);
  }
  return c | ((__float_as_uint(v) >> 24) & 0x80u);
}

// MXFP8 of n values (n % 32 == 0), one thread per 32-block: codes [n], E8M0 [n / 32].
__global__ void __launch_bounds__(kThreads) quantize_mx_kernel(const void *__restrict__ src,
                                                               int src_dtype, int64_t nb,
                                                               uint8_t *__restrict__ q,
                                                               uint8_t *__restrict__ e8) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nb) return;
  float v[32];
  if (src_dtype == COLI_SRC_BF16) {
    const uint4 *s = reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(src) + 32 * b);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 w = s[j];
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * j + 2 * i] = __uint_as_float(d[i] << 16);
        v[8 * j + 2 * i + 1] = __uint_as_float(d[i] & 0xffff0000u);
      }
    }
  } else {
    const float4 *s = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(src) + 32 * b);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 w = s[j];
      v[4 * j] = w.x;
      v[4 * j + 1] = w.y;
      v[4 * j + 2] = w.z;
      v[4 * j + 3] = w.w;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t E = mx8_exponent(amax);
  uint32_t w[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = mx8_code(v[4 * j], E) | (mx8_code(v[4 * j + 1], E) << 8) |
           (mx8_code(v[4 * j + 2], E) << 16) | (mx8_code(v[4 * j + 3], E) << 24);
  uint4 *dst = reinterpret_cast<uint4 *>(q + 32 * b);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  e8[b] = (uint8_t)E;
}

// Stages filled by DMA (global_load_lds), as in dgemm_kernel: one stage
// holds 256 k of the item's 128 weight rows (E2M1, 16 KB) and of its 64
// token rows (E4M3, 16 KB), with both sides' E8M0 scale bytes.  Layouts are
// XOR-swizzled at 16-byte granularity so that every DMA instruction moves
// whole 128-byte lines and every 16-byte operand read of a half-wavefront
// hits distinct banks: weight row r keeps 16-byte chunk c at c ^ ((r>>1)&7),
// token t keeps chunk j at j ^ (t & 15).
struct MStage {
  uint4 w[BR * 8];   // [row][chunk]: 32 E2M1 codes = one 32-block of one row
  uint4 a[BM * 16];  // [token][chunk]: 16 E4M3 codes
  uint2 sw[BR];      // [row]: E8M0 of the stage's 8 blocks
  uint2 sa[BM];      // [token]: E8M0 of the stage's 8 blocks
};

// One item from DMA-filled stages.  Wave wv computes weight rows
// [16wv, 16wv+16) and [64+16wv, 64+16wv+16) (gate/up: gate and up of the
// same 16 channels) against each 16-token subtile that holds a token (NTS).
template <int MODE, int NTS>
COLI_DEV void mxd_item(const GemmArgs &g, const Item &it, const int *rowid, const int *outrow,
                       MStage &B0, MStage &B1, float (*xch)[4][16], uint8_t *qh_out,
                       uint8_t *eh_out, float *o_out) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = lane >> 4, lr = lane & 15;
  const int nst = g.K / kSK;
  const uint8_t *act = reinterpret_cast<const uint8_t *>(g.act);
  const uint8_t *act_e = reinterpret_cast<const uint8_t *>(g.act_d);
  // ---- DMA sources of this lane
  const uint8_t *sw_src, *sa_src, *w_src[4], *a_src[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * wv + 8 * j + (lane >> 3);  // instruction 4wv + j: rows 8(4wv+j)..+7
    const int chunk = (lane & 7) ^ ((row >> 1) & 7);
    const uint8_t *q;
    const uint16_t *unused;
    weight_row<MODE == kDots ? kDown : MODE>(g, it.n0, row, q, unused);
    w_src[j] = q + 16 * chunk;
    const int t = 16 * wv + 4 * j + (lane >> 4);   // tokens 4(4wv+j)..+3
    a_src[j] = act + (int64_t)rowid[t] * g.K + 16 * ((lane & 15) ^ (t & 15));
  }
  {
    const int row = 32 * wv + (lane >> 1);
    const uint8_t *unused;
    const uint16_t *sc;
    weight_row<MODE == kDots ? kDown : MODE>(g, it.n0, row, unused, sc);
    sw_src = reinterpret_cast<const uint8_t *>(sc) + 4 * (lane & 1);
    const int t = 32 * (wv & 1) + (lane >> 1);
    sa_src = act_e + (int64_t)rowid[t] * (g.K / 32) + 4 * (lane & 1);
  }
  const bool tok_live = wv < NTS;              // tokens 16wv..16wv+15 hold one
  const bool sa_live = wv < 2 && 2 * wv < NTS;  // waves 0, 1 move 32 tokens' scales each
  // DMA instruction p (0..9) of stage st
  auto issue_part = [&](MStage &B, int st, int p) {
    if (p < 4) {
      dma16(w_src[p] + st * (kSK / 2), &B.w[(4 * wv + p) * 64]);
    } else if (p < 8) {
      if (tok_live) dma16(a_src[p - 4] + st * kSK, &B.a[(4 * wv + p - 4) * 64]);
    } else if (p == 8) {
      dma4(sw_src + st * 8, reinterpret_cast<uint8_t *>(B.sw) + 256 * wv);
    } else if (sa_live) {
      dma4(sa_src + st * 8, reinterpret_cast<uint8_t *>(B.sa) + 256 * wv);
    }
  };

  coli_f32x4v acc[2][NTS];
#pragma unroll
  for (int rs = 0; rs < 2; ++rs)
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) acc[rs][ts] = coli_f32x4v{0.f, 0.f, 0.f, 0.f};

  const int rA = 16 * wv + lr;  // row of tile rs = 0 (tile 1: + 64, same swizzle)
  const uint32_t offA = rA * 128, fA = (rA >> 1) & 7;
  // one stage: two 128-k steps; stage `nxt`'s DMA goes out along the way
  auto compute = [&](const MStage &B, MStage &N, int nxt) {
    uint2 swv[2], sav[NTS];
#pragma unroll
    for (int rs = 0; rs < 2; ++rs) swv[rs] = B.sw[rA + 64 * rs];
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) sav[ts] = B.sa[16 * ts + lr];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (nxt >= 0) {
#pragma unroll
        for (int p = 5 * s; p < 5 * s + 5; ++p) issue_part(N, nxt, p);
      }
      coli_i32x8 av[2], bv[NTS];
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        const uint4 v = *reinterpret_cast<const uint4 *>(
            reinterpret_cast<const char *>(B.w) + offA + rs * 64 * 128 + 16 * ((4 * s + kq) ^ fA));
        av[rs] = coli_i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int ts = 0; ts < NTS; ++ts) {
        const int t = 16 * ts + lr;
        const char *row = reinterpret_cast<const char *>(B.a) + t * 256;
        const uint4 v0 = *reinterpret_cast<const uint4 *>(row + 16 * ((8 * s + kq) ^ (t & 15)));
        const uint4 v1 = *reinterpret_cast<const uint4 *>(row + 16 * ((8 * s + 4 + kq) ^ (t & 15)));
        bv[ts] = coli_i32x8{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                            (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      }
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        const uint32_t sa = ((s ? swv[rs].y : swv[rs].x) >> (8 * kq)) & 0xffu;
#pragma unroll
        for (int ts = 0; ts < NTS; ++ts) {
          const uint32_t sb = ((s ? sav[ts].y : sav[ts].x) >> (8 * kq)) & 0xffu;
          // formats: A E2M1 (4), B E4M3 (0); scale byte 0 of each register
          acc[rs][ts] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              av[rs], bv[ts], acc[rs][ts], 4, 0, 0, (int)sa, 0, (int)sb);
        }
      }
    }
  };

#pragma unroll
  for (int p = 0; p < 10; ++p) issue_part(B0, 0, p);
  wait_dma();
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    compute(B0, B1, st + 1 < nst ? st + 1 : -1);
    wait_dma();
    __syncthreads();
    if (st + 1 >= nst) break;
    compute(B1, B0, st + 2 < nst ? st + 2 : -1);
    wait_dma();
    __syncthreads();
  }

  // ---- epilogue
  if (MODE == kGateUp) {
    // h = silu(g) * u for channels n0 + 16wv + 4kq + i; MXFP8 of h per 32
    // channels: waves 2p and 2p+1 hold the two halves of block p
    float hv[NTS][4], am[NTS];
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[ts][i] = silu_mul(acc[0][ts][i], acc[1][ts][i]);
        a = fmaxf(a, fabsf(hv[ts][i]));
      }
      a = fmaxf(a, __shfl_xor(a, 16, 64));
      a = fmaxf(a, __shfl_xor(a, 32, 64));
      am[ts] = a;
      if (kq == 0) xch[wv][ts][lr] = a;
    }
    __syncthreads();
    const int I = g.rows;
    const int ch0 = it.n0 + 16 * wv;
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const uint32_t E = mx8_exponent(fmaxf(am[ts], xch[wv ^ 1][ts][lr]));
      const uint32_t packed = mx8_code(hv[ts][0], E) | (mx8_code(hv[ts][1], E) << 8) |
                              (mx8_code(hv[ts][2], E) << 16) | (mx8_code(hv[ts][3], E) << 24);
      const int m = 16 * ts + lr;
      if (m < it.ntok && ch0 < I) {
        const int64_t orow = outrow[m];
        *reinterpret_cast<uint32_t *>(qh_out + orow * I + ch0 + 4 * kq) = packed;
        if ((wv & 1) == 0 && kq == 0) eh_out[orow * (I / 32) + ch0 / 32] = (uint8_t)E;
      }
    }
  } else {
#pragma unroll
    for (int ts = 0; ts < NTS; ++ts) {
      const int m = 16 * ts + lr;
      if (m >= it.ntok) continue;
#pragma unroll
      for (int rs = 0; rs < 2; ++rs) {
        const int n = it.n0 + 16 * wv + 64 * rs + 4 * kq;
        if (n < g.rows)
          *reinterpret_cast<float4 *>(o_out + (int64_t)outrow[m] * g.rows + n) =
              make_float4(acc[rs][ts][0], acc[rs][ts][1], acc[rs][ts][2], acc[rs][ts][3]);
      }
    }
  }
}

template <int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
mxgemm_kernel(GemmArgs g, coli_moe_route_t r, const int4 *__restrict__ tiles,
              const int *__restrict__ ntiles_p, int fixed_ntok, int fixed_expert, int T, int k,
              int n_ntiles, int64_t expert_stride_q, int64_t expert_stride_s,
              uint8_t *__restrict__ qh_out, uint8_t *__restrict__ eh_out,
              float *__restrict__ o_out) {
  __shared__ MStage B0;
  __shared__ MStage B1;
  __shared__ int rowid[BM];
  __shared__ int outrow[BM];
  __shared__ float xch[4][4][16];
  const int ntiles = tiles ? ntiles_p[0] : (fixed_ntok + BM - 1) / BM;
  const int items = band_items(ntiles, n_ntiles);
  const int G = gridDim.x;
  const int vid = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  for (int item = vid; item < items; item += G) {
    int tile, ntile;
    item_coords(item, n_ntiles, tile, ntile);
    if (tile >= ntiles) continue;
    const Item it = setup_item<MODE>(tile, ntile, tiles, fixed_ntok, fixed_expert, r, T, k,
                                     rowid, outrow);
    GemmArgs ge = g;
    ge.wq = g.wq + (int64_t)it.expert * expert_stride_q;
    ge.ws = g.ws + (int64_t)it.expert * expert_stride_s;
    switch ((it.ntok + 15) >> 4) {
      case 1: mxd_item<MODE, 1>(ge, it, rowid, outrow, B0, B1, xch, qh_out, eh_out, o_out); break;
      case 2: mxd_item<MODE, 2>(ge, it, rowid, outrow, B0, B1, xch, qh_out, eh_out, o_out); break;
      case 3: mxd_item<MODE, 3>(ge, it, rowid, outrow, B0, B1, xch, qh_out, eh_out, o_out); break;
      default: mxd_item<MODE, 4>(ge, it, rowid, outrow, B0, B1, xch, qh_out, eh_out, o_out); break;
    }
  }
}

struct PrefillWs {
  int8_t *qx;
  uint16_t *dx;
  int8_t *qh;
  uint16_t *dh;
  float2 *rx;  // DMA GEMM: block records of x and of h
  float2 *rh;
  float *o;
  int4 *tiles;
  int *ntiles;
  size_t total;
};

// Layers the DMA GEMM serves: int4 codes, both reduction lengths whole
// 256-k stages.
bool dgemm_layer(const Layer &L) { return !L.w8 && !L.f4 && L.H % kSK == 0 && L.I % kSK == 0; }

int max_tiles(const Layer &L, int T) {
  const int64_t P = (int64_t)T * L.k;
  return (int)(P / BM + max_union(L, T) + (L.S ? (T + BM - 1) / BM : 0) + 1);
}

PrefillWs carve(const Layer &L, int T, void *base) {
  PrefillWs w{};
  const int64_t rows = pair_rows(L, T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return reinterpret_cast<char *>(base) + o;
  };
  w.qx = reinterpret_cast<int8_t *>(take((size_t)T * L.H));
  w.dx = reinterpret_cast<uint16_t *>(take((size_t)T * (L.H / 32) * 2));
  w.qh = reinterpret_cast<int8_t *>(take((size_t)rows * L.I));
  w.dh = reinterpret_cast<uint16_t *>(take((size_t)rows * (L.I / 32) * 2));
  w.rx = reinterpret_cast<float2 *>(take((size_t)T * (L.H / 32) * 8));
  w.rh = reinterpret_cast<float2 *>(take((size_t)rows * (L.I / 32) * 8));
  w.o = reinterpret_cast<float *>(take((size_t)rows * L.H * 4));
  w.tiles = reinterpret_cast<int4 *>(take((size_t)max_tiles(L, T) * sizeof(int4)));
  w.ntiles = reinterpret_cast<int *>(take(sizeof(int)));
  w.total = off;
  return w;
}

// grid size: one workgroup per item up to a cap, a multiple of 8 so the
// XCD-aware remap of workgroup ids is a bijection
int64_t band_items_host(int64_t ntiles, int64_t n_ntiles) {
  return (ntiles + kBand - 1) / kBand * kBand * n_ntiles;
}

int grid_for(int64_t items) {
  const int64_t g = items < 16384 ? items : 16384;
  return (int)((g + 7) / 8 * 8);
}

}  // namespace

size_t prefill_workspace(const Layer &L, int T) { return carve(L, T, nullptr).total; }

int launch_quantize_q8_0(const void *src, int src_dtype, int64_t n, int8_t *q, uint16_t *d,
                         hipStream_t s) {
  const int64_t nb = n / 32;
  const int64_t grid = (nb + kThreads - 1) / kThreads;
  launch_k(COLI_K_QUANTIZE, quantize_kernel<false>, dim3((unsigned)grid), dim3(kThreads), 0, s,
           src, src_dtype, nb, q, d, nullptr);
  return hip_status(hipGetLastError());
}

int launch_quantize_mxfp8(const void *src, int src_dtype, int64_t n, uint8_t *q, uint8_t *e8,
                          hipStream_t s) {
  const int64_t nb = n / 32;
  launch_k(COLI_K_QUANTIZE, quantize_mx_kernel, dim3((unsigned)((nb + kThreads - 1) / kThreads)),
           dim3(kThreads), 0, s, src, src_dtype, nb, q, e8);
  return hip_status(hipGetLastError());
}

int launch_mx_dots(const Layer &L, int expert, int matrix, const uint8_t *qa, const uint8_t *ea,
                   int T, float *out, hipStream_t s) {
  GemmArgs g{};
  g.rs = 1;
  g.wq = L.q4 + (int64_t)matrix * L.I * L.H / 2;
  g.ws = L.scales + (int64_t)matrix * L.I * L.H / 64;
  g.rows = matrix == 2 ? L.H : L.I;
  g.K = matrix == 2 ? L.I : L.H;
  g.act = reinterpret_cast<const int8_t *>(qa);
  g.act_d = reinterpret_cast<const uint16_t *>(ea);
  const int nn = (g.rows + BR - 1) / BR;
  const int ntile = (T + BM - 1) / BM;
  coli_moe_route_t none{};
  launch_k(COLI_K_BLOCK_DOTS, mxgemm_kernel<kDots>, dim3(grid_for(band_items_host(ntile, nn))),
           dim3(kThreads), 0, s, g, none, (const int4 *)nullptr, (const int *)nullptr, T, expert,
           T, 1, nn, L.expert_bytes, L.expert_scales, (uint8_t *)nullptr, (uint8_t *)nullptr, out);
  return hip_status(hipGetLastError());
}

namespace {

// The int4 forward on the DMA GEMM (dgemm_layer).
int launch_prefill_dgemm(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                         void *y, int y_dtype, const PrefillWs &w, hipStream_t s) {
  {
    const int64_t nb = (int64_t)T * L.H / 32;
    launch_k(COLI_K_QUANTIZE, quantize_kernel<true>, dim3((unsigned)((nb + kThreads - 1) / kThreads)),
             dim3(kThreads), 0, s, (const void *)x, (int)COLI_SRC_BF16, nb, w.qx,
             (uint16_t *)nullptr, w.rx);
  }
  launch_k(COLI_K_PLAN, plan_kernel, dim3(1), dim3(1024), 0, s, r, T, L.k, L.E, L.S, w.tiles,
           w.ntiles);
  if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  const int mt = max_tiles(L, T);
  {  // gate / up + SwiGLU + Q8_0(h)
    GemmArgs g{};
    g.wq = L.q4;
    g.ws = L.scales;
    g.rows = L.I;
    g.K = L.H;
    g.rs = 1;
    g.act = w.qx;
    g.up_offset_q = (int64_t)L.I * L.H / 2;
    g.up_offset_s = (int64_t)L.I * L.H / 64;
    const int nn = L.I / 64;
    launch_k(COLI_K_GEMM_GATEUP, dgemm_kernel<kGateUp>,
             dim3(grid_for(band_items_host(mt, nn))), dim3(kThreads), 0, s, g, r, w.tiles,
             w.ntiles, 0, 0, T, L.k, nn, L.expert_bytes, L.expert_scales,
             (const float2 *)w.rx, w.qh, w.rh, (float *)nullptr, (int32_t *)nullptr);
    if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  }
  {  // down
    GemmArgs g{};
    g.rs = 1;
    g.wq = L.q4 + (int64_t)L.I * L.H;
    g.ws = L.scales + (int64_t)2 * L.I * L.H / 64;
    g.rows = L.H;
    g.K = L.I;
    g.act = w.qh;
    const int nn = (L.H + BR - 1) / BR;
    launch_k(COLI_K_GEMM_DOWN, dgemm_kernel<kDown>, dim3(grid_for(band_items_host(mt, nn))),
             dim3(kThreads), 0, s, g, r, w.tiles, w.ntiles, 0, 0, T, L.k, nn, L.expert_bytes,
             L.expert_scales, (const float2 *)w.rh, (int8_t *)nullptr, (float2 *)nullptr, w.o,
             (int32_t *)nullptr);
    if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  }
  launch_combine(w.o, r, T, L.H, L.k, L.S, y, y_dtype, s);
  return hip_status(hipGetLastError());
}

}  // namespace

namespace {

// The MX forward (MXFP4 weights, COLI_ACT_MXFP8): MXFP8 of x, plan, the two
// MX GEMMs (h in MXFP8 between them), combine.
int launch_prefill_mx(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                      void *y, int y_dtype, const PrefillWs &w, hipStream_t s) {
  uint8_t *qx = reinterpret_cast<uint8_t *>(w.qx), *ex = reinterpret_cast<uint8_t *>(w.dx);
  uint8_t *qh = reinterpret_cast<uint8_t *>(w.qh), *eh = reinterpret_cast<uint8_t *>(w.dh);
  int rc = launch_quantize_mxfp8(x, COLI_SRC_BF16, (int64_t)T * L.H, qx, ex, s);
  if (rc) return rc;
  launch_k(COLI_K_PLAN, plan_kernel, dim3(1), dim3(1024), 0, s, r, T, L.k, L.E, L.S, w.tiles,
           w.ntiles);
  if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  const int mt = max_tiles(L, T);
  {  // gate / up + SwiGLU + MXFP8(h)
    GemmArgs g{};
    g.rs = 1;
    g.wq = L.q4;
    g.ws = L.scales;
    g.rows = L.I;
    g.K = L.H;
    g.act = reinterpret_cast<const int8_t *>(qx);
    g.act_d = reinterpret_cast<const uint16_t *>(ex);
    g.up_offset_q = (int64_t)L.I * L.H / 2;
    g.up_offset_s = (int64_t)L.I * L.H / 64;
    const int nn = (L.I + 63) / 64;
    launch_k(COLI_K_GEMM_GATEUP, mxgemm_kernel<kGateUp>, dim3(grid_for(band_items_host(mt, nn))),
             dim3(kThreads), 0, s, g, r, (const int4 *)w.tiles, (const int *)w.ntiles, 0, 0, T,
             L.k, nn, L.expert_bytes, L.expert_scales, qh, eh, (float *)nullptr);
    if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  }
  {  // down
    GemmArgs g{};
    g.rs = 1;
    g.wq = L.q4 + (int64_t)L.I * L.H;
    g.ws = L.scales + (int64_t)2 * L.I * L.H / 64;
    g.rows = L.H;
    g.K = L.I;
    g.act = reinterpret_cast<const int8_t *>(qh);
    g.act_d = reinterpret_cast<const uint16_t *>(eh);
    const int nn = (L.H + BR - 1) / BR;
    launch_k(COLI_K_GEMM_DOWN, mxgemm_kernel<kDown>, dim3(grid_for(band_items_host(mt, nn))),
             dim3(kThreads), 0, s, g, r, (const int4 *)w.tiles, (const int *)w.ntiles, 0, 0, T,
             L.k, nn, L.expert_bytes, L.expert_scales, (uint8_t *)nullptr, (uint8_t *)nullptr,
             w.o);
    if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  }
  launch_combine(w.o, r, T, L.H, L.k, L.S, y, y_dtype, s);
  return hip_status(hipGetLastError());
}

}  // namespace

int launch_prefill(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T, void *y,
                   int y_dtype, void *ws, hipStream_t s) {
  const PrefillWs w = carve(L, T, ws);
  if (L.f4 && (L.flags & COLI_ACT_MXFP8)) return launch_prefill_mx(L, r, x, T, y, y_dtype, w, s);
  if (dgemm_layer(L)) return launch_prefill_dgemm(L, r, x, T, y, y_dtype, w, s);
  int rc = launch_quantize_q8_0(x, COLI_SRC_BF16, (int64_t)T * L.H, w.qx, w.dx, s);
  if (rc) return rc;
  launch_k(COLI_K_PLAN, plan_kernel, dim3(1), dim3(1024), 0, s, r, T, L.k, L.E, L.S, w.tiles,
           w.ntiles);
  if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  const int mt = max_tiles(L, T);
  {  // gate / up + SwiGLU + Q8_0(h)
    GemmArgs g{};
    g.wq = L.q4;
    g.ws = L.scales;
    g.rows = L.I;
    g.K = L.H;
    g.rs = L.w8 ? 0 : 1;
    const int wf = L.f4 ? kFmtF4 : (L.w8 ? kFmtI8 : kFmtI4);
    g.act = w.qx;
    g.act_d = w.dx;
    g.up_offset_q = ((int64_t)L.I * L.H) >> g.rs;
    g.up_offset_s = (int64_t)L.I * L.H / 64;
    const int nn = (L.I + 63) / 64;
    launch_k(COLI_K_GEMM_GATEUP,
             L.H % 256 ? (wf == kFmtF4   ? gemm_kernel<kGateUp, kFmtF4>
                          : wf == kFmtI8 ? gemm_kernel<kGateUp, kFmtI8>
                                         : gemm_kernel<kGateUp, kFmtI4>)
             : wf == kFmtF4 ? gemm4_kernel<kGateUp, kFmtF4>
             : wf == kFmtI8 ? gemm4_kernel<kGateUp, kFmtI8>
                            : gemm4_kernel<kGateUp, kFmtI4>,
             dim3(grid_for(band_items_host(mt, nn))), dim3(kThreads), 0, s, g, r, w.tiles, w.ntiles, 0,
             0, T, L.k, nn, L.expert_bytes, L.expert_scales, w.qh, w.dh, nullptr, nullptr);
    if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  }
  {  // down
    GemmArgs g{};
    g.rs = L.w8 ? 0 : 1;
    const int wf = L.f4 ? kFmtF4 : (L.w8 ? kFmtI8 : kFmtI4);
    g.wq = L.q4 + (((int64_t)2 * L.I * L.H) >> g.rs);
    g.ws = L.scales + (int64_t)2 * L.I * L.H / 64;
    g.rows = L.H;
    g.K = L.I;
    g.act = w.qh;
    g.act_d = w.dh;
    const int nn = (L.H + BR - 1) / BR;
    launch_k(COLI_K_GEMM_DOWN,
             L.I % 256 ? (wf == kFmtF4   ? gemm_kernel<kDown, kFmtF4>
                          : wf == kFmtI8 ? gemm_kernel<kDown, kFmtI8>
                                         : gemm_kernel<kDown, kFmtI4>)
             : wf == kFmtF4 ? gemm4_kernel<kDown, kFmtF4>
             : wf == kFmtI8 ? gemm4_kernel<kDown, kFmtI8>
                            : gemm4_kernel<kDown, kFmtI4>,
             dim3(grid_for(band_items_host(mt, nn))), dim3(kThreads), 0, s, g, r, w.tiles, w.ntiles, 0,
             0, T, L.k, nn, L.expert_bytes, L.expert_scales, nullptr, nullptr, w.o, nullptr);
    if (hipGetLastError() != hipSuccess) return COLI_E_HIP;
  }
  launch_combine(w.o, r, T, L.H, L.k, L.S, y, y_dtype, s);
  return hip_status(hipGetLastError());
}

int launch_block_dots(const Layer &L, int expert, int matrix, const int8_t *q_act, int T,
                      int32_t *dots, hipStream_t s) {
  GemmArgs g{};
  g.rs = L.w8 ? 0 : 1;
  const int wf = L.f4 ? kFmtF4 : (L.w8 ? kFmtI8 : kFmtI4);
  const int64_t moff = ((int64_t)matrix * L.I * L.H) >> g.rs;
  g.wq = L.q4 + moff;
  g.ws = L.scales + (int64_t)matrix * L.I * L.H / 64;
  g.rows = matrix == 2 ? L.H : L.I;
  g.K = matrix == 2 ? L.I : L.H;
  g.act = q_act;
  g.act_d = nullptr;
  const int nn = (g.rows + BR - 1) / BR;
  const int ntile = (T + BM - 1) / BM;
  coli_moe_route_t none{};
  if (dgemm_layer(L)) {
    launch_k(COLI_K_BLOCK_DOTS, dgemm_kernel<kDots>, dim3(grid_for(band_items_host(ntile, nn))),
             dim3(kThreads), 0, s, g, none, (const int4 *)nullptr, (const int *)nullptr, T, expert,
             T, 1, nn, L.expert_bytes, L.expert_scales, (const float2 *)nullptr, (int8_t *)nullptr,
             (float2 *)nullptr, (float *)nullptr, dots);
    return hip_status(hipGetLastError());
  }
  launch_k(COLI_K_BLOCK_DOTS,
           g.K % 256 ? (wf == kFmtF4   ? gemm_kernel<kDots, kFmtF4>
                        : wf == kFmtI8 ? gemm_kernel<kDots, kFmtI8>
                                       : gemm_kernel<kDots, kFmtI4>)
           : wf == kFmtF4 ? gemm4_kernel<kDots, kFmtF4>
           : wf == kFmtI8 ? gemm4_kernel<kDots, kFmtI8>
                          : gemm4_kernel<kDots, kFmtI4>,
           dim3(grid_for(band_items_host(ntile, nn))),
           dim3(kThreads), 0, s, g, none, nullptr, nullptr, T, expert, T, 1, nn, L.expert_bytes,
           L.expert_scales, nullptr, nullptr, nullptr, dots);
  return hip_status(hipGetLastError());
}

}  // namespace coli
