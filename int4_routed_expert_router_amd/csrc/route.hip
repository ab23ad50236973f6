// route.hip -- router top-k, routing weights and the batch-union grouping.
//
// The router's choice decides which experts a token uses (aixq.cc article on
// colibri, section "为什么值得关注"), and a batch reads every distinct expert
// once (tantan.ink post on colibri, section "几个关键工程动作").  Selection
// and grouping are exact: only fp32 comparisons and integer counts, so the
// indices and pair lists are bit-identical to any correct implementation.
//
// Kernels
//  topk  : one wavefront per token; each lane holds E/64 scores; k rounds of
//          a wave-wide (score desc, index asc) argmax.  Weights in fp32.
//  group : one 1024-thread workgroup; LDS histogram, LDS scan, then a stable
//          scatter whose in-expert rank comes from per-64-token bit masks:
//          rank(t, e) = #tokens before t (in the batch) that chose e.
//  fused : topk + group in one workgroup for T <= 16 (decode / verify).
#include <float.h>
#include <limits.h>

#include "device_common.h"
#include "internal.h"

namespace coli {
namespace {

constexpr int kGroupThreads = 1024;
constexpr int kMaskWords = 4096;  // 64-token masks held in LDS at once

// ---------------------------------------------------------------- top-k

// Selection key of expert e with score s: the order-preserving unsigned image
// of s in the high word, ~e in the low word, so one unsigned max picks the
// largest score and, among equal scores, the lower index.  -0 is folded
// onto +0 (they compare equal as floats); NaN scores rank below -inf.
COLI_DEV uint64_t select_key(float s, int e) {
  uint32_t u = __float_as_uint(s + 0.0f);
  uint32_t hi = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  if (s != s) hi = 0x007ffffeu;  // just below -inf, whose image is 0x007fffff
  return ((uint64_t)hi << 32) | (uint32_t)(~(uint32_t)e);
}

// Wave-wide reductions with DPP moves (no LDS round trips): four steps
// inside each row of 16 lanes (swap neighbours, swap pairs, mirror halves of
// 8, mirror the row), then row_bcast:15 and row_bcast:31 carry the row
// results up, so that lane 63 holds the reduction of all 64 lanes; it is read
// into a scalar register.  Rows a broadcast does not write keep `idle`, the
// operation's neutral value.  The operation order is fixed, so a token's
// result never depends on which wavefront or batch computes it.
template <int CTRL, int ROWS = 0xf>
COLI_DEV uint32_t dpp_u32(uint32_t idle, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)idle, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS = 0xf>
COLI_DEV float dpp_f32(float idle, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(idle), __float_as_int(v), CTRL,
                                                    ROWS, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kHalfMirror = 0x141, kRowMirror = 0x140;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;

COLI_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kQuadXor1>(0u, v));
  v = max(v, dpp_u32<kQuadXor2>(0u, v));
  v = max(v, dpp_u32<kHalfMirror>(0u, v));
  v = max(v, dpp_u32<kRowMirror>(0u, v));
  v = max(v, dpp_u32<kBcast15, 0xa>(0u, v));
  v = max(v, dpp_u32<kBcast31, 0xc>(0u, v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
COLI_DEV float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kQuadXor1>(-FLT_MAX, v));
  v = fmaxf(v, dpp_f32<kQuadXor2>(-FLT_MAX, v));
  v = fmaxf(v, dpp_f32<kHalfMirror>(-FLT_MAX, v));
  v = fmaxf(v, dpp_f32<kRowMirror>(-FLT_MAX, v));
  v = fmaxf(v, dpp_f32<kBcast15, 0xa>(-FLT_MAX, v));
  v = fmaxf(v, dpp_f32<kBcast31, 0xc>(-FLT_MAX, v));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
COLI_DEV float wave_sum_f32(float v) {
  v += dpp_f32<kQuadXor1>(0.0f, v);
  v += dpp_f32<kQuadXor2>(0.0f, v);
  v += dpp_f32<kHalfMirror>(0.0f, v);
  v += dpp_f32<kRowMirror>(0.0f, v);
  v += dpp_f32<kBcast15, 0xa>(0.0f, v);
  v += dpp_f32<kBcast31, 0xc>(0.0f, v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sorts a lane's NPL (key, logit) entries by key, descending (odd-even
// transposition: NPL rounds of neighbour compare-exchanges).
template <int NPL>
COLI_DEV void sort_lane(uint64_t (&key)[NPL], float (&lg)[NPL]) {
#pragma unroll
  for (int rnd = 0; rnd < NPL; ++rnd)
#pragma unroll
    for (int i = rnd & 1; i + 1 < NPL; i += 2) {
      const bool sw = key[i + 1] > key[i];
      const uint64_t ka = key[i], kb = key[i + 1];
      const float la = lg[i], lb = lg[i + 1];
      key[i] = sw ? kb : ka;
      key[i + 1] = sw ? ka : kb;
      lg[i] = sw ? lb : la;
      lg[i + 1] = sw ? la : lb;
    }
}

// One wavefront selects the k experts of one token.  Lane j < k ends with
// the j-th chosen expert (*my_e) and its routing weight (returned); the
// weights use the raw logits (see COLI_ROUTE_*).
template <int NPL>
COLI_DEV float topk_wave(const float *__restrict__ lg_row, const float *__restrict__ bias, int E,
                         int k, uint32_t flags, float routed_scale, int *my_e) {
  const int lane = threadIdx.x & 63;
  float lg[NPL], bs[NPL];
  uint64_t key[NPL];
  // every load issued before any is used: lanes past E read entry E-1, and
  // with no bias the logits are read a second time in its place
  const float *bsrc = bias ? bias : lg_row;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = min(lane + 64 * i, E - 1);
    lg[i] = lg_row[e];
    bs[i] = bsrc[e];
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) lg[i] = 0.0f;
    key[i] = e < E ? select_key(bias ? lg[i] + bs[i] : lg[i], e) : 0ull;
  }
  float m = -FLT_MAX, z = 0.0f;
  if ((flags & COLI_ROUTE_SIGMOID) == 0) {
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i < E) m = fmaxf(m, lg[i]);
    m = wave_max_f32(m);
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (lane + 64 * i < E) z += expf(lg[i] - m);
    z = wave_sum_f32(z);
  }
  // Each lane keeps its entries sorted, so its best is key[0].  A round takes
  // the largest score image over the wave (32-bit DPP max); among lanes whose
  // best has that score (ties are rare) the lower expert index, i.e. the
  // larger low word, wins.  The owner drops its head.
  sort_lane<NPL>(key, lg);
  float my_l = 0.0f;
  int me = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t hi = (uint32_t)(key[0] >> 32), lo = (uint32_t)key[0];
    const uint32_t mx = wave_max_u32(hi);
    uint64_t ball = __ballot(hi == mx);
    if (__popcll(ball) > 1) {  // all lanes take part in the reduction
      const uint32_t mlo = wave_max_u32(hi == mx ? lo : 0u);
      ball = __ballot(hi == mx && lo == mlo);
    }
    const int owner = __ffsll((long long)ball) - 1;
    const int e = (int)~(uint32_t)__builtin_amdgcn_readlane((int)lo, owner);
    const float wl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lg[0]), owner));
    if (lane == owner) {
#pragma unroll
      for (int i = 0; i + 1 < NPL; ++i) {
        key[i] = key[i + 1];
        lg[i] = lg[i + 1];
      }
      key[NPL - 1] = 0ull;
    }
    if (lane == j) {
      me = e;
      my_l = wl;
    }
  }
  float w = (flags & COLI_ROUTE_SIGMOID) ? 1.0f / (1.0f + expf(-my_l)) : expf(my_l - m) / z;
  if (flags & COLI_ROUTE_RENORM) w = w / wave_sum_f32(lane < k ? w : 0.0f);
  *my_e = me;
  return w * routed_scale;
}

// Returns, in lane j < k, the j-th chosen expert (also written to idx_out).
template <int NPL>
__device__ int topk_token(const float *__restrict__ lg_row, const float *__restrict__ bias,
                          int E, int k, uint32_t flags, float routed_scale,
                          int32_t *__restrict__ idx_out, float *__restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  int me;
  const float w = topk_wave<NPL>(lg_row, bias, E, k, flags, routed_scale, &me);
  if (lane < k) {
    idx_out[lane] = me;
    w_out[lane] = w;
  }
  return me;
}

// Single token: one wavefront does the selection and the grouping, which
// for one token has a closed form -- offsets[e] counts the winners below e,
// and pair j's position is offsets[its expert].  The winners are marked in
// an LDS table of E flags; one ballot per 64 experts gives their bit masks,
// and the counts below follow from popcounts.
template <int NPL>
__global__ void __launch_bounds__(64) single_kernel(const float *__restrict__ logits,
                                                    const float *__restrict__ bias, int E, int k,
                                                    uint32_t flags, float routed_scale,
                                                    coli_moe_route_t r) {
  __shared__ uint32_t won[64 * NPL];
  const int lane = threadIdx.x;
#pragma unroll
  for (int i = 0; i < NPL; ++i) won[lane + 64 * i] = 0u;
  int me;
  const float w = topk_wave<NPL>(logits, bias, E, k, flags, routed_scale, &me);
  if (lane < k) won[me] = 1u;
  __syncthreads();
  int hit[NPL], cnt_lt[NPL];
  int below = 0;           // winners in the 64-expert words before word i
  int rank = 0;            // winners below this lane's own expert (lanes < k)
  const int my_word = me >> 6;
  const uint64_t my_bits = (1ull << (me & 63)) - 1ull;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    hit[i] = (int)won[lane + 64 * i];
    const uint64_t mask = __ballot(hit[i] != 0);
    cnt_lt[i] = below + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
    if (my_word == i) rank = below + __popcll(mask & my_bits);
    below += __popcll(mask);
  }
  if (lane < k) {
    r.topk_idx[lane] = me;
    r.topk_w[lane] = w;
    r.pairs[rank] = lane;
    r.pair_pos[lane] = rank;
    r.union_ids[rank] = me;
  }
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) {
      r.counts[e] = hit[i];
      r.offsets[e] = cnt_lt[i];
    }
  }
  if (lane == 0) {
    r.offsets[E] = k;
    r.n_union[0] = k;
  }
}

template <int NPL>
__global__ void __launch_bounds__(256) topk_kernel(const float *__restrict__ logits,
                                                   const float *__restrict__ bias, int T, int E,
                                                   int k, uint32_t flags, float routed_scale,
                                                   int32_t *__restrict__ idx,
                                                   float *__restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token<NPL>(logits + (int64_t)t * E, bias, E, k, flags, routed_scale,
                  idx + (int64_t)t * k, w + (int64_t)t * k);
}

// ---------------------------------------------------------------- group

struct GroupShared {
  int cnt[1024];
  int off[1025];
  int run[1024];
  int wsum[16];
  unsigned long long mask[kMaskWords];
  int cbase[kMaskWords];
};

// Exclusive scan of v over the block (1024 threads); returns the prefix and
// writes the total to *total.
__device__ int block_exclusive_scan(int v, int *wsum, int *total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wsum[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < kGroupThreads / 64; ++i) {
      const int t = wsum[i];
      wsum[i] = acc;
      acc += t;
    }
    *total = acc;
  }
  __syncthreads();
  const int r = wsum[wid] + inc - v;
  __syncthreads();
  return r;
}

__device__ void group_pairs(const int32_t *__restrict__ idx, int T, int k, int E,
                            const coli_moe_route_t &r, GroupShared &sh) {
  const int tid = threadIdx.x;
  const int64_t P = (int64_t)T * k;
  __shared__ int total;
  for (int e = tid; e < E; e += kGroupThreads) sh.cnt[e] = 0;
  __syncthreads();
  for (int64_t p = tid; p < P; p += kGroupThreads) atomicAdd(&sh.cnt[idx[p]], 1);
  __syncthreads();
  // offsets and the batch union (E <= 1024: one expert per thread)
  const int c = tid < E ? sh.cnt[tid] : 0;
  const int off = block_exclusive_scan(c, sh.wsum, &total);
  if (tid < E) {
    sh.off[tid] = off;
    sh.run[tid] = 0;
    r.counts[tid] = c;
    r.offsets[tid] = off;
  }
  if (tid == 0) r.offsets[E] = (int)P;
  const int upos = block_exclusive_scan(c > 0 ? 1 : 0, sh.wsum, &total);
  if (tid < E && c > 0) r.union_ids[upos] = tid;
  if (tid == 0) r.n_union[0] = total;
  __syncthreads();
  // stable scatter, in super-chunks of 64-token chunks
  const int max_chunks = kMaskWords / E;
  for (int t0 = 0; t0 < T; t0 += 64 * max_chunks) {
    const int t1 = min(T, t0 + 64 * max_chunks);
    const int nc = (t1 - t0 + 63) >> 6;
    for (int i = tid; i < nc * E; i += kGroupThreads) sh.mask[i] = 0ull;
    __syncthreads();
    for (int64_t p = (int64_t)t0 * k + tid; p < (int64_t)t1 * k; p += kGroupThreads) {
      const int t = (int)(p / k) - t0;
      atomicOr(&sh.mask[(t >> 6) * E + idx[p]], 1ull << (t & 63));
    }
    __syncthreads();
    for (int e = tid; e < E; e += kGroupThreads) {
      int run = sh.run[e];
      for (int ch = 0; ch < nc; ++ch) {
        sh.cbase[ch * E + e] = run;
        run += __popcll(sh.mask[ch * E + e]);
      }
      sh.run[e] = run;
    }
    __syncthreads();
    for (int64_t p = (int64_t)t0 * k + tid; p < (int64_t)t1 * k; p += kGroupThreads) {
      const int t = (int)(p / k) - t0;
      const int e = idx[p];
      const int w = (t >> 6) * E + e;
      const unsigned long long below = sh.mask[w] & ((1ull << (t & 63)) - 1ull);
      const int pos = sh.off[e] + sh.cbase[w] + __popcll(below);
      r.pairs[pos] = (int)p;
      r.pair_pos[p] = pos;
    }
    __syncthreads();
  }
}

__global__ void __launch_bounds__(kGroupThreads) group_kernel(int T, int k, int E,
                                                              coli_moe_route_t r) {
  __shared__ GroupShared sh;
  group_pairs(r.topk_idx, T, k, E, r, sh);
}

// Small batches (T <= 16, decode / verify): top-k and grouping in one
// workgroup with every intermediate in LDS, so the only global read is the
// logits.  A token picks an expert at most once, so the stable in-expert
// rank of token t is the number of earlier tokens in the expert's 64-bit
// token mask.
constexpr int kSmallT = 16;

template <int NPL>
__global__ void __launch_bounds__(kGroupThreads) fused_kernel(const float *__restrict__ logits,
                                                              const float *__restrict__ bias,
                                                              int T, int E, int k, uint32_t flags,
                                                              float routed_scale,
                                                              coli_moe_route_t r) {
  __shared__ int s_idx[kSmallT * 32];
  __shared__ int s_cnt[1024];
  __shared__ int s_off[1024];
  __shared__ unsigned long long s_mask[1024];
  __shared__ int wsum[16];
  __shared__ int total;
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int e = tid; e < E; e += nthr) {
    s_cnt[e] = 0;
    s_mask[e] = 0ull;
  }
  const int t = tid >> 6;
  if (t < T) {
    const int mine = topk_token<NPL>(logits + (int64_t)t * E, bias, E, k, flags, routed_scale,
                                     r.topk_idx + (int64_t)t * k, r.topk_w + (int64_t)t * k);
    const int lane = tid & 63;
    if (lane < k) s_idx[t * k + lane] = mine;
  }
  __syncthreads();
  const int P = T * k;
  for (int p = tid; p < P; p += nthr) {
    const int e = s_idx[p];
    atomicAdd(&s_cnt[e], 1);
    atomicOr(&s_mask[e], 1ull << (p / k));
  }
  __syncthreads();
  // offsets and the batch union: one expert per thread (E <= blockDim)
  const int lane = tid & 63, wid = tid >> 6, nw = nthr >> 6;
  const int c = tid < E ? s_cnt[tid] : 0;
  int inc_c = c, inc_u = c > 0 ? 1 : 0;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int nc = __shfl_up(inc_c, o, 64), nu = __shfl_up(inc_u, o, 64);
    if (lane >= o) {
      inc_c += nc;
      inc_u += nu;
    }
  }
  if (lane == 63) wsum[wid] = inc_c | (inc_u << 16);  // both fit in 16 bits (P, E <= 1024)
  __syncthreads();
  if (tid == 0) {
    int ac = 0, au = 0;
    for (int i = 0; i < nw; ++i) {
      const int v = wsum[i];
      wsum[i] = ac | (au << 16);
      ac += v & 0xffff;
      au += v >> 16;
    }
    total = au;
  }
  __syncthreads();
  const int off = (wsum[wid] & 0xffff) + inc_c - c;
  const int upos = (wsum[wid] >> 16) + inc_u - (c > 0 ? 1 : 0);
  if (tid < E) {
    s_off[tid] = off;
    r.counts[tid] = c;
    r.offsets[tid] = off;
    if (c > 0) r.union_ids[upos] = tid;
  }
  if (tid == 0) {
    r.offsets[E] = P;
    r.n_union[0] = total;
  }
  __syncthreads();
  for (int p = tid; p < P; p += nthr) {
    const int e = s_idx[p], tok = p / k;
    const int pos = s_off[e] + __popcll(s_mask[e] & ((1ull << tok) - 1ull));
    r.pairs[pos] = p;
    r.pair_pos[p] = pos;
  }
}

template <int NPL>
int launch_npl(const Layer &L, const float *logits, const float *bias, int T,
               const coli_moe_route_t &r, hipStream_t s) {
  if (T == 1) {
    launch_k(COLI_K_ROUTE_FUSED, single_kernel<NPL>, dim3(1), dim3(64), 0, s, logits, bias, L.E,
             L.k, L.flags, L.routed_scale, r);
  } else if (T <= kSmallT) {
    // enough wavefronts for one token each and one thread per expert
    const int need = max(64 * T, L.E);
    const int threads = need <= 256 ? 256 : (need <= 512 ? 512 : 1024);
    launch_k(COLI_K_ROUTE_FUSED, fused_kernel<NPL>, dim3(1), dim3(threads), 0, s, logits, bias, T,
             L.E, L.k, L.flags, L.routed_scale, r);
  } else {
    launch_k(COLI_K_TOPK, topk_kernel<NPL>, dim3((T + 3) / 4), dim3(256), 0, s, logits, bias, T,
             L.E, L.k, L.flags, L.routed_scale, r.topk_idx, r.topk_w);
    launch_k(COLI_K_GROUP, group_kernel, dim3(1), dim3(kGroupThreads), 0, s, T, L.k, L.E, r);
  }
  return hip_status(hipGetLastError());
}

}  // namespace

int launch_route(const Layer &L, const float *logits, const float *bias, int T,
                 const coli_moe_route_t &r, hipStream_t s) {
  const int npl = (L.E + 63) / 64;
  if (npl <= 1) return launch_npl<1>(L, logits, bias, T, r, s);
  if (npl <= 2) return launch_npl<2>(L, logits, bias, T, r, s);
  if (npl <= 4) return launch_npl<4>(L, logits, bias, T, r, s);
  if (npl <= 8) return launch_npl<8>(L, logits, bias, T, r, s);
  return launch_npl<16>(L, logits, bias, T, r, s);
}

}  // namespace coli
