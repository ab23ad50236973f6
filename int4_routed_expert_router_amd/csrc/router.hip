// router.hip -- router logits from the layer input: logits = x . W_r^T.
//
// The router decides which experts a token loads and runs ahead of the
// expert loads (aixq.cc article on colibri, sections "为什么值得关注" and
// "我的真实看法").  The pages give no formula; it is read as a dense linear
// layer without bias, bf16 weights [E][H] and bf16 activations [T][H], with
// fp32 accumulation and fp32 logits.
//
// Every batch size gets the same arithmetic per (token, expert), so a
// token's logits -- and hence its expert choice -- do not depend on the rest
// of the batch:
//  - K is cut into tiles of 512 values; lane L of a wavefront owns the
//    8-value chunk L of every tile (chunk index 64 * tile + L), and adds it
//    to its running sum as four bf16 dot2 steps, tile after tile;
//  - the 64 lane sums are then added by one fixed butterfly (xor 32 .. 1).
// Only the grouping of the work changes with T: in router_kernel a
// wavefront computes EPW experts x TT tokens (TT tokens per workgroup, staged
// per tile in LDS, double-buffered), with the next tile's weights already in
// flight; router_one_kernel (up to 16 tokens) loads everything at once.
#include "device_common.h"
#include "internal.h"

namespace coli {
namespace {

constexpr int kThreads = 256;  // 4 wavefronts

COLI_DEV float chunk8_dot(const uint4 w, const uint4 x, float acc) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  return dot2_bf16(w.w, x.w, acc);
}

template <int EPW, int TT>
__global__ void __launch_bounds__(kThreads) router_kernel(const uint16_t *__restrict__ w,
                                                          const uint16_t *__restrict__ x, int T,
                                                          int E, int H,
                                                          float *__restrict__ logits) {
  __shared__ uint4 xs[2][TT][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = (blockIdx.x * 4 + wv) * EPW;  // first expert of this wavefront
  const int t0 = blockIdx.y * TT;              // first token of this workgroup
  const int nt = min(TT, T - t0);
  const int nch = H >> 3;                      // 8-value chunks per row
  const int ntiles = (nch + 63) >> 6;

  // x chunks of one tile for the workgroup's tokens (zeros past the end)
  auto stage = [&](int tile, int buf) {
#pragma unroll
    for (int p = 0; p < (TT * 64 + kThreads - 1) / kThreads; ++p) {
      const int i = threadIdx.x + kThreads * p;
      if (i < TT * 64) {
        const int tt = i >> 6, c = 64 * tile + (i & 63);
        uint4 v = make_uint4(0, 0, 0, 0);
        if (tt < nt && c < nch)
          v = *reinterpret_cast<const uint4 *>(x + (int64_t)(t0 + tt) * H + 8 * c);
        xs[buf][tt][i & 63] = v;
      }
    }
  };
  // this lane's weight chunk of one tile for each of the wavefront's experts
  auto load_w = [&](int tile, uint4 (&wq)[EPW]) {
    const int c = 64 * tile + lane;
#pragma unroll
    for (int ee = 0; ee < EPW; ++ee)
      wq[ee] = (c < nch && e0 + ee < E)
                   ? *reinterpret_cast<const uint4 *>(w + (int64_t)(e0 + ee) * H + 8 * c)
                   : make_uint4(0, 0, 0, 0);
  };

  float acc[EPW][TT];
#pragma unroll
  for (int ee = 0; ee < EPW; ++ee)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) acc[ee][tt] = 0.0f;

  uint4 wcur[EPW], wnext[EPW];
  load_w(0, wcur);
  stage(0, 0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    if (tile + 1 < ntiles) {
      load_w(tile + 1, wnext);
      stage(tile + 1, (tile + 1) & 1);
    }
    if (64 * tile + lane < nch) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const uint4 xq = xs[tile & 1][tt][lane];
#pragma unroll
        for (int ee = 0; ee < EPW; ++ee) acc[ee][tt] = chunk8_dot(wcur[ee], xq, acc[ee][tt]);
      }
    }
    __syncthreads();  // the next iteration stages into the buffer read here
#pragma unroll
    for (int ee = 0; ee < EPW; ++ee) wcur[ee] = wnext[ee];
  }

#pragma unroll
  for (int ee = 0; ee < EPW; ++ee)
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      float v = acc[ee][tt];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      if (lane == 0 && tt < nt && e0 + ee < E) logits[(int64_t)(t0 + tt) * E + e0 + ee] = v;
    }
}

// Small batches: no staging.  Each wavefront (one expert, one token: token
// blockIdx.y) requests all of its lane's weight and activation chunks at
// once -- NT tiles, one 16-byte chunk of each per lane -- then adds them in
// the same order as router_kernel.  The router weights are read once per
// token, mostly from L2.
template <int NT>
__global__ void __launch_bounds__(kThreads) router_one_kernel(const uint16_t *__restrict__ w,
                                                              const uint16_t *__restrict__ x,
                                                              int E, int H,
                                                              float *__restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int e = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (e >= E) return;
  const int nch = H >> 3;
  x += (int64_t)blockIdx.y * H;
  logits += (int64_t)blockIdx.y * E;
  uint4 wq[NT], xq[NT];
#pragma unroll
  for (int tile = 0; tile < NT; ++tile) {
    const int c = 64 * tile + lane;
    const bool ok = c < nch;
    wq[tile] = ok ? *reinterpret_cast<const uint4 *>(w + (int64_t)e * H + 8 * c)
                  : make_uint4(0, 0, 0, 0);
    xq[tile] = ok ? *reinterpret_cast<const uint4 *>(x + 8 * c) : make_uint4(0, 0, 0, 0);
  }
  float v = 0.0f;
#pragma unroll
  for (int tile = 0; tile < NT; ++tile)
    if (64 * tile + lane < nch) v = chunk8_dot(wq[tile], xq[tile], v);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) logits[e] = v;
}

template <int EPW, int TT>
void launch_cfg(const uint16_t *w, const uint16_t *x, int T, int E, int H, float *logits,
                hipStream_t s) {
  const dim3 grid((E + 4 * EPW - 1) / (4 * EPW), (T + TT - 1) / TT);
  launch_k(COLI_K_ROUTER_LOGITS, router_kernel<EPW, TT>, grid, dim3(kThreads), 0, s, w, x, T,
           E, H, logits);
}

}  // namespace

int launch_router_logits(const Layer &L, const uint16_t *w, const uint16_t *x, int T,
                         float *logits, hipStream_t s) {
  // up to 16 tokens (H <= 8192): one wavefront per (expert, token), all
  // loads at once; otherwise staged tiles -- one expert per wavefront and the
  // whole batch per workgroup up to 16 tokens, else 4 experts x 16 tokens
  // per wavefront
  const int ntiles = (L.H / 8 + 63) / 64;
  if (T <= 16 && ntiles <= 16) {
    const dim3 grid((L.E + 3) / 4, T);
    if (ntiles <= 4)
      launch_k(COLI_K_ROUTER_LOGITS, router_one_kernel<4>, grid, dim3(kThreads), 0, s, w, x,
               L.E, L.H, logits);
    else if (ntiles <= 8)
      launch_k(COLI_K_ROUTER_LOGITS, router_one_kernel<8>, grid, dim3(kThreads), 0, s, w, x,
               L.E, L.H, logits);
    else if (ntiles <= 12)
      launch_k(COLI_K_ROUTER_LOGITS, router_one_kernel<12>, grid, dim3(kThreads), 0, s, w, x,
               L.E, L.H, logits);
    else
      launch_k(COLI_K_ROUTER_LOGITS, router_one_kernel<16>, grid, dim3(kThreads), 0, s, w, x,
               L.E, L.H, logits);
  } else if (T <= 1) launch_cfg<1, 1>(w, x, T, L.E, L.H, logits, s);
  else if (T <= 2) launch_cfg<1, 2>(w, x, T, L.E, L.H, logits, s);
  else if (T <= 4) launch_cfg<1, 4>(w, x, T, L.E, L.H, logits, s);
  else if (T <= 8) launch_cfg<1, 8>(w, x, T, L.E, L.H, logits, s);
  else if (T <= 16) launch_cfg<1, 16>(w, x, T, L.E, L.H, logits, s);
  else launch_cfg<4, 16>(w, x, T, L.E, L.H, logits, s);
  return hip_status(hipGetLastError());
}

}  // namespace coli
