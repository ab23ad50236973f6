// probe.hip -- measurement aids: a plain streaming read, to time the HBM
// read rate a kernel gets on this chip (the ceiling the decode GEMVs are
// compared with), and a register-only matrix-core loop, to time the issue
// rate of the instructions the prefill and decode kernels use.
//
// The access pattern is the decode GEMVs' without their arithmetic: 256-thread
// workgroups, every lane four 16-byte loads requested before any is used, so
// each load instruction of a wavefront reads 1 KiB contiguous and a
// wavefront 4 KiB.  The words are xor-combined and written only if the
// result is a fixed value, which keeps the loads live.
#include "device_common.h"
#include "internal.h"

namespace coli {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 4;  // 16-byte loads per lane

__global__ void __launch_bounds__(kThreads) read_probe_kernel(const uint4 *__restrict__ src,
                                                              int64_t n16,
                                                              uint32_t *__restrict__ sink) {
  const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int64_t base = wave * 64 * kLoads + (threadIdx.x & 63);
  uint4 v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
    v[i] = base + 64 * i < n16 ? src[base + 64 * i] : make_uint4(0u, 0u, 0u, 0u);
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kLoads; ++i) x ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
  if (x == 0x12345678u) sink[0] = x;
}

// Matrix cores: four independent accumulator chains per wavefront, so no
// instruction waits for the previous result of its own chain.  The chains
// start from different values: identical chains would be merged into one.
// iters >= 1, so the loop is a do-while.
constexpr int kChains = 4;
typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x4 __attribute__((ext_vector_type(4)));

template <int KIND>
__global__ void __launch_bounds__(kThreads) mfma_probe_kernel(int iters, uint32_t *__restrict__ sink) {
  const int l = threadIdx.x;
  const coli_i32x4 a = {l, 3 * l + 1, l ^ 0x55, (int)blockIdx.x};
  const coli_i32x4 b = {7 * l, l + 11, (int)blockIdx.x * 5, l ^ 0x3c};
  uint32_t x = 0;
  if constexpr (KIND == COLI_MFMA_BF16_K32) {
    // small finite bf16 operands: the bit patterns masked to exponents < 128
    const coli_i32x4 m = {0x3f7f3f7f, 0x3f7f3f7f, 0x3f7f3f7f, 0x3f7f3f7f};
    const probe_bf16x8 av = __builtin_bit_cast(probe_bf16x8, a & m);
    const probe_bf16x8 bv = __builtin_bit_cast(probe_bf16x8, b & m);
    probe_f32x4 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = probe_f32x4{(float)(l + j), 0.0f, (float)j, 1.0f};
    int n = iters;
    do {
#pragma unroll
      for (int j = 0; j < kChains; ++j)
        c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, c[j], 0, 0, 0);
    } while (--n > 0);
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      for (int v = 0; v < 4; ++v) x ^= __float_as_uint(c[j][v]);
  } else {
    coli_i32x4 c[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) c[j] = coli_i32x4{l + j, j, 0, 1};
    const long a2 = (long)(((uint64_t)(uint32_t)a.y << 32) | (uint32_t)a.x);
    const long b2 = (long)(((uint64_t)(uint32_t)b.y << 32) | (uint32_t)b.x);
    int n = iters;
    do {
#pragma unroll
      for (int j = 0; j < kChains; ++j) {
        if constexpr (KIND == COLI_MFMA_I8_K64)
          c[j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c[j], 0, 0, 0);
        else
          c[j] = __builtin_amdgcn_mfma_i32_16x16x32_i8(a2, b2, c[j], 0, 0, 0);
      }
    } while (--n > 0);
#pragma unroll
    for (int j = 0; j < kChains; ++j)
      for (int v = 0; v < 4; ++v) x ^= (uint32_t)c[j][v];
  }
  if (x == 0x12345678u) sink[0] = x;
}

}  // namespace

int launch_mfma_probe(int kind, int iters, int workgroups, uint32_t *sink, hipStream_t s) {
  const dim3 grid((unsigned)workgroups), block(kThreads);
  if (kind == COLI_MFMA_I8_K32)
    launch_k(COLI_K_MFMA_PROBE, mfma_probe_kernel<COLI_MFMA_I8_K32>, grid, block, 0, s, iters, sink);
  else if (kind == COLI_MFMA_I8_K64)
    launch_k(COLI_K_MFMA_PROBE, mfma_probe_kernel<COLI_MFMA_I8_K64>, grid, block, 0, s, iters, sink);
  else
    launch_k(COLI_K_MFMA_PROBE, mfma_probe_kernel<COLI_MFMA_BF16_K32>, grid, block, 0, s, iters,
             sink);
  return hip_status(hipGetLastError());
}

int launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s) {
  const int64_t n16 = bytes / 16;
  const int64_t per_block = (int64_t)kThreads * kLoads;
  const dim3 grid((unsigned)((n16 + per_block - 1) / per_block));
  launch_k(COLI_K_READ_PROBE, read_probe_kernel, grid, dim3(kThreads), 0, s,
           reinterpret_cast<const uint4 *>(src), n16, sink);
  return hip_status(hipGetLastError());
}

}  // namespace coli
