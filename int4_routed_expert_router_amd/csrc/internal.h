// internal.h -- host-side declarations shared by the library's source files.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stddef.h>
#include <stdint.h>

#include "coli_moe.h"

namespace coli {

// A validated copy of the layer description with derived sizes.
struct Layer {
  int H, I, E, S, k;
  uint32_t flags;
  float routed_scale;
  const uint8_t *q4;
  const uint16_t *scales;
  int w8;                 // int8 byte codes (else nibbles)
  int f4;                 // MXFP4: E2M1 nibbles, one E8M0 scale byte per 32 weights
  int64_t expert_bytes;   // 3*I*H/2 (int4, MXFP4) or 3*I*H (int8)
  int64_t expert_scales;  // 3*I*H/64 16-bit units (fp16 per 64, or two E8M0 bytes)
};

// Workspace carving: every region 256-byte aligned.
inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

// Upper bound of distinct routed experts in a batch of T tokens.
inline int max_union(const Layer &L, int T) {
  long long p = (long long)T * L.k;
  return (int)(p < L.E ? p : L.E);
}

// Rows of the pair-major intermediate buffers: T*k routed pairs, then T
// shared-expert rows.
inline int64_t pair_rows(const Layer &L, int T) { return (int64_t)T * (L.k + L.S); }

size_t decode_workspace(const Layer &L, int T);
size_t prefill_workspace(const Layer &L, int T);

int launch_route(const Layer &L, const float *logits, const float *sel_bias, int T,
                 const coli_moe_route_t &r, hipStream_t s);
int launch_decode(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                  void *y, int y_dtype, void *ws, hipStream_t s);
int launch_prefill(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                   void *y, int y_dtype, void *ws, hipStream_t s);
// Router logits x . W_r^T (router.hip).
int launch_router_logits(const Layer &L, const uint16_t *w, const uint16_t *x, int T,
                         float *logits, hipStream_t s);
// Streaming gate/up + down GEMVs for decode batches of up to kMaxStreamT
// tokens (decode_stream.hip); false if the shape has no streaming path.
constexpr int kMaxStreamT = 16;
bool launch_decode_stream(const Layer &L, const coli_moe_route_t &r, const uint16_t *x, int T,
                          float *h, float *o, hipStream_t s, hipError_t *err);
void launch_combine(const float *o, const coli_moe_route_t &r, int T, int H, int k, int S,
                    void *y, int y_dtype, hipStream_t s);
int launch_quantize_q8_0(const void *src, int src_dtype, int64_t n, int8_t *q, uint16_t *d,
                         hipStream_t s);
int launch_quantize_int4(const void *src, int src_dtype, int64_t n, uint8_t *q4,
                         uint16_t *scales, hipStream_t s);
int launch_quantize_int8(const void *src, int src_dtype, int64_t n, int8_t *q, uint16_t *scales,
                         hipStream_t s);
int launch_quantize_mxfp4(const void *src, int src_dtype, int64_t n, uint8_t *q4, uint8_t *e8,
                          hipStream_t s);
int launch_block_dots(const Layer &L, int expert, int matrix, const int8_t *q_act, int T,
                      int32_t *dots, hipStream_t s);
// MX path (prefill.hip): MXFP8 quantiser and one matrix's MX GEMM in fp32.
int launch_quantize_mxfp8(const void *src, int src_dtype, int64_t n, uint8_t *q, uint8_t *e8,
                          hipStream_t s);
int launch_mx_dots(const Layer &L, int expert, int matrix, const uint8_t *qa, const uint8_t *ea,
                   int T, float *out, hipStream_t s);

inline int hip_status(hipError_t e) { return e == hipSuccess ? COLI_OK : COLI_E_HIP; }

// Optional per-kernel timing (coli_moe_set_trace).  Every kernel goes out
// through launch_k: with a trace set and a free slot, the dispatch itself
// stamps the slot's start and stop events (hipExtLaunchKernel), so the
// recorded span is the kernel's own execution and nothing is queued between
// kernels; otherwise it is a plain launch (which a HIP graph can capture).
extern coli_moe_trace_t *g_trace;
template <typename... P, typename... A>
void launch_k(int kernel_id, void (*kernel)(P...), dim3 grid, dim3 block, size_t lds,
              hipStream_t s, A... args) {
  coli_moe_trace_t *t = g_trace;
  if (t && t->count < t->capacity) {
    const int slot = t->count++;
    t->kernel[slot] = kernel_id;
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s,
                          reinterpret_cast<hipEvent_t>(t->start[slot]),
                          reinterpret_cast<hipEvent_t>(t->stop[slot]), 0u, static_cast<P>(args)...);
  } else {
    kernel<<<grid, block, lds, s>>>(static_cast<P>(args)...);
  }
}

}  // namespace coli
