// abi.hip -- the extern "C" entry points: argument checks, workspace sizing,
// dispatch to the kernel launchers.  Every check runs on the host before any
// HIP call, so an invalid call launches nothing and writes nothing.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"

namespace coli {
namespace {

constexpr int kMaxHidden = 16384;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxDecodeT = 64;
constexpr int kMaxDecodeInter = 15360;  // the down GEMV stages 4.125*I bytes of LDS
constexpr int kMaxT = 65536;
constexpr int64_t kMaxPairs = int64_t(1) << 20;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_layer(const coli_moe_layer_t *l, Layer *out) {
  if (!l) return COLI_E_INVALID;
  const int H = l->hidden, I = l->inter;
  if (H < 64 || I < 64 || H > kMaxHidden || I > kMaxHidden || H % 64 || I % 64)
    return COLI_E_INVALID;
  if (l->n_experts < 1 || l->n_experts > kMaxExperts) return COLI_E_INVALID;
  if (l->n_shared < 0 || l->n_shared > 1) return COLI_E_INVALID;
  if (l->top_k < 1 || l->top_k > l->n_experts || l->top_k > kMaxTopK) return COLI_E_INVALID;
  if (l->flags & ~(uint32_t)(COLI_ROUTE_SIGMOID | COLI_ROUTE_RENORM | COLI_ACT_MXFP8))
    return COLI_E_INVALID;
  if (!isfinite(l->routed_scale)) return COLI_E_INVALID;
  if (l->weight_format != COLI_WEIGHTS_INT4 && l->weight_format != COLI_WEIGHTS_INT8 &&
      l->weight_format != COLI_WEIGHTS_MXFP4)
    return COLI_E_INVALID;
  // MXFP8 activations pair with MXFP4 weights only
  if ((l->flags & COLI_ACT_MXFP8) && l->weight_format != COLI_WEIGHTS_MXFP4) return COLI_E_INVALID;
  if (out) {
    out->H = H;
    out->I = I;
    out->E = l->n_experts;
    out->S = l->n_shared;
    out->k = l->top_k;
    out->flags = l->flags;
    out->routed_scale = l->routed_scale;
    out->q4 = l->q4;
    out->scales = l->scales;
    out->w8 = l->weight_format == COLI_WEIGHTS_INT8;
    out->f4 = l->weight_format == COLI_WEIGHTS_MXFP4;
    out->expert_bytes = out->w8 ? (int64_t)3 * I * H : (int64_t)3 * I * H / 2;
    out->expert_scales = (int64_t)3 * I * H / 64;
  }
  return COLI_OK;
}

int check_weights(const Layer &L) {
  if (!L.q4 || !L.scales) return COLI_E_INVALID;
  if (!aligned(L.q4, 16) || !aligned(L.scales, 16)) return COLI_E_ALIGN;
  return COLI_OK;
}

int check_route(const coli_moe_route_t *r) {
  if (!r || !r->topk_idx || !r->topk_w || !r->counts || !r->offsets || !r->pairs ||
      !r->pair_pos || !r->union_ids || !r->n_union)
    return COLI_E_INVALID;
  return COLI_OK;
}

int check_tokens(const Layer &L, int T, int max_t) {
  if (T < 1 || T > max_t) return COLI_E_INVALID;
  if ((int64_t)T * L.k > kMaxPairs) return COLI_E_INVALID;
  return COLI_OK;
}

int check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need) return COLI_E_WORKSPACE;
  if (need && !ws) return COLI_E_INVALID;
  if (need && !aligned(ws, 256)) return COLI_E_ALIGN;
  return COLI_OK;
}

int check_forward(const coli_moe_layer_t *layer, const coli_moe_route_t *route,
                  const uint16_t *x, int T, void *y, int y_dtype, void *ws, size_t ws_bytes,
                  int entry, Layer *L) {
  int rc = check_layer(layer, L);
  if (rc) return rc;
  if ((rc = check_weights(*L))) return rc;
  if ((rc = check_route(route))) return rc;
  if ((rc = check_tokens(*L, T, entry == COLI_ENTRY_DECODE ? kMaxDecodeT : kMaxT))) return rc;
  if (entry == COLI_ENTRY_DECODE && L->I > kMaxDecodeInter) return COLI_E_UNSUPPORTED;
  // the MX prefill stages k 256 at a time
  if (entry != COLI_ENTRY_DECODE && (L->flags & COLI_ACT_MXFP8) && (L->H % 256 || L->I % 256))
    return COLI_E_UNSUPPORTED;
  if (!x || !y) return COLI_E_INVALID;
  if (y_dtype != COLI_OUT_BF16 && y_dtype != COLI_OUT_F32) return COLI_E_INVALID;
  if (!aligned(x, 16) || !aligned(y, 16)) return COLI_E_ALIGN;
  const size_t need = entry == COLI_ENTRY_DECODE ? decode_workspace(*L, T)
                                                 : prefill_workspace(*L, T);
  return check_ws(ws, ws_bytes, need);
}

}  // namespace
}  // namespace coli

namespace coli {
coli_moe_trace_t *g_trace = nullptr;
// probe.hip: the plain streaming read behind coli_moe_read_probe
int launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, hipStream_t s);
int launch_mfma_probe(int kind, int iters, int workgroups, uint32_t *sink, hipStream_t s);
}

namespace coli {
namespace {

// Library-owned decode workspace for coli_moe_forward_decode_noalloc: one
// copy per GPU, held until the process ends.  Host code never uses this
// name as an address (on the host it is only a stand-in for the symbol);
// the device address of each GPU's copy comes from hipGetSymbolAddress and
// is cached per device below.
constexpr size_t kScratchBytes = size_t(32) << 20;
static_assert(kScratchBytes == COLI_NOALLOC_SCRATCH_BYTES, "scratch size and header disagree");
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of the current device's scratch array, looked up on the
// first call on that device (with that device current) and cached.
int scratch_ptr(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return COLI_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return COLI_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return COLI_OK;
}

}  // namespace
}  // namespace coli

using namespace coli;

extern "C" {

size_t coli_moe_workspace_bytes(const coli_moe_layer_t *layer, int32_t T, int32_t entry) {
  Layer L;
  if (check_layer(layer, &L)) return 0;
  switch (entry) {
    case COLI_ENTRY_ROUTE:
      return 0;  // routing needs no workspace
    case COLI_ENTRY_DECODE:
      return check_tokens(L, T, kMaxDecodeT) ? 0 : decode_workspace(L, T);
    case COLI_ENTRY_PREFILL:
      return check_tokens(L, T, kMaxT) ? 0 : prefill_workspace(L, T);
    default:
      return 0;
  }
}

int coli_moe_route(const coli_moe_layer_t *layer, const float *logits, const float *sel_bias,
                   int32_t T, const coli_moe_route_t *route, void *ws, size_t ws_bytes,
                   void *stream) {
  (void)ws;
  (void)ws_bytes;
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if ((rc = check_route(route))) return rc;
  if ((rc = check_tokens(L, T, kMaxT))) return rc;
  if (!logits) return COLI_E_INVALID;
  if (!aligned(logits, 4) || (sel_bias && !aligned(sel_bias, 4))) return COLI_E_ALIGN;
  return launch_route(L, logits, sel_bias, T, *route, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_route_hidden(const coli_moe_layer_t *layer, const uint16_t *w_router,
                          const uint16_t *x, const float *sel_bias, int32_t T, float *logits,
                          const coli_moe_route_t *route, void *ws, size_t ws_bytes,
                          void *stream) {
  (void)ws;
  (void)ws_bytes;
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if ((rc = check_route(route))) return rc;
  if ((rc = check_tokens(L, T, kMaxT))) return rc;
  if (!w_router || !x || !logits) return COLI_E_INVALID;
  if (!aligned(w_router, 16) || !aligned(x, 16) || !aligned(logits, 4) ||
      (sel_bias && !aligned(sel_bias, 4)))
    return COLI_E_ALIGN;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if ((rc = launch_router_logits(L, w_router, x, T, logits, s))) return rc;
  return launch_route(L, logits, sel_bias, T, *route, s);
}

int coli_moe_forward_decode(const coli_moe_layer_t *layer, const coli_moe_route_t *route,
                            const uint16_t *x, int32_t T, void *y, int32_t y_dtype, void *ws,
                            size_t ws_bytes, void *stream) {
  Layer L;
  const int rc = check_forward(layer, route, x, T, y, y_dtype, ws, ws_bytes, COLI_ENTRY_DECODE, &L);
  if (rc) return rc;
  return launch_decode(L, *route, x, T, y, y_dtype, ws, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_forward_decode_noalloc(const coli_moe_layer_t *layer, const coli_moe_route_t *route,
                                    const uint16_t *x, int32_t T, void *y, int32_t y_dtype,
                                    void *stream) {
  Layer L;
  // validated against the scratch size with a stand-in address (256-aligned,
  // never dereferenced); the real address is only taken once the call is valid
  void *const stand_in = reinterpret_cast<void *>(uintptr_t(256));
  const int rc = check_forward(layer, route, x, T, y, y_dtype, stand_in, kScratchBytes,
                               COLI_ENTRY_DECODE, &L);
  if (rc) return rc;
  void *ws = nullptr;
  const int prc = scratch_ptr(&ws);
  if (prc) return prc;
  return launch_decode(L, *route, x, T, y, y_dtype, ws, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_forward_prefill(const coli_moe_layer_t *layer, const coli_moe_route_t *route,
                             const uint16_t *x, int32_t T, void *y, int32_t y_dtype, void *ws,
                             size_t ws_bytes, void *stream) {
  Layer L;
  const int rc = check_forward(layer, route, x, T, y, y_dtype, ws, ws_bytes, COLI_ENTRY_PREFILL, &L);
  if (rc) return rc;
  return launch_prefill(L, *route, x, T, y, y_dtype, ws, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_quantize_q8_0(const void *src, int32_t src_dtype, int64_t n, int8_t *q,
                           uint16_t *d, void *stream) {
  if (!src || !q || !d) return COLI_E_INVALID;
  if (src_dtype != COLI_SRC_BF16 && src_dtype != COLI_SRC_F32) return COLI_E_INVALID;
  if (n < 32 || n % 32 || n > (int64_t(1) << 34)) return COLI_E_INVALID;
  if (!aligned(src, 16) || !aligned(q, 16) || !aligned(d, 4)) return COLI_E_ALIGN;
  return launch_quantize_q8_0(src, src_dtype, n, q, d, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_quantize_int4_gs64(const void *src, int32_t src_dtype, int64_t rows, int64_t K,
                                uint8_t *q4, uint16_t *scales, void *stream) {
  if (!src || !q4 || !scales) return COLI_E_INVALID;
  if (src_dtype != COLI_SRC_BF16 && src_dtype != COLI_SRC_F32) return COLI_E_INVALID;
  if (rows < 1 || K < 64 || K % 64 || rows > (int64_t(1) << 34) / K) return COLI_E_INVALID;
  if (!aligned(src, 16) || !aligned(q4, 4) || !aligned(scales, 2)) return COLI_E_ALIGN;
  return launch_quantize_int4(src, src_dtype, rows * K, q4, scales,
                              reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_quantize_int8_gs64(const void *src, int32_t src_dtype, int64_t rows, int64_t K,
                                int8_t *q, uint16_t *scales, void *stream) {
  if (!src || !q || !scales) return COLI_E_INVALID;
  if (src_dtype != COLI_SRC_BF16 && src_dtype != COLI_SRC_F32) return COLI_E_INVALID;
  if (rows < 1 || K < 64 || K % 64 || rows > (int64_t(1) << 34) / K) return COLI_E_INVALID;
  if (!aligned(src, 16) || !aligned(q, 8) || !aligned(scales, 2)) return COLI_E_ALIGN;
  return launch_quantize_int8(src, src_dtype, rows * K, q, scales,
                              reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_quantize_mxfp4(const void *src, int32_t src_dtype, int64_t rows, int64_t K,
                            uint8_t *q4, uint8_t *e8m0, void *stream) {
  if (!src || !q4 || !e8m0) return COLI_E_INVALID;
  if (src_dtype != COLI_SRC_BF16 && src_dtype != COLI_SRC_F32) return COLI_E_INVALID;
  if (rows < 1 || K < 32 || K % 32 || rows > (int64_t(1) << 34) / K) return COLI_E_INVALID;
  if (!aligned(src, 16) || !aligned(q4, 4)) return COLI_E_ALIGN;
  return launch_quantize_mxfp4(src, src_dtype, rows * K, q4, e8m0,
                               reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_read_probe(const void *src, int64_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink || bytes < 16 || bytes % 16 || bytes > (int64_t(1) << 36))
    return COLI_E_INVALID;
  if (!aligned(src, 16) || !aligned(sink, 4)) return COLI_E_ALIGN;
  return launch_read_probe(src, bytes, sink, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_mfma_probe(int32_t kind, int32_t iters, int32_t workgroups, uint32_t *sink,
                        void *stream) {
  if (kind < COLI_MFMA_I8_K32 || kind > COLI_MFMA_BF16_K32 || !sink || iters < 1 ||
      iters > (1 << 20) || workgroups < 1 || workgroups > (1 << 20))
    return COLI_E_INVALID;
  if (!aligned(sink, 4)) return COLI_E_ALIGN;
  return launch_mfma_probe(kind, iters, workgroups, sink, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_block_dots(const coli_moe_layer_t *layer, int32_t expert, int32_t matrix,
                        const int8_t *q_act, int32_t T, int32_t *dots, void *stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if ((rc = check_weights(L))) return rc;
  if (expert < 0 || expert >= L.E + L.S || matrix < 0 || matrix > 2) return COLI_E_INVALID;
  if (T < 1 || T > 4096 || !q_act || !dots) return COLI_E_INVALID;
  if (!aligned(q_act, 16) || !aligned(dots, 16)) return COLI_E_ALIGN;
  return launch_block_dots(L, expert, matrix, q_act, T, dots, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_quantize_mxfp8(const void *src, int32_t src_dtype, int64_t n, uint8_t *q,
                            uint8_t *e8m0, void *stream) {
  if (!src || !q || !e8m0) return COLI_E_INVALID;
  if (src_dtype != COLI_SRC_BF16 && src_dtype != COLI_SRC_F32) return COLI_E_INVALID;
  if (n < 32 || n % 32 || n > (int64_t(1) << 34)) return COLI_E_INVALID;
  if (!aligned(src, 16) || !aligned(q, 16)) return COLI_E_ALIGN;
  return launch_quantize_mxfp8(src, src_dtype, n, q, e8m0, reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_mx_dots(const coli_moe_layer_t *layer, int32_t expert, int32_t matrix,
                     const uint8_t *q_act, const uint8_t *e_act, int32_t T, float *out,
                     void *stream) {
  Layer L;
  int rc = check_layer(layer, &L);
  if (rc) return rc;
  if ((rc = check_weights(L))) return rc;
  if (!L.f4) return COLI_E_INVALID;
  if (expert < 0 || expert >= L.E + L.S || matrix < 0 || matrix > 2) return COLI_E_INVALID;
  if (T < 1 || T > 4096 || !q_act || !e_act || !out) return COLI_E_INVALID;
  if ((matrix == 2 ? L.I : L.H) % 256) return COLI_E_UNSUPPORTED;
  if (!aligned(q_act, 16) || !aligned(e_act, 4) || !aligned(out, 16)) return COLI_E_ALIGN;
  return launch_mx_dots(L, expert, matrix, q_act, e_act, T, out,
                        reinterpret_cast<hipStream_t>(stream));
}

int coli_moe_set_trace(coli_moe_trace_t *trace) {
  if (trace && (!trace->start || !trace->stop || !trace->kernel || trace->capacity < 0))
    return COLI_E_INVALID;
  g_trace = trace;
  return COLI_OK;
}

const char *coli_moe_strerror(int status) {
  switch (status) {
    case COLI_OK: return "ok";
    case COLI_E_INVALID: return "invalid argument";
    case COLI_E_UNSUPPORTED: return "unsupported layer shape";
    case COLI_E_WORKSPACE: return "workspace too small";
    case COLI_E_ALIGN: return "pointer misaligned";
    case COLI_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char *coli_moe_version(void) { return "0.1.0"; }

}  // extern "C"
