/*
 * coli_moe.h -- C ABI of the routed-expert MoE layer library (gfx950 / MI355X).
 *
 * One MoE layer of a colibri-style engine: a router picks the top-k routed
 * experts per token, the chosen (token, expert) pairs are grouped by expert so
 * that each distinct expert's weights are read once per batch (the "batch
 * union"), every chosen expert applies an int4 group-quantised gate/up
 * projection, SwiGLU and an int4 down projection, and the expert outputs are
 * summed with the routing weights (plus an always-on shared expert).
 *
 * Sources (web pages about the colibri engine):
 *  - tantan.ink post "colibri: 把 744B 模型当数据流..." section "它的核心判断":
 *    routed experts of about 19 MB int4 each, streamed on demand.
 *  - same post, section "几个关键工程动作": within a batch each distinct expert
 *    is read once, and its three matrices gate/up/down are stored adjacently.
 *  - same post, section "我看到的几个坑": the int4 container is group-scaled
 *    with one scale per 64 weights (gs64), not one per row.
 *  - alphamatch.ai blog "Colibri：革命性 AI 引擎..." section "優化整數核心":
 *    the integer kernel takes Q8_0-style int8 activations.
 *  - aixq.cc article, section "为什么值得关注": the router's choice decides
 *    which experts are loaded.
 * The pages state no formula for the router, the activation or the quantiser;
 * the readings taken here are written next to each definition below.
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless the comment says "host".  The caller
 *    owns every buffer; the library never allocates, frees or synchronises.
 *  - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL means the null stream).
 *  - Arguments are validated on the host before any launch.  On a failed
 *    check nothing is launched, no output is written, and a negative
 *    COLI_E_* code is returned.  A failed launch returns COLI_E_HIP; a fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give bit-identical outputs on
 *    every run (no floating-point atomics anywhere).
 *  - Calls that share a workspace or route buffer must not overlap in time.
 */
#ifndef COLI_MOE_H
#define COLI_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  COLI_OK = 0,
  COLI_E_INVALID = -1,     /* a NULL pointer, a size out of range, a bad flag */
  COLI_E_UNSUPPORTED = -2, /* a valid layer shape this build does not run */
  COLI_E_WORKSPACE = -3,   /* ws_bytes below coli_moe_workspace_bytes() */
  COLI_E_ALIGN = -4,       /* a pointer below its required alignment */
  COLI_E_HIP = -5          /* a HIP launch or device query failed */
};

/* ---- routing flags (coli_moe_layer_t.flags) ------------------------------
 * The pages do not name the routing function; both used by the model families
 * they list are provided.
 *  SOFTMAX: p = softmax over ALL E logits; w_j = p[idx_j].
 *  SIGMOID: w_j = 1 / (1 + exp(-logit[idx_j])).
 *  RENORM : afterwards w_j /= sum_j w_j over the k selected experts.
 * In every case w_j is then multiplied by routed_scale.  The weights always
 * use the raw logits; the optional selection bias only moves the choice.  */
enum {
  COLI_ROUTE_SOFTMAX = 0u,
  COLI_ROUTE_SIGMOID = 1u,
  COLI_ROUTE_RENORM = 1u << 8
};

/* ---- activation format of the prefill path (coli_moe_layer_t.flags) ------
 * COLI_ACT_MXFP8: for MXFP4 layers only (COLI_E_INVALID otherwise).  The
 * pages pair fp4 experts with fp8-e4m3 elsewhere in the same model
 * (ai-tools-nav review, model family table, the DeepSeek V4 row); with this
 * flag coli_moe_forward_prefill quantises the activations (x, and h between
 * the GEMMs) to MXFP8 -- OCP FP8 E4M3 codes with one E8M0 scale per 32
 * values, see coli_moe_quantize_mxfp8 -- instead of Q8_0, and runs both
 * GEMMs on gfx950's MX matrix cores, which apply the weight and activation
 * block scales themselves.  Needs H and I multiples of 256
 * (COLI_E_UNSUPPORTED otherwise).  Decode ignores the flag. */
enum { COLI_ACT_MXFP8 = 1u << 16 };

/* output element type of the forward calls */
enum { COLI_OUT_BF16 = 0, COLI_OUT_F32 = 1 };

/* source element type of the quantisers */
enum { COLI_SRC_BF16 = 0, COLI_SRC_F32 = 1 };

/* weight code width of the expert container (coli_moe_layer_t.weight_format) */
enum { COLI_WEIGHTS_INT4 = 0, COLI_WEIGHTS_INT8 = 1, COLI_WEIGHTS_MXFP4 = 2 };

/* workspace selector for coli_moe_workspace_bytes */
enum { COLI_ENTRY_ROUTE = 0, COLI_ENTRY_DECODE = 1, COLI_ENTRY_PREFILL = 2 };

/* ---- the gs64 expert container --------------------------------------------
 * Experts e = 0 .. E-1 are routed; when n_shared == 1, expert E is the shared
 * expert.  Every expert owns three matrices, stored adjacently in this order:
 *     gate [I rows x H]   up [I rows x H]   down [H rows x I]
 * Each matrix is row-major with its reduction dimension K contiguous
 * (K = H for gate/up, K = I for down).
 *  q4     : (E+S) * 3*I*H/2 bytes.  Byte j of row n holds weight k = 2j in
 *           its low nibble and k = 2j+1 in its high nibble; a nibble is a
 *           4-bit two's-complement integer q in [-8, 7].
 *           Expert e starts at byte e * 3*I*H/2; within it gate starts at 0,
 *           up at I*H/2, down at I*H.
 *  scales : (E+S) * 3*I*H/64 IEEE fp16 values.  Scale s[n][g] covers weights
 *           k in [64g, 64g+64) of row n; row n of a matrix holds K/64 scales.
 *           Expert e starts at element e * 3*I*H/64; gate at 0, up at I*H/64,
 *           down at 2*I*H/64.
 * The weight is w = q * s (symmetric, no zero point).  With H = 6144 and
 * I = 2048 one expert is 18,874,368 + 1,179,648 = 20,054,016 bytes, which
 * matches the roughly 19 MB per routed expert given for GLM-5.2 (tantan.ink
 * post, section "它的核心判断").
 * Requirements: H, I multiples of 64 in [64, 16384]; 1 <= E <= 1024;
 * n_shared in {0, 1}; 1 <= k <= min(E, 32); q4 and scales 16-byte aligned.
 *
 * int8 codes (weight_format = COLI_WEIGHTS_INT8): the same container with one
 * byte per weight, a two's-complement integer q in [-128, 127], in place of
 * a nibble: row n holds K bytes (byte k is weight k); a matrix is I*H bytes
 * and expert e starts at byte e * 3*I*H (gate at 0, up at I*H, down at
 * 2*I*H).  Scales are unchanged: one fp16 per 64 weights, w = q * s.  The
 * pages require int8 experts for the MTP layer (int4 there collapses the
 * draft acceptance; tantan.ink post, section "我看到的几个坑") and list the
 * OLMoE container as int8 (ai-tools-nav review, model family table); they do
 * not give its scale granularity, read here as the same gs64.  int8 layers
 * take every call and shape that int4 layers take.
 *
 * MXFP4 codes (weight_format = COLI_WEIGHTS_MXFP4): the pages list fp4
 * experts for Kimi K3 and DeepSeek V4 (ai-tools-nav review, model family
 * table) without the format; read as OCP MXFP4.  Codes are FP4 E2M1 nibbles
 * (bit 3 sign, bits 2-1 exponent with bias 1, bit 0 mantissa: 0, 0.5, 1,
 * 1.5, 2, 3, 4, 6), packed and laid out exactly like the int4 codes.  The
 * scales pointer holds E8M0 bytes instead of fp16: byte E[n][b] scales
 * weights k in [32b, 32b+32) of row n by 2^(E-127); E must be below 255.
 * One E8M0 byte per 32 weights takes the bytes of one fp16 per 64, so the
 * scale layout per expert and matrix is the same (gate at byte 0, up at
 * I*H/32, down at 2*I*H/32; expert e at byte e * 3*I*H/32).  Same calls and
 * shapes as int4 codes.  On the integer path the codes enter the
 * int8 matrix cores as 2 * E2M1 (integers in [-12, 12], exact) with the
 * scale halved; coli_moe_block_dots returns the dots of those doubled codes.
 */
typedef struct coli_moe_layer {
  int32_t hidden;        /* H */
  int32_t inter;         /* I */
  int32_t n_experts;     /* E, routed experts */
  int32_t n_shared;      /* S, 0 or 1 always-on shared experts (index E) */
  int32_t top_k;         /* k */
  uint32_t flags;        /* COLI_ROUTE_* | COLI_ACT_MXFP8 */
  float routed_scale;    /* multiplies every routing weight (1.0f usually) */
  const uint8_t *q4;     /* device, see above */
  const uint16_t *scales;/* device, fp16 bit patterns, see above */
  int32_t weight_format; /* COLI_WEIGHTS_INT4 (0), _INT8 or _MXFP4 */
} coli_moe_layer_t;

/* ---- route buffers (caller-allocated device memory) ---------------------
 * Written by coli_moe_route, read by the forward calls.  P = T*k pairs; pair
 * p = t*k + j is token t's j-th choice.
 *  topk_idx [P] int32 : experts of token t, by score descending, ties to the
 *                       lower expert index (score = logit [+ sel_bias]).
 *  topk_w   [P] fp32  : routing weights, see COLI_ROUTE_*.
 *  counts   [E] int32 : pairs routed to expert e.
 *  offsets  [E+1]     : exclusive prefix sum of counts; offsets[E] = P.
 *  pairs    [P] int32 : pair ids grouped by expert (expert 0 first); within
 *                       an expert in ascending pair id (= ascending token).
 *  pair_pos [P] int32 : inverse of pairs: pairs[pair_pos[p]] == p.
 *  union_ids[E] int32 : the batch union, experts with counts > 0 ascending;
 *                       entries past n_union are left unspecified.
 *  n_union  [1] int32 : size of the batch union (routed experts only).
 */
typedef struct coli_moe_route {
  int32_t *topk_idx;
  float *topk_w;
  int32_t *counts;
  int32_t *offsets;
  int32_t *pairs;
  int32_t *pair_pos;
  int32_t *union_ids;
  int32_t *n_union;
} coli_moe_route_t;

/* Bytes of device workspace an entry point needs for T tokens (entry is a
 * COLI_ENTRY_*).  Returns 0 for invalid arguments.  Host-only, no HIP call.
 * The workspace holds what the layer definition makes between its steps:
 * the SwiGLU output h and the down outputs o of every (token, expert) row of
 * the batch union, and on the integer path the Q8_0 codes and scales of x
 * and h (alphamatch.ai blog, section "優化整數核心"; batch union: tantan.ink
 * post, section "几个关键工程动作"). */
size_t coli_moe_workspace_bytes(const coli_moe_layer_t *layer, int32_t T,
                                int32_t entry);

/* Route T tokens: top-k selection, routing weights and grouping by expert.
 *  logits   [T*E] fp32 row-major, finite values.
 *  sel_bias [E] fp32 or NULL: added to the logits for selection only.
 *  T in [1, 65536] with T*k <= 2^20.
 * Selection and grouping are exact (comparisons and integer counts only).
 * Source: aixq.cc article, section "为什么值得关注" (the router decides which
 * experts load); tantan.ink post, section "几个关键工程动作" (batch union). */
int coli_moe_route(const coli_moe_layer_t *layer, const float *logits,
                   const float *sel_bias, int32_t T,
                   const coli_moe_route_t *route, void *ws, size_t ws_bytes,
                   void *stream);

/* Route T tokens from the layer input: router logits, then exactly what
 * coli_moe_route does with them.
 *   logits[t][e] = sum over k < H of x[t][k] * w_router[e][k]
 *  w_router [E*H] bf16 row-major (no bias);  x [T*H] bf16;  both 16-byte
 *           aligned.
 *  logits   [T*E] fp32, written (device memory owned by the caller).
 *  sel_bias, T, route, ws: as for coli_moe_route.
 * The products are exact in fp32 and summed in fp32 in one fixed order per
 * (token, expert) -- lane chunks of 8 values, 64 chunks per 512-value tile,
 * tiles in order, then a fixed butterfly -- whatever T is, so a token's
 * logits and its expert choice do not depend on the rest of the batch.
 * Source: aixq.cc article, sections "为什么值得关注" and "我的真实看法" (the
 * router picks the experts and runs ahead of their loads); the pages give
 * no formula, so the router is read as a dense linear layer without bias. */
int coli_moe_route_hidden(const coli_moe_layer_t *layer, const uint16_t *w_router,
                          const uint16_t *x, const float *sel_bias, int32_t T,
                          float *logits, const coli_moe_route_t *route, void *ws,
                          size_t ws_bytes, void *stream);

/* Decode-shaped forward, T in [1, 64] tokens (single-token decode and
 * multi-token verify); needs I <= 15360 (COLI_E_UNSUPPORTED otherwise).  Activations stay bf16 -> fp32; weights are
 * dequantised in registers (w = q*s exactly); products are accumulated in
 * fp32.  For each token t:
 *   y[t] = sum_j topk_w[t,j] * FFN_{topk_idx[t,j]}(x[t]) + [S] FFN_E(x[t])
 *   FFN_e(x) = W_down * (silu(W_gate x) .* (W_up x)),  silu(g) = g/(1+e^-g)
 * Every distinct expert's weights are streamed from HBM once per call.
 * A token's result does not depend on which other tokens share the batch,
 * among batches of 1-16 tokens and among batches of 17-64 tokens; with
 * I = 2048 the down projection of the two ranges runs on different units
 * (matrix cores, vector dot products) and rounds differently.
 *  x [T*H] bf16;  y [T*H] bf16 (round-to-nearest-even) or fp32 (y_dtype).
 * Sources: tantan.ink post, sections "它的核心判断" and "几个关键工程动作". */
int coli_moe_forward_decode(const coli_moe_layer_t *layer,
                            const coli_moe_route_t *route, const uint16_t *x,
                            int32_t T, void *y, int32_t y_dtype, void *ws,
                            size_t ws_bytes, void *stream);

/* coli_moe_forward_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The h and o rows live in a
 * library-owned device array of 32 MiB (COLI_NOALLOC_SCRATCH_BYTES), one
 * per GPU, held until the process ends; the call allocates and frees
 * nothing.  Same arguments, kernels and results as coli_moe_forward_decode.
 * Returns COLI_E_WORKSPACE, before any launch, when coli_moe_workspace_bytes
 * (layer, T, COLI_ENTRY_DECODE) -- T*(k+S) rows of H + I fp32 values --
 * exceeds the array; every GLM-shaped call (H + I = 8192, k + S = 9,
 * T <= 64) fits, 64 tokens at k = 32 and H = 16384 do not.  The first call on a device
 * looks up that device's copy (hipGetSymbolAddress) with it current; make
 * it outside graph capture.  Every call on one GPU uses the same array, so
 * calls that overlap on one GPU (several streams, several host threads) race
 * and must be serialised by the caller.  No memory has to start at zero. */
#define COLI_NOALLOC_SCRATCH_BYTES (32u << 20)
int coli_moe_forward_decode_noalloc(const coli_moe_layer_t *layer,
                                    const coli_moe_route_t *route, const uint16_t *x,
                                    int32_t T, void *y, int32_t y_dtype, void *stream);

/* Prefill-shaped forward, T in [1, 65536] tokens, on the integer path:
 *  1. x[t] (bf16 -> fp32) is quantised Q8_0 per 32 values (see below).
 *  2. g, u = sum over 32-blocks b of s[n][b/2] * d_x[t][b] * dot_b, where
 *     dot_b is the exact int32 product of the int4 weights and the int8
 *     activations over block b (int8 matrix cores).
 *  3. h = silu(g) * u in fp32, quantised Q8_0 per 32 values along I.
 *  4. o = the same block-scaled integer product of W_down and q_h.
 *  5. y[t] = sum_j topk_w[t,j] * o_{t,j} + [S] o_shared(t).
 * Source: alphamatch.ai blog, section "優化整數核心" (Q8_0-style int8
 * activations feeding an integer dot kernel) and section "技術卓越"
 * (batched-union MoE in prefill). */
int coli_moe_forward_prefill(const coli_moe_layer_t *layer,
                             const coli_moe_route_t *route, const uint16_t *x,
                             int32_t T, void *y, int32_t y_dtype, void *ws,
                             size_t ws_bytes, void *stream);

/* Q8_0 quantisation of n values (n a multiple of 32), the activation format
 * of the integer path (alphamatch.ai blog, section "優化整數核心").  Per block
 * of 32 fp32 values v: a = max|v|; d = a / 127 (IEEE fp32 division);
 * q = round-half-away-from-zero(v / d) clamped to [-127, 127], or 0 when
 * a == 0; the stored scale is d rounded to fp16 (nearest-even).  The values
 * are quantised with the fp32 d, and the fp16 d is what the dot products use.
 *  src [n] bf16 or fp32 (src_dtype);  q [n] int8;  d [n/32] fp16 bits.
 * The same device code as the prefill path's quantiser. */
int coli_moe_quantize_q8_0(const void *src, int32_t src_dtype, int64_t n,
                           int8_t *q, uint16_t *d, void *stream);

/* The int4 gs64 container from float weights: quantises rows x K values
 * (K a multiple of 64, row-major, K contiguous) into the container's nibble
 * and scale layout.  The container's format is fixed by the pages (tantan.ink
 * post, section "我看到的几个坑": symmetric int4 with one fp16 scale per 64
 * weights); the offline conversion of a float checkpoint into it, shard by
 * shard, by the tantan.ink post (section "几个关键工程动作") and the siami.tw
 * article (section "技術核心").  The quantiser is not given there; per group
 * of 64 consecutive weights w:
 *   a = max |w|;  s = a / 7 (IEEE fp32 division);  s16 = s rounded to fp16
 *   (nearest-even);  q = round-half-away-from-zero(w / float(s16)) (IEEE fp32
 *   division), clamped to [-8, 7];  q = 0 for every weight of a group whose
 *   s16 is 0.
 *  src    [rows*K] bf16 or fp32 (src_dtype), device, 16-byte aligned; the
 *         values must be finite with max |w| <= 7 * 65504.
 *  q4     [rows*K/2] bytes, device, 4-byte aligned: weight k of a row in the
 *         low nibble of byte k/2 when k is even, else the high nibble.
 *  scales [rows*K/64] fp16 bits, device, 2-byte aligned.
 * Groups are independent and flat, so matrices stored back to back (gate,
 * up and down of an expert, or a whole container in container order) can be
 * quantised in one call with rows*K their total size; rows*K <= 2^34 (one
 * work-item per 8 values keeps the grid within a dispatch's 2^32 items).
 * Returns COLI_E_INVALID for a bad size, dtype or null pointer and
 * COLI_E_ALIGN for misaligned buffers; the outputs are then untouched. */
int coli_moe_quantize_int4_gs64(const void *src, int32_t src_dtype, int64_t rows,
                                int64_t K, uint8_t *q4, uint16_t *scales, void *stream);

/* The int8 gs64 container (COLI_WEIGHTS_INT8) from float weights: the int4
 * rule above widened to bytes -- per group of 64, s16 = fp16_RNE(max|w| /
 * 127), q = round-half-away-from-zero(w / float(s16)) clamped to [-128, 127]
 * (0 for a group whose s16 is 0).  The pages require int8 experts in the
 * MTP layer (tantan.ink post, section "我看到的几个坑") without the rule.
 *  src [rows*K] bf16 or fp32, 16-byte aligned, finite, max|w| <= 127 * 65504;
 *  q [rows*K] int8, 8-byte aligned (byte k of row n at n*K + k);
 *  scales [rows*K/64] fp16 bits, 2-byte aligned.  K % 64 == 0,
 *  rows*K <= 2^34.  Errors as for coli_moe_quantize_int4_gs64. */
int coli_moe_quantize_int8_gs64(const void *src, int32_t src_dtype, int64_t rows,
                                int64_t K, int8_t *q, uint16_t *scales, void *stream);

/* MXFP4 (COLI_WEIGHTS_MXFP4) from float weights by the OCP microscaling
 * conversion: per block of 32 consecutive weights, E = floor(log2 max|w|) -
 * 2 + 127 clamped to [0, 254] (0 for an all-zero block), stored as the E8M0
 * byte; each weight becomes the FP4 E2M1 code nearest to w / 2^(E-127),
 * ties to the even code, saturating at +-6, with the sign of w (also of a
 * zero).  The pages list fp4 experts (ai-tools-nav review, model family
 * table); this is the published MX conversion.
 *  src [rows*K] bf16 or fp32, 16-byte aligned, finite;  q4 [rows*K/2]
 *  nibbles (even k low), 4-byte aligned;  e8m0 [rows*K/32] bytes.
 *  K % 32 == 0, rows*K <= 2^34.  Errors as for coli_moe_quantize_int4_gs64. */
int coli_moe_quantize_mxfp4(const void *src, int32_t src_dtype, int64_t rows, int64_t K,
                            uint8_t *q4, uint8_t *e8m0, void *stream);

/* Measurement aid, not a step of the layer: reads `bytes` bytes of device
 * memory once with the access pattern of the decode GEMVs and none of their
 * arithmetic (256-thread workgroups, each lane four 16-byte loads, each load
 * instruction of a wavefront 1 KiB contiguous), so that a caller can time
 * the plain read rate a kernel gets from HBM on this chip.  The loaded words
 * are combined, and sink[0] is written only if the result equals 0x12345678,
 * which keeps the loads live without a write per workgroup.
 *  src device, 16-byte aligned; bytes a positive multiple of 16, at most
 *  2^36.  COLI_E_INVALID / COLI_E_ALIGN on bad arguments. */
int coli_moe_read_probe(const void *src, int64_t bytes, uint32_t *sink, void *stream);

/* Measurement aid, not a step of the layer: the matrix-core issue rate of
 * one instruction on this chip, with no memory traffic.  `workgroups`
 * workgroups of 4 wavefronts; each wavefront runs `iters` rounds of 4
 * independent accumulations of the instruction `kind` on register operands.
 * Operations per launch = workgroups x 4 x iters x 4 x ops(kind), where
 * ops = 2 x 16 x 16 x K: K = 32 (COLI_MFMA_I8_K32, the instruction the
 * prefill kernels issue), 64 (COLI_MFMA_I8_K64, the instruction the int8
 * peak is quoted for) or 32 (COLI_MFMA_BF16_K32, the decode down kernel's).
 * sink[0] is written only if the accumulators combine to 0x12345678.
 *  iters and workgroups in [1, 2^20].  COLI_E_INVALID / COLI_E_ALIGN. */
enum { COLI_MFMA_I8_K32 = 0, COLI_MFMA_I8_K64 = 1, COLI_MFMA_BF16_K32 = 2 };
int coli_moe_mfma_probe(int32_t kind, int32_t iters, int32_t workgroups, uint32_t *sink,
                        void *stream);

/* The exact int32 block dot products of one weight matrix of one expert
 * with T rows of int8 activations -- the integer unit of the pages' kernel,
 * which multiplies Q8_0-style int8 activations with the integer weight codes
 * (alphamatch.ai blog, section "優化整數核心").  Weight scales cover 64
 * codes and activation scales 32 values, so the 32-wide block is the unit
 * both scales are constant over:
 *   dots[t][n][b] = sum_{k in [32b, 32b+32)} qw[n][k] * q_act[t][k]
 *  matrix 0 = gate, 1 = up (K = H, rows = I), 2 = down (K = I, rows = H).
 *  q_act [T*K] int8, T in [1, 4096];  dots [T*rows*(K/32)] int32.
 * Computed by the prefill path's int8 matrix-core tile code, for checking it
 * bit for bit. */
int coli_moe_block_dots(const coli_moe_layer_t *layer, int32_t expert,
                        int32_t matrix, const int8_t *q_act, int32_t T,
                        int32_t *dots, void *stream);

/* MXFP8 quantisation of n values (n a multiple of 32), the activation format
 * of the MX path (COLI_ACT_MXFP8), following the OCP microscaling
 * conversion.  Per block of 32 values v: X = floor(log2 max|v|) - 8 (8 = the
 * largest FP8 E4M3 exponent), stored as E8M0 byte E = X + 127 clamped to
 * [0, 254] (E = 0 for an all-zero block); each value becomes the E4M3 code
 * (bit 7 sign, exponent bias 7, 3 mantissa bits, subnormals, magnitude 0x7f
 * unused) nearest to v / 2^(E-127), ties to the even code, saturating at
 * +-448, the sign kept also for zero.
 *  src [n] bf16 or fp32 (src_dtype);  q [n] E4M3 codes;  e8m0 [n/32].
 * The same device code as the MX prefill path's quantiser. */
int coli_moe_quantize_mxfp8(const void *src, int32_t src_dtype, int64_t n,
                            uint8_t *q, uint8_t *e8m0, void *stream);

/* One weight matrix of one expert of an MXFP4 layer against T rows of MXFP8
 * activations, on the MX matrix cores -- the GEMM of the MX prefill path:
 *   out[t][n] = sum over 32-blocks b of 2^(Ew[n][b]-127) * 2^(Ea[t][b]-127)
 *               * sum_{k in block b} e2m1(w[n][k]) * e4m3(a[t][k])
 * accumulated in fp32 by the hardware (its order is not specified).
 *  matrix 0 = gate, 1 = up (K = H, rows = I), 2 = down (K = I, rows = H);
 *  K must be a multiple of 256 (COLI_E_UNSUPPORTED otherwise).
 *  q_act [T*K] E4M3 codes, e_act [T*K/32] E8M0, T in [1, 4096];
 *  out [T*rows] fp32.  COLI_E_INVALID for layers that are not MXFP4. */
int coli_moe_mx_dots(const coli_moe_layer_t *layer, int32_t expert, int32_t matrix,
                     const uint8_t *q_act, const uint8_t *e_act, int32_t T, float *out,
                     void *stream);

/* ---- optional kernel timing ----------------------------------------------
 * For benchmarks and profilers.  After coli_moe_set_trace(t) with t != NULL,
 * every later launch hands t->start[i] and t->stop[i] to the dispatch of its
 * i-th kernel (hipExtLaunchKernel), so the two events carry that kernel's own
 * start and end times on the call's stream; it stores the kernel's COLI_K_*
 * id in t->kernel[i] (host memory) and increments t->count, until count
 * reaches capacity (further kernels launch untimed).  start/stop hold
 * hipEvent_t handles created by the caller.  Timed launches cannot be
 * captured into a HIP graph; coli_moe_set_trace(NULL) turns timing off.  The
 * trace pointer is process-wide: set it from one thread, with no call in
 * flight. */
enum {
  COLI_K_ROUTE_FUSED = 0, COLI_K_TOPK = 1, COLI_K_GROUP = 2, COLI_K_DECODE_GATEUP = 3,
  COLI_K_DECODE_DOWN = 4, COLI_K_COMBINE = 5, COLI_K_QUANTIZE = 6, COLI_K_PLAN = 7,
  COLI_K_GEMM_GATEUP = 8, COLI_K_GEMM_DOWN = 9, COLI_K_BLOCK_DOTS = 10,
  COLI_K_ROUTER_LOGITS = 11, COLI_K_QUANTIZE_INT4 = 12, COLI_K_QUANTIZE_INT8 = 13,
  COLI_K_QUANTIZE_MXFP4 = 14, COLI_K_READ_PROBE = 15,
  COLI_K_MFMA_PROBE = 16, COLI_K_COUNT = 17
};
typedef struct coli_moe_trace {
  void **start;     /* hipEvent_t[capacity] */
  void **stop;      /* hipEvent_t[capacity] */
  int32_t *kernel;  /* host [capacity]: COLI_K_* of each timed kernel */
  int32_t capacity;
  int32_t count;    /* kernels timed so far */
} coli_moe_trace_t;
int coli_moe_set_trace(coli_moe_trace_t *trace);

/* Static description of a status code. */
const char *coli_moe_strerror(int status);

/* Library version, "major.minor.patch". */
const char *coli_moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* COLI_MOE_H */
