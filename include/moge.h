/*
 * moge.h - C ABI of the MoGE (Mixture of Grouped Experts) expert-layer forward
 * pass for AMD MI355X (gfx950).
 *
 * The layer (TechWalker, "华为发布Pangu Pro MoE...", section 一 创新架构; Reportify
 * concept page "分组混合专家模型", 技术创新细节; mokono.cn "盘古Pro MoE", 核心亮点 1):
 *   scores   l = x W_r^T (+ b)                          [T,N] float32
 *   softmax  p = softmax(l) over all N routed experts    (before any selection)
 *   routing  the N experts form M contiguous groups of G = N/M; every token takes
 *            its K' best experts from every group (K = M*K' slots per token), so
 *            each group receives exactly T*K' (token, expert) pairs: the imbalance
 *            score (busiest minus idlest group load) is zero by construction.
 *   experts  each routed expert e is a SwiGLU FFN
 *              FFN_e(v) = W_down,e ( silu(W_gate,e v) * (W_up,e v) )
 *   shared   always-on shared experts, stored as one SwiGLU of width I_s (the
 *            concatenation of the S shared experts), weight 1
 *   combine  y[t] = shared(x_t) + sum_k gate[t,k] * FFN_{idx[t,k]}(x_t),
 *            gate[t,k] = p[t, idx[t,k]] (not renormalised).
 *
 * Conventions shared by every entry point
 *   - Every pointer except `dims` is DEVICE memory owned by the caller; the library
 *     never allocates or frees device memory and keeps no device state.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream. Every
 *     call only validates on the host and enqueues kernels on `stream`; it never
 *     synchronises and never reads device data on the host. Device faults appear at
 *     the caller's next synchronisation.
 *   - Tensors marked "dtype" hold dims->dtype elements (float32 or bfloat16 bit
 *     patterns); scores, probabilities, gates and the router bias are float32;
 *     indices and counts are int32. Accumulation is float32; bf16 results are
 *     rounded to nearest-even.
 *   - All tensors are dense row-major. Weights keep the contraction dimension
 *     contiguous: w_gate/w_up [N, I, d], w_down [N, d, I], ws_gate/ws_up [I_s, d],
 *     ws_down [d, I_s], w_router [N, d].
 *   - Alignment: dtype tensors 16 bytes, int32/float32 arrays 4 bytes.
 *   - Errors: the status is returned and moge_last_error() holds a message for the
 *     calling thread. Invalid dims, a NULL required pointer or a misaligned pointer
 *     -> MOGE_ERR_INVALID_ARG; shapes outside the implemented limits ->
 *     MOGE_ERR_UNSUPPORTED; a workspace that is NULL or smaller than
 *     moge_workspace_size() -> MOGE_ERR_WORKSPACE; a failed kernel launch ->
 *     MOGE_ERR_HIP. In every error case nothing has been enqueued. T = 0 returns
 *     MOGE_OK and enqueues nothing.
 *   - Limits: N <= 256, K = M*K' <= 64, d, I and I_s multiples of 32 (one MFMA
 *     operand fragment spans 32 contraction elements, and every kernel reads whole
 *     fragments), T*K < 2^31,
 *     and under 4 GiB each: every activation buffer ([T*K, d], [T*K, I], [T, I_s])
 *     and one expert's gate and up weights together (2*I*d elements; 2*I_s*d for
 *     the shared experts), which the kernels address with 32-bit offsets.
 *   - Results are deterministic: repeated calls on the same inputs give identical
 *     bits (no floating-point atomics; integer histogram counts only).
 *
 * Tie rule for routing (the pages do not fix one): inside a group the larger
 * score wins; on equal float32 scores the lower expert index wins; +0.0 == -0.0.
 * Slot order: idx[t, g*K' + j] is the j-th choice of group g.
 */
#ifndef MOGE_H
#define MOGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOGE_F32 = 0, MOGE_BF16 = 1 } moge_dtype_t;

typedef enum {
  MOGE_OK = 0,
  MOGE_ERR_INVALID_ARG = 1,
  MOGE_ERR_UNSUPPORTED = 2,
  MOGE_ERR_WORKSPACE = 3,
  MOGE_ERR_HIP = 4
} moge_status_t;

typedef struct {
  int32_t T;            /* tokens in the batch (>= 0) */
  int32_t d;            /* hidden size */
  int32_t N;            /* routed experts */
  int32_t M;            /* expert groups; N % M == 0 */
  int32_t k_per_group;  /* K': experts taken from every group, 1 <= K' <= N/M */
  int32_t inter;        /* routed SwiGLU intermediate width I */
  int32_t shared_inter; /* total shared SwiGLU width I_s (0 = no shared experts) */
  int32_t dtype;        /* moge_dtype_t of activations and weights */
} moge_dims_t;

/* ABI version of this header (increments on any signature change). */
int32_t moge_abi_version(void);

/* Bytes of device workspace that moge_permute, moge_expert_ffn and
 * moge_layer_forward need for these dims (the maximum over the three);
 * 0 if the dims are invalid or unsupported. Pure host function. */
size_t moge_workspace_size(const moge_dims_t* dims);

/* Message of the last failed call on this thread ("" if none); never NULL. */
const char* moge_last_error(void);

/* Routing: global softmax then per-group top-K' (section 一 of the TechWalker page;
 * the Reportify concept page: every group routes its own top-K).
 *   logits    [T,N] float32 in        router scores
 *   probs     [T,N] float32 out       softmax over all N experts (nullable)
 *   topk_idx  [T,K] int32 out         chosen experts, slot g*K'+j = group g
 *   topk_gate [T,K] float32 out       p[t, topk_idx[t,k]]
 * Selection compares the float32 scores themselves, so it is exact and does not
 * depend on how exp() rounds. */
moge_status_t moge_route(const moge_dims_t* dims, const float* logits, float* probs,
                         int32_t* topk_idx, float* topk_gate, void* stream);

/* Permutation of the T*K (token, slot) pairs into expert-contiguous order: rows
 * sorted by expert, then by token; pair p = t*K + k.  Grouped routing gives every
 * expert group the same number of pairs (TechWalker page, section 一: with K'
 * experts taken per group, each device's load is T*K'); group_counts exposes it,
 * so the zero imbalance score can be checked per group.  The pages do not fix the
 * order of the rows inside an expert; token ascending (a stable counting sort) is
 * this library's choice, and it makes the permutation unique and bit-exact.
 *   topk_idx     [T,K] int32 in
 *   x            [T,d] dtype in
 *   counts       [N]   int32 out     rows per expert
 *   offsets      [N+1] int32 out     exclusive prefix sum of counts
 *   group_counts [M]   int32 out     rows per group; always T*K' (imbalance 0)
 *   sorted_pair  [R]   int32 out     row -> pair   (R = T*K)
 *   pair_row     [R]   int32 out     pair -> row
 *   x_perm       [R,d] dtype out     x_perm[row] = x[sorted_pair[row] / K] (nullable)
 *   ws, ws_bytes                     workspace (>= moge_workspace_size(dims))
 * Bit-exact and deterministic. topk_idx entries must lie in [0, N) and be distinct
 * within a token (as moge_route produces); other inputs give unspecified rows. */
moge_status_t moge_permute(const moge_dims_t* dims, const int32_t* topk_idx, const void* x,
                           int32_t* counts, int32_t* offsets, int32_t* group_counts,
                           int32_t* sorted_pair, int32_t* pair_row, void* x_perm,
                           void* ws, size_t ws_bytes, void* stream);

/* Grouped SwiGLU expert FFN over expert-contiguous rows (the grouped matmul of the
 * TechWalker page, section 三, "SwiftGMM"/"GroupMatmul"):
 *   y_perm[r] = FFN_e(x_perm[r])  for offsets[e] <= r < offsets[e+1]
 *   x_perm  [R,d] dtype in, R = T*K from dims
 *   offsets [N+1] int32 in (device)   row ranges per expert, offsets[N] == R
 *   w_gate, w_up [N,I,d], w_down [N,d,I] dtype in
 *   y_perm  [R,d] dtype out
 * Each expert takes the weight-streaming path or an MFMA tile path, chosen on the
 * device from its row count, within row ranges the host sets from the mean rows
 * per expert (R / N; no device data is read). The shared experts are this call with dims
 * N = M = K' = 1, inter = I_s, x_perm = x and offsets = {0, T}. */
moge_status_t moge_expert_ffn(const moge_dims_t* dims, const void* x_perm,
                              const int32_t* offsets, const void* w_gate, const void* w_up,
                              const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                              void* stream);

/* Gate-weighted combine back to token order (TechWalker page, section 一: a
 * token's output is the sum of its chosen experts' outputs weighted by their
 * probabilities from the softmax over all experts; mokono.cn 核心亮点 1: the
 * shared experts are always on and join the sum with weight 1):
 *   y[t] = shared_out[t] + sum_{k=0..K-1} topk_gate[t,k] * y_perm[pair_row[t*K+k]]
 * summed in float32 in slot order (the pages give no order; a fixed one keeps the
 * result deterministic), rounded once to dtype.
 *   y_perm [R,d] dtype, pair_row [R] int32, topk_gate [T,K] float32,
 *   shared_out [T,d] dtype (nullable = no shared term), y [T,d] dtype out. */
moge_status_t moge_combine(const moge_dims_t* dims, const void* y_perm, const int32_t* pair_row,
                           const float* topk_gate, const void* shared_out, void* y,
                           void* stream);

/* The whole layer forward pass on one stream with no host synchronisation
 * (TechWalker page, sections 一 and 三; mokono.cn 核心亮点 1): scores -> softmax
 * over all N experts -> per-group top-K' -> permutation -> routed experts (each
 * reads its token rows straight from x) -> shared experts -> combine.
 * Beyond the plain layer call it takes one optional input, logits_in (route on
 * scores the caller already has: the same fp32 scores on both sides of a parity
 * check, or scores computed elsewhere), and returns the gates as well as the
 * indices (topk_gate_out), so that a caller can rebuild the combine.
 *   x [T,d], w_router [N,d], router_bias [N] float32 (nullable),
 *   w_gate/w_up [N,I,d], w_down [N,d,I], ws_gate/ws_up [I_s,d], ws_down [d,I_s]
 *     (the ws_* pointers may be NULL only when shared_inter == 0),
 *   logits_in [T,N] float32 (nullable): route on these scores instead of computing
 *     x W_r^T + b (w_router/router_bias are then ignored and may be NULL),
 *   y [T,d] dtype out,
 *   logits_out [T,N] float32, topk_idx_out [T,K] int32, topk_gate_out [T,K]
 *     float32, group_counts_out [M] int32: optional copies of the intermediate
 *     results (nullable),
 *   ws, ws_bytes: workspace (>= moge_workspace_size(dims)). */
moge_status_t moge_layer_forward(const moge_dims_t* dims, const void* x, const void* w_router,
                                 const float* router_bias, const void* w_gate, const void* w_up,
                                 const void* w_down, const void* ws_gate, const void* ws_up,
                                 const void* ws_down, const float* logits_in, void* y,
                                 float* logits_out, int32_t* topk_idx_out, float* topk_gate_out,
                                 int32_t* group_counts_out, void* ws, size_t ws_bytes,
                                 void* stream);

/* Packed expert weights.  The layer's throughput at decode batch sizes is the
 * rate at which the expert weights stream from HBM.  Read in their row-major
 * layout, every load of the MFMA fragment a wave needs (16 weight rows x 32
 * contraction elements) touches 16 rows 64 bytes at a time; in the packed layout
 * that fragment is 512 contiguous elements and a wave's whole weight stream is one
 * contiguous range.  Pack once (weights are parameters), then run
 * moge_layer_forward_packed; results are bit-identical to moge_layer_forward.
 *
 * Layout: fragment tile = 16 rows x 32 contraction elements stored as 64 chunks of
 * 8 consecutive contraction elements; chunk l holds row l % 16, elements
 * 8*(l/16) .. 8*(l/16)+7.  Gate/up part of an expert: for row block b < I/16 and
 * step s < d/32, the gate tile then the up tile of rows 16b..16b+15, at tile index
 * (b*(d/32) + s)*2 + {0,1}.  Down part: for row block b < d/32 (32 rows) and step
 * s < I/32, the tiles of rows 32b..32b+15 and 32b+16..32b+31 at tile index
 * (b*(I/32) + s)*2 + {0,1}.  Buffer order: routed gate/up parts of experts 0..N-1,
 * routed down parts of experts 0..N-1, shared gate/up part, shared down part.
 * Its size equals the total size of the six row-major weight tensors. */

/* Bytes of the packed weight buffer for these dims; 0 if the dims are invalid. */
size_t moge_packed_weights_size(const moge_dims_t* dims);

/* Write the packed layout of the six row-major weight tensors into `packed`
 * (device, 256-byte aligned, >= moge_packed_weights_size bytes, caller-owned). A
 * pure copy; asynchronous on `stream`. */
moge_status_t moge_pack_weights(const moge_dims_t* dims, const void* w_gate, const void* w_up,
                                const void* w_down, const void* ws_gate, const void* ws_up,
                                const void* ws_down, void* packed, size_t packed_bytes,
                                void* stream);

/* moge_layer_forward with the expert weights taken from a moge_pack_weights
 * buffer (same arguments otherwise; same results, bit for bit). */
moge_status_t moge_layer_forward_packed(const moge_dims_t* dims, const void* x,
                                        const void* w_router, const float* router_bias,
                                        const void* packed, const float* logits_in, void* y,
                                        float* logits_out, int32_t* topk_idx_out,
                                        float* topk_gate_out, int32_t* group_counts_out,
                                        void* ws, size_t ws_bytes, void* stream);

/* moge_layer_forward_packed with no workspace argument, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  The workspace is a fixed
 * device array inside the library, MOGE_NOALLOC_SCRATCH_BYTES (128 MiB), of which
 * every GPU that loads the library holds its own copy until the process ends.
 * Dims whose moge_workspace_size() exceeds it give MOGE_ERR_UNSUPPORTED; at the
 * Pangu-Pro shape (d 5120, 64 experts, K 8, width 1344, shared width 5376) that
 * allows up to 645 tokens.  Arguments and results are those of
 * moge_layer_forward_packed, bit for bit.  The current device must be the
 * stream's device (MOGE_ERR_INVALID_ARG otherwise); the first call on a device
 * looks up the array's address there.  It never allocates or frees memory.
 * Every call on one GPU uses the same array, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls on one stream are
 * ordered and safe, but calls that overlap in time on one GPU (several streams or
 * threads) race and give undefined results. */
#define MOGE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
moge_status_t moge_layer_forward_packed_noalloc(const moge_dims_t* dims, const void* x,
                                                const void* w_router, const float* router_bias,
                                                const void* packed, const float* logits_in,
                                                void* y, float* logits_out,
                                                int32_t* topk_idx_out, float* topk_gate_out,
                                                int32_t* group_counts_out, void* stream);

/* Weight-only int8 experts (W8A16).  Quantised deployment of the experts is part
 * of the inference work on the TechWalker page (section 三 推理性能优化, expert-aware
 * quantisation); the CSDN page reports W8A8 within 1.2% of full accuracy.  This is
 * the weight half: every row of W_gate, W_up, W_down and of the shared experts'
 * weights holds int8 codes q with one float32 scale s, weight = s * q; activations,
 * H and the outputs stay bf16.  At decode batch sizes the layer streams its expert
 * weights from HBM, so one byte per weight halves the dominant stream.  Experts
 * with at most 32 rows stream their codes; larger ones (and the shared experts
 * of a batch above 32 tokens) take 64-row MFMA tiles that widen the codes from
 * LDS.  The int8 layer is meant for decode and mid-size batches; prefill batches,
 * where the matrix cores and not the weight stream set the time, belong to the
 * bf16 packed layer.
 * Requirements: dtype MOGE_BF16; d, inter and shared_inter multiples of 64
 * (MOGE_ERR_UNSUPPORTED otherwise).
 *
 * Buffer layout (each region starts at a 256-byte boundary):
 *   code tiles: routed gate/up parts of experts 0..N-1, routed down parts, shared
 *     gate/up part, shared down part;
 *   scales (float32): gate [N,I], up [N,I], down [N,d], shared gate [I_s],
 *     shared up [I_s], shared down [d].
 * Code tile = 16 rows x 64 contraction elements (1 KiB) stored as 64 chunks of 16
 * consecutive elements; chunk l holds row l % 16, elements 16*(l/16) ..
 * 16*(l/16)+15.  Gate/up part of an expert: for row block b < I/16 and step
 * s < d/64, the gate tile then the up tile of rows 16b..16b+15 at tile index
 * (b*(d/64) + s)*2 + {0,1}.  Down part: for row block b < d/32 and step s < I/64,
 * the tiles of rows 32b..32b+15 and 32b+16..32b+31 at tile index
 * (b*(I/64) + s)*2 + {0,1}. */

/* Bytes of the int8 expert-weight buffer for these dims; 0 if the dims are invalid
 * or outside the requirements above. */
size_t moge_w8_weights_size(const moge_dims_t* dims);

/* Build the int8 buffer from codes and scales the caller already has (a pure copy;
 * asynchronous on `stream`).  All device pointers:
 *   q_gate, q_up [N,I,d], q_down [N,d,I] int8 (16-byte aligned),
 *   s_gate, s_up [N,I], s_down [N,d] float32,
 *   qs_gate, qs_up [I_s,d], qs_down [d,I_s] int8, ss_gate, ss_up [I_s], ss_down [d]
 *     float32 (may be NULL only when shared_inter == 0),
 *   w8: 256-byte aligned, >= moge_w8_weights_size bytes, caller-owned. */
moge_status_t moge_pack_weights_w8(const moge_dims_t* dims, const int8_t* q_gate,
                                   const int8_t* q_up, const int8_t* q_down, const float* s_gate,
                                   const float* s_up, const float* s_down, const int8_t* qs_gate,
                                   const int8_t* qs_up, const int8_t* qs_down,
                                   const float* ss_gate, const float* ss_up,
                                   const float* ss_down, void* w8, size_t w8_bytes,
                                   void* stream);

/* Quantise the six row-major bf16 weight tensors (shapes as moge_layer_forward,
 * 16-byte aligned) into the int8 buffer, symmetric per output row:
 *   s = max_k |w[k]| / 127, q[k] = rint(w[k] / s) with ties to even, clamped to
 *   [-127, 127]; every step in float32 (IEEE division); a row of zeros gets s = 0,
 *   q = 0.  Weights must be finite.  Asynchronous on `stream`. */
moge_status_t moge_quantize_weights_w8(const moge_dims_t* dims, const void* w_gate,
                                       const void* w_up, const void* w_down, const void* ws_gate,
                                       const void* ws_up, const void* ws_down, void* w8,
                                       size_t w8_bytes, void* stream);

/* moge_layer_forward with the expert weights taken from an int8 buffer (other
 * arguments and the workspace as moge_layer_forward).  Routing, permutation and
 * combine are the same kernels; the experts compute, per output channel,
 * s * (sum_k a[k] * q[k]) in float32 from bf16 activations a, then SwiGLU and the
 * bf16 roundings of the bf16 layer. */
moge_status_t moge_layer_forward_w8(const moge_dims_t* dims, const void* x, const void* w_router,
                                    const float* router_bias, const void* w8,
                                    const float* logits_in, void* y, float* logits_out,
                                    int32_t* topk_idx_out, float* topk_gate_out,
                                    int32_t* group_counts_out, void* ws, size_t ws_bytes,
                                    void* stream);

/* Stage timing for profiling.  events: MOGE_STAGE_EVENTS hipEvent_t handles
 * (passed as void*) created by the caller; moge_layer_forward then records
 * events[0] before its first kernel and events[i] after stage i on its stream:
 * 1 router scores, 2 softmax + grouped top-K', 3 permutation, 4 gate/up + SwiGLU
 * (routed and shared), 5 down projection (routed and shared), 6 combine.
 * A NULL entry skips that point (each recorded event costs a few microseconds of
 * GPU time).  events == NULL or n_events == 0 turns recording off.  The setting
 * belongs to the calling thread.  Any other n_events -> MOGE_ERR_INVALID_ARG.
 * moge_layer_forward, moge_layer_forward_packed and moge_layer_forward_w8 record
 * them. */
#define MOGE_STAGE_EVENTS 7
moge_status_t moge_set_stage_events(void* const* events, int32_t n_events);

#ifdef __cplusplus
}
#endif

#endif /* MOGE_H */
