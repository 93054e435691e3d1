/*
 * moe.h - C ABI of one GPU's Mixture-of-Experts layer for AMD Instinct MI355X
 * (gfx950).
 *
 * The layer is the one laid out on the AMD blog "MoE Training Optimization
 * with Primus" (MegaMoE section, layer dataflow of Figure 7), without its two
 * all-to-all stages.  A router gives every token a score per expert and keeps
 * the k best; the tokens are reordered so that each expert's rows sit
 * together; per expert, an up-projection pair (gate and up) feeds a SwiGLU
 * whose output the down-projection maps back, both as grouped GEMMs over all
 * experts; the last stage weights each token's k expert outputs by its gates
 * and sums them into the token's row.  The permuted buffer is padding-free in the sense of the
 * X-MoE verdict page on pith.science (key_machinery field): it holds only the
 * routed rows, with token ids, counts and combine weights beside it.  The
 * backward follows the same page's dispatch/combine duality (data-gradient
 * GEMMs, and weight-gradient GEMMs whose contraction length is each expert's
 * row count).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees, keeps or allocates memory.  Arrays are row-major and
 *    contiguous.  Outputs must not alias inputs.
 *  - Pointers must be 16-byte aligned (moe_mx_quantize_t relaxes this for
 *    its outputs, as stated there).
 *  - Everything is asynchronous and ordered on `stream` (a hipStream_t; NULL
 *    is the null stream).  No call synchronises the host, copies device data
 *    to the host, or allocates: per-expert counts stay on the GPU.
 *  - Scratch memory is the caller's `ws` buffer of `ws_bytes` bytes, sized by
 *    moe_workspace_size(); it may be reused between calls that are ordered
 *    on one stream.
 *  - Arguments are validated before anything is enqueued.  On error the call
 *    returns a negative moe_status, launches nothing and leaves every output
 *    untouched.  A failed kernel launch returns MOE_ERR_HIP.
 *  - Results are bitwise deterministic run to run (no floating-point
 *    atomics), with stated exceptions: moe_grouped_ffn_combine and
 *    moe_grouped_ffn_mxfp8_combine, whose fp32 atomic additions are
 *    order-independent only with at most two addends per output element.
 *    The library keeps no mutable global state (moe_set_phase_events keeps
 *    one per-thread pointer for measurement).
 *
 * Dtypes: `dtype` selects the storage type of x, the weights and the
 * materialised intermediates x_perm, h, y_perm, gu_save (MOE_DTYPE_BF16 or
 * MOE_DTYPE_F32).  Every GEMM accumulates in fp32.  Router logits, gates, the
 * combined output y and every gradient output are fp32.
 *
 * Weight layouts ([out_features, in_features] per expert, so that every
 * forward GEMM contracts over contiguous memory):
 *     w_router [E, d]       logits  = x . w_router^T (+ router_bias)
 *     w_gate   [E, F, d]    g       = x_perm[rows of e] . w_gate[e]^T
 *     w_up     [E, F, d]    u       = x_perm[rows of e] . w_up[e]^T
 *     w_down   [E, d, F]    y_perm  = (silu(g) * u) . w_down[e]^T
 *     ws_gate, ws_up [Fs, d]; ws_down [d, Fs]  the shared expert
 * All experts of one matrix live in one contiguous tensor.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a null, misaligned or out-of-range argument   */
  MOE_ERR_UNSUPPORTED = -2, /* a valid shape this build does not run         */
  MOE_ERR_WORKSPACE = -3,   /* ws is null or smaller than moe_workspace_size  */
  MOE_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed    */
} moe_status;

enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_FFN = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_BACKWARD = 4,
  MOE_OP_FFN_MXFP8 = 5,
  MOE_OP_BACKWARD_RECOMPUTE = 6,  /* moe_ffn_backward with gu_save NULL */
  MOE_OP_FFN_COMBINE = 7,         /* moe_grouped_ffn_combine */
  MOE_OP_BACKWARD_MXFP8 = 8       /* moe_ffn_backward_mxfp8 */
};

/* The layer's parameters: tokens T, hidden d, routed experts E, experts per
 * token k, routed expert FFN width F, shared expert width F_shared (the
 * DeepSeek-V3 memory-model page's b*s, h, N, N_r, h_E).  R := T * k routed
 * rows.
 * Limits: T >= 0, d >= 1, 1 <= E <= 1024, 1 <= k <= min(E, 64), F >= 1,
 * F_shared >= 0.  n_groups >= 1 divides E, n_groups <= 64,
 * 1 <= topk_groups <= n_groups, topk_groups * (E / n_groups) >= k; a group
 * limit (n_groups > 1) needs score = MOE_SCORE_SIGMOID.  renorm is 0 or 1.
 * wgrad_mx is 0 or 1.  T * k, T * max(d, 2F, F_shared, E) and F * d must
 * be below 2^31 (R * d itself is not bounded: routed rows are addressed
 * with 64-bit offsets). */
typedef struct moe_shape {
  int32_t T, d, E, k, F;
  int32_t F_shared;
  int32_t n_groups, topk_groups;
  int32_t score;
  int32_t renorm;
  int32_t dtype;
  int32_t wgrad_dtype;  /* storage of moe_ffn_backward's weight gradients:
                           MOE_DTYPE_F32 (0, the default) or MOE_DTYPE_BF16 */
  int32_t wgrad_mx;     /* moe_ffn_backward_mxfp8 only: 0 (the default) keeps
                           its weight-gradient GEMMs in bf16; 1 runs them on
                           MXFP8 operands quantised along each expert's rows
                           (its row count padded to a multiple of 128 with
                           zero rows).  Ignored by every other call. */
} moe_shape;

/* Bytes of scratch memory `op` (MOE_OP_*) needs for `shape`.  Host-only, no
 * GPU work.  Returns MOE_ERR_INVALID_ARG for a bad shape or op. */
int moe_workspace_size(const moe_shape* shape, int op, size_t* bytes);

/* Router scoring and top-k gating (Primus blog, MegaMoE section: a router
 * gives every token a score per expert and keeps the k best; sigmoid scores with a
 * selection bias and a group limit are DeepSeek-V3's router).
 *
 *  x [T, d] dtype, w_router [E, d] dtype, router_bias [E] fp32 or NULL:
 *      logits[t, e] = x[t] . w_router[e] + router_bias[e], fp32 accumulate.
 *      If x and w_router are both NULL, `logits` is an INPUT instead.
 *  logits [T, E] fp32 (output, or input as above).
 *  score_bias [E] fp32 or NULL: SIGMOID only, added to the scores for
 *      selection, never to the gates.
 *  topk_idx [T, k] int32 out: chosen experts in descending key order, ties to
 *      the lower expert index.  SOFTMAX keys are the logits.  SIGMOID: s =
 *      fp32(1 / (1 + exp(-l))) evaluated in fp64, key = fp32(s + bias);
 *      groups are n_groups contiguous blocks scored by the fp32 sum of their
 *      two largest keys (the key itself for one-expert groups) and only the
 *      topk_groups best (ties to the lower group) are searched.
 *  topk_w [T, k] fp32 out: SOFTMAX renorm=1: softmax over the k selected
 *      logits; renorm=0: full softmax probability.  SIGMOID: s / sum of the k
 *      picked s (renorm=1) or s.
 *  ws: MOE_OP_ROUTE bytes when the logits are computed here (the bf16
 *      router GEMM splits its contraction when its output tiles are few and
 *      keeps fp32 partial sums there, added in a fixed order); may be NULL
 *      when that size is 0 or when logits are an input. */
int moe_route_topk(const moe_shape* shape, const void* x, const void* w_router,
                   const float* router_bias, float* logits,
                   const float* score_bias, int32_t* topk_idx, float* topk_w,
                   void* ws, size_t ws_bytes, void* stream);

/* Padding-free permutation into expert-contiguous order (Primus blog,
 * MegaMoE section: tokens are reordered so that each expert's rows are
 * contiguous):
 * expert histogram, exclusive prefix scan, stable scatter.
 *
 *  x [T, d] dtype; topk_idx [T, k] int32 with k distinct experts per token in
 *      [0, E); topk_w [T, k] fp32.
 *  expert_offsets [E+1] int32 out: offsets[e] = sum of counts of experts < e;
 *      offsets[E] = R.
 *  row_token [R] int32 out: source token of each permuted row; rows of one
 *      expert are in ascending token order.
 *  token_row [T, k] int32 out: inverse map, row of (t, j).
 *  row_gate [R] fp32 out: topk_w of each row.
 *  x_perm [R, d] dtype out: x_perm[token_row[t, j]] = x[t], bit-exact copy;
 *      or NULL: only the maps are produced (x is then not read and may be
 *      NULL), for a moe_grouped_ffn call that gathers its rows from x.
 *  Entries of topk_idx outside [0, E) are skipped (token_row = -1); repeated
 *  experts within a token give unspecified (memory-safe) maps.
 *  ws: MOE_OP_PERMUTE bytes. */
int moe_permute(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                const float* topk_w, int32_t* expert_offsets,
                int32_t* row_token, int32_t* token_row, float* row_gate,
                void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_permute without a workspace, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, outputs and results as moe_permute, bit for
 * bit; its scratch (per-(expert, block of 256 tokens) counts and first rows)
 * lives in a fixed 2 MiB device array of the library instead, which each GPU
 * the library runs on holds until the process ends.  Limit:
 * E * ceil(T / 256) <= 262144 (e.g. T <= 65536 at E = 1024); larger shapes
 * return MOE_ERR_WORKSPACE before any launch.  Calls on one GPU share that
 * array: calls that overlap on one GPU (concurrent streams, threads) race and
 * give undefined maps.  Allocates nothing (no hipMalloc, no hipFree). */
int moe_permute_noalloc(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                        const float* topk_w, int32_t* expert_offsets,
                        int32_t* row_token, int32_t* token_row, float* row_gate,
                        void* x_perm, void* stream);

/* Grouped SwiGLU expert FFN over ragged, expert-contiguous row ranges, in one
 * launch per GEMM (Primus blog, MegaMoE section: FC1 (gate/up) -> SwiGLU ->
 * FC2 (down)), plus the shared expert over all T tokens when F_shared > 0
 * (the blog's layer combines such a shared expert with the routed ones).
 *
 *  x_perm [R, d] dtype, or NULL: then FC1 reads routed row r straight from
 *      x[row_token[r]] (the permutation fused into FC1's operand load; x and
 *      row_token [R] int32 are required, and T * d * sizeof(dtype) must stay
 *      below 2^31, else MOE_ERR_UNSUPPORTED).  row_token is ignored when
 *      x_perm is given.
 *  expert_offsets [E+1] int32 (as from moe_permute; read on the device only).
 *  w_gate, w_up [E, F, d]; w_down [E, d, F] dtype.
 *  x [T, d], ws_gate, ws_up [Fs, d], ws_down [d, Fs] dtype: x is read for the
 *      gathered rows above or the shared expert, the weights only when
 *      F_shared > 0 (may be NULL otherwise).
 *  y_perm [R, d] dtype out: rows of expert e = (silu(g) * u) . w_down[e]^T,
 *      with h = silu(g) * u rounded to dtype before FC2.
 *  y_shared [T, d] dtype out (F_shared > 0, else ignored).
 *  gu_save [R, 2F] dtype out or NULL: g in columns [0, F), u in [F, 2F),
 *      rounded to dtype; needed by moe_ffn_backward.  With F_shared > 0 the
 *      buffer continues with the shared expert's [T, 2F_shared] (g | u of
 *      every token), so it holds R * 2F + T * 2F_shared elements.
 *  ws: MOE_OP_FFN bytes (holds h). */
int moe_grouped_ffn(const moe_shape* shape, const void* x_perm,
                    const int32_t* row_token, const int32_t* expert_offsets,
                    const void* w_gate, const void* w_up, const void* w_down,
                    const void* x,
                    const void* ws_gate, const void* ws_up,
                    const void* ws_down, void* y_perm, void* y_shared,
                    void* gu_save, void* ws, size_t ws_bytes, void* stream);

/* The grouped SwiGLU FFN with the unpermute-and-scale folded into FC2's
 * epilogue (Primus blog, MegaMoE section: combine fused into the second
 * grouped GEMM, so the expert outputs are never materialised):
 *      y[t] = ys[t] + sum_j topk_w[t, j] * (h_r . w_down[e]^T),  r = token_row[t, j]
 * with h rounded to dtype as in moe_grouped_ffn, but each expert output
 * kept in fp32 (it is never stored), scaled by its gate and added into y.
 *
 *  x_perm [R, d] dtype, or NULL: FC1 gathers row r from x[row_token[r]]
 *      (then x is required and T * d * sizeof(dtype) < 2^31, else
 *      MOE_ERR_UNSUPPORTED).
 *  row_token [R], row_gate [R] fp32 (as from moe_permute): routed row r adds
 *      row_gate[r] times its FC2 output into y[row_token[r]].
 *  expert_offsets, w_gate, w_up, w_down, x, ws_gate, ws_up, ws_down as in
 *      moe_grouped_ffn; the shared expert (F_shared > 0) adds its output
 *      with gate 1.
 *  y [T, d] fp32 out: overwritten (zeroed, then accumulated).
 * The additions into y are fp32 atomics, so their order varies between
 * runs: the result is bitwise reproducible when every element receives at
 * most two additions (k = 1 or 2, no shared expert and no split of FC2's
 * contraction: 0 + a + b commutes exactly); otherwise runs may differ in the
 * last bits (each order's rounding error is bounded by n * 2^-24 * sum |terms|
 * for n terms).  Forward only: neither g | u nor the expert outputs that
 * moe_ffn_backward reads are produced.
 *  ws: MOE_OP_FFN_COMBINE bytes (holds h). */
int moe_grouped_ffn_combine(const moe_shape* shape, const void* x_perm,
                            const int32_t* row_token, const float* row_gate,
                            const int32_t* expert_offsets,
                            const void* w_gate, const void* w_up, const void* w_down,
                            const void* x, const void* ws_gate, const void* ws_up,
                            const void* ws_down, float* y, void* ws, size_t ws_bytes,
                            void* stream);

/* Unpermute-and-scale (Primus blog, MegaMoE section: the last stage sums each
 * token's k gate-weighted expert outputs back into its row):
 *      y[t] = y_shared[t] + sum_{j=0..k-1} topk_w[t, j] * y_perm[token_row[t, j]]
 * accumulated in fp32 in that order, as a per-token gather (no atomics).
 *  y_perm [R, d] dtype; token_row [T, k]; topk_w [T, k] fp32;
 *  y_shared [T, d] dtype or NULL; y [T, d] fp32 out.
 *  Entries with token_row < 0 contribute nothing.
 *  ws: MOE_OP_COMBINE bytes (may be NULL when that is 0). */
int moe_unpermute_combine(const moe_shape* shape, const void* y_perm,
                          const int32_t* token_row, const float* topk_w,
                          const void* y_shared, float* y, void* ws,
                          size_t ws_bytes, void* stream);

/* Backward of the layer (Primus blog, MegaMoE section: the backward
 * mirrors the forward through dispatch/combine duality, with the FC2 and FC1
 * data gradients and weight-gradient GEMMs over each expert's rows).  From the
 * upstream gradient dy of y it produces:
 *   dY_perm[token_row[t,j]] = rnd(w[t,j] dy[t]);  d_gate[t,j] = <dy[t], y_perm[row]>
 *   dh = dY_perm . w_down[e];  dg = rnd(dh u silu'(g));  du = rnd(dh silu(g))
 *   dw_down[e] = dY_perm^T . h,  h = rnd(silu(g) u) from the saved g, u
 *   dw_gate[e] = dg^T . x_perm,  dw_up[e] = du^T . x_perm
 *   dX_perm = rnd(dg . w_gate[e] + du . w_up[e]);  dx[t] = sum_j dX_perm[row]
 *   d_logits: d_gate through the gate function (zero for unpicked experts)
 * where rnd rounds to dtype.  The router's own linear map (dx through the
 * logits, d w_router) is left to the caller.
 *
 *  dy [T, d] dtype; x_perm, y_perm [R, d]; gu_save [R, 2F] dtype;
 *  expert_offsets [E+1], row_token [R], token_row [T, k], topk_idx [T, k]
 *  int32; topk_w [T, k], logits [T, E] fp32; w_gate, w_up, w_down as in
 *  moe_grouped_ffn.
 *  Outputs: dx [T, d], d_gate [T, k], d_logits [T, E] fp32; dw_gate, dw_up
 *  [E, F, d] and dw_down [E, d, F] (exactly zero for experts with no rows)
 *  stored as shape.wgrad_dtype: fp32, or bf16 rounded once from the fp32
 *  accumulator (the Primus blog's precision-aware optimizer keeps main
 *  gradients in BF16; this halves the weight-gradient writes).
 *
 *  With F_shared > 0 the shared expert (gate 1 on every token, beside the
 *  routed experts as in the Primus blog's layer) gets the same backward over all
 *  T tokens with dY = dy, from its g | u saved at the end of gu_save:
 *    dws_down = dy^T . hs;  dws_gate = dgs^T . x;  dws_up = dus^T . x
 *    dx[t] += rnd(dgs . ws_gate + dus . ws_up)[t], added after the routed terms.
 *  x [T, d], ws_gate, ws_up [F_shared, d], ws_down [d, F_shared] dtype and
 *  dws_gate, dws_up [F_shared, d], dws_down [d, F_shared] out (as
 *  shape.wgrad_dtype; zero when T = 0) are only
 *  touched when F_shared > 0 (may be NULL otherwise); gu_save then holds
 *  R * 2F + T * 2F_shared elements, as moe_grouped_ffn writes it.
 *
 *  Selective rematerialisation: with gu_save NULL the call first runs FC1
 *  again on x_perm (and x for the shared expert), with the same kernels and
 *  schedule as moe_grouped_ffn, into its workspace, and then proceeds as
 *  above.  The results are bitwise those of the call given the saved g | u;
 *  the forward then need not keep g | u (R * 2F + T * 2F_shared elements)
 *  alive until the backward.
 *  ws: MOE_OP_BACKWARD bytes, or MOE_OP_BACKWARD_RECOMPUTE bytes when
 *  gu_save is NULL. */
int moe_ffn_backward(const moe_shape* shape, const void* dy, const void* x_perm,
                     const void* gu_save, const void* y_perm,
                     const int32_t* expert_offsets, const int32_t* row_token,
                     const int32_t* token_row, const int32_t* topk_idx,
                     const float* topk_w, const float* logits,
                     const void* w_gate, const void* w_up, const void* w_down,
                     const void* x, const void* ws_gate, const void* ws_up,
                     const void* ws_down, float* dx, void* dw_gate, void* dw_up,
                     void* dw_down, void* dws_gate, void* dws_up, void* dws_down,
                     float* d_gate, float* d_logits, void* ws, size_t ws_bytes,
                     void* stream);

/* MXFP8 block quantisation (Primus blog, low-precision section: MXFP8
 * expert GEMMs on gfx950 with the OCP E4M3 element format, one E8M0
 * power-of-two scale per block of 32 values).  Each row of the bf16 matrix
 * src [rows, cols] (cols a multiple of 32) is cut into blocks of 32
 * consecutive values; block b with largest magnitude amax gets the scale
 * 2^s, s = floor(log2 amax) - 8 (8 being the exponent of E4M3's largest
 * power of two), clipped to [-127, 127], and s = -127 when amax is 0; its
 * values become the E4M3 codes nearest v / 2^s (ties to even, saturating at
 * +-448).
 *  q [rows, cols] uint8 out: E4M3 codes (1 sign, 4 exponent bits with bias
 *      7, 3 mantissa bits; 0x7f/0xff never written).
 *  scales [rows, cols / 32] uint8 out: the E8M0 byte s + 127.
 * Used for the activations each step and once for the weights, whose codes
 * the caller keeps (quantised-weight caching).  rows >= 0; NaN/Inf inputs
 * give unspecified codes.  No workspace. */
int moe_mx_quantize(const void* src, int64_t rows, int32_t cols, uint8_t* q,
                    uint8_t* scales, void* stream);

/* moe_grouped_ffn with MXFP8 operands on the scaled MFMA (Primus blog,
 * low-precision section), routed rows gathered from the quantised x.
 *  xq [T, d], xs [T, d / 32]: x quantised by moe_mx_quantize.  Routed row r
 *      reads token row_token[r] (row_token [R], expert_offsets [E+1] as from
 *      moe_permute; since quantisation is row-wise this equals quantising
 *      x_perm).
 *  w_gate_q, w_up_q [E, F, d] with scales [E, F, d / 32]; w_down_q [E, d, F]
 *      with scales [E, d, F / 32]: the weights quantised along their
 *      contraction dimension (moe_mx_quantize with cols = d, resp. F).
 *  ws_*_q, ws_*_s: the shared expert's weights likewise ([Fs, d], [d, Fs]),
 *      read only when F_shared > 0 (may be NULL otherwise).
 *  y_perm [R, d] bf16 out: per expert, g = xq . w_gate^T and u = xq . w_up^T
 *      on the dequantised values with fp32 accumulation; h = silu(g) * u is
 *      quantised to MXFP8 along F (blocks of 32 columns, the rule above)
 *      and y = hq . w_down^T, fp32 accumulate, rounded to bf16.
 *  y_shared [T, d] bf16 out (F_shared > 0, else ignored): the same for the
 *      shared expert over all T tokens.
 * shape.dtype must be MOE_DTYPE_BF16.  d, F and F_shared must be multiples
 * of 128 (else MOE_ERR_UNSUPPORTED).  Forward only: no g | u is saved.
 *  ws: MOE_OP_FFN_MXFP8 bytes (holds the quantised h). */
int moe_grouped_ffn_mxfp8(const moe_shape* shape, const uint8_t* xq,
                          const uint8_t* xs, const int32_t* row_token,
                          const int32_t* expert_offsets,
                          const uint8_t* w_gate_q, const uint8_t* w_gate_s,
                          const uint8_t* w_up_q, const uint8_t* w_up_s,
                          const uint8_t* w_down_q, const uint8_t* w_down_s,
                          const uint8_t* ws_gate_q, const uint8_t* ws_gate_s,
                          const uint8_t* ws_up_q, const uint8_t* ws_up_s,
                          const uint8_t* ws_down_q, const uint8_t* ws_down_s,
                          void* y_perm, void* y_shared, void* ws,
                          size_t ws_bytes, void* stream);

/* The MXFP8 grouped FFN with the unpermute-and-scale folded into FC2's
 * epilogue (Primus blog, MegaMoE section: combine fused into the second
 * grouped GEMM): moe_grouped_ffn_mxfp8's FC1, then FC2's fp32 rows (never
 * stored, so not rounded to bf16), scaled by row_gate[r] (1 for the shared
 * expert), added into y[row_token[r]] (resp. y[t]) with fp32 atomics.
 *  Arguments as moe_grouped_ffn_mxfp8, with row_gate [R] fp32 (moe_permute)
 *  in place of y_perm / y_shared, and y [T, d] fp32 out (overwritten).
 * No split of the contraction here, so each element of y receives k
 * additions (k + 1 with a shared expert): bitwise reproducible when that is
 * at most two, else as described at moe_grouped_ffn_combine.
 *  ws: MOE_OP_FFN_MXFP8 bytes. */
int moe_grouped_ffn_mxfp8_combine(const moe_shape* shape, const uint8_t* xq,
                                  const uint8_t* xs, const int32_t* row_token,
                                  const float* row_gate, const int32_t* expert_offsets,
                                  const uint8_t* w_gate_q, const uint8_t* w_gate_s,
                                  const uint8_t* w_up_q, const uint8_t* w_up_s,
                                  const uint8_t* w_down_q, const uint8_t* w_down_s,
                                  const uint8_t* ws_gate_q, const uint8_t* ws_gate_s,
                                  const uint8_t* ws_up_q, const uint8_t* ws_up_s,
                                  const uint8_t* ws_down_q, const uint8_t* ws_down_s,
                                  float* y, void* ws, size_t ws_bytes, void* stream);

/* MXFP8 quantisation along the ROWS of each of `batches` row-major
 * [rows, cols] bf16 matrices, written transposed (Primus blog, low-precision
 * section: MXFP8 block scaling, applied to the backward's GEMMs, which read
 * the weights against their storage order): element (r, c) of batch b is
 * quantised with rows 32 (r / 32) .. + 31 of its column, by the rule of
 * moe_mx_quantize, and written as code q[(b * cols + c) * ldq + r] with
 * scale byte scales[(b * cols + c) * (ldq / 32) + r / 32].  With ldq > rows
 * several matrices can share one output row (the backward's [w_gate; w_up]
 * concatenation along F: w_gate into q, w_up into q + F, scales + F / 32).
 *  rows % 32 == 0, ldq % 32 == 0, ldq >= rows, batches <= 65535; q 8-byte
 *  aligned, src 16-byte aligned; else MOE_ERR_INVALID_ARG. */
int moe_mx_quantize_t(const void* src, int64_t batches, int32_t rows, int32_t cols,
                      int32_t ldq, uint8_t* q, uint8_t* scales, void* stream);

/* The layer's backward with its two data-gradient GEMMs on MXFP8 operands
 * (Primus blog, low-precision section: the grouped expert GEMMs of the
 * backward in MXFP8), each quantised along its contraction dimension:
 *   dh      = dY_perm_q . w_down_q   (dY_perm and w_down along d)
 *   dX_perm = [dg | du]_q . [w_gate; w_up]_q   (along F)
 * dY_perm is quantised inside the call; dg | du are quantised in dh's
 * epilogue after rounding to bf16.  Everything else is moe_ffn_backward's:
 * the dispatch gradient, d_gate and d_logits, the SwiGLU backward (dh stays
 * fp32 until dg, du and h are rounded to bf16), the weight-gradient GEMMs
 * in bf16 with fp32 accumulation (stored as shape.wgrad_dtype), and the dx
 * gather.  The shared expert (F_shared > 0) gets the same over all T tokens,
 * with dy quantised along d.
 *
 *  dy, x_perm, gu_save (required unless T = 0: no recomputation), y_perm,
 *      maps, topk_*, logits, x and every output as in moe_ffn_backward.
 *  w_down_tq [E, F, d], w_down_ts [E, F, d / 32]: w_down quantised along d
 *      (moe_mx_quantize_t with batches E, rows d, cols F, ldq d).
 *  w_gu_tq [E, d, 2F], w_gu_ts [E, d, 2F / 32]: w_gate then w_up quantised
 *      along F (moe_mx_quantize_t of each with rows F, cols d, ldq 2F; w_up
 *      at column offset F).
 *  ws_down_tq/ts [Fs, d], ws_gu_tq/ts [d, 2Fs]: the shared expert's, likewise
 *      (read only when F_shared > 0).
 * shape.dtype must be MOE_DTYPE_BF16; d, F and F_shared multiples of 128
 * (else MOE_ERR_UNSUPPORTED).
 *  ws: MOE_OP_BACKWARD_MXFP8 bytes. */
int moe_ffn_backward_mxfp8(const moe_shape* shape, const void* dy, const void* x_perm,
                           const void* gu_save, const void* y_perm,
                           const int32_t* expert_offsets, const int32_t* row_token,
                           const int32_t* token_row, const int32_t* topk_idx,
                           const float* topk_w, const float* logits,
                           const uint8_t* w_down_tq, const uint8_t* w_down_ts,
                           const uint8_t* w_gu_tq, const uint8_t* w_gu_ts, const void* x,
                           const uint8_t* ws_down_tq, const uint8_t* ws_down_ts,
                           const uint8_t* ws_gu_tq, const uint8_t* ws_gu_ts, float* dx,
                           void* dw_gate, void* dw_up, void* dw_down, void* dws_gate,
                           void* dws_up, void* dws_down, float* d_gate, float* d_logits,
                           void* ws, size_t ws_bytes, void* stream);

/* Static text for a moe_status value (never NULL). */
const char* moe_status_string(int status);

/* Measurement aid: the kernels each MOE_PHASE_* names, bracketed by HIP
 * events on the call's stream, so that a caller can time one kernel inside
 * a call (the Primus blog times its MoE layer with HIP events; this reaches
 * inside moe_grouped_ffn and moe_ffn_backward).  The routed experts' kernels
 * only: the shared expert's own backward launches are not bracketed, and in
 * the forward it shares FC1's and FC2's launches. */
enum {
  MOE_PHASE_FC1 = 0,            /* FC1 + SwiGLU grouped GEMM                   */
  MOE_PHASE_FC2 = 1,            /* FC2 grouped GEMM (+ its split-K reduce)     */
  MOE_PHASE_BWD_DISPATCH = 2,   /* dY_perm, d_gate and d_logits                */
  MOE_PHASE_BWD_DH = 3,         /* dh with the SwiGLU backward                 */
  MOE_PHASE_BWD_DW_DOWN = 4,    /* dw_down = dY_perm^T . h                     */
  MOE_PHASE_BWD_DX = 5,         /* dX_perm = dg . w_gate + du . w_up           */
  MOE_PHASE_BWD_DW_GATE_UP = 6, /* dw_gate | dw_up = [dg | du]^T . x_perm      */
  MOE_PHASE_BWD_GATHER = 7,     /* dx[t] = sum_j dX_perm[row]                  */
  MOE_PHASE_COUNT = 8
};

/* Sets, for the calling thread, the events that later calls of
 * moe_grouped_ffn and moe_ffn_backward record (moe_ffn_backward_mxfp8: its
 * two weight-gradient phases): events[2 p] (a hipEvent_t)
 * just before the kernels of phase p are enqueued and events[2 p + 1] just
 * after them, for every p with 2 p + 1 < n_events and non-NULL entries.
 * The array is the caller's and must stay valid until the next call of this
 * function; n_events = 0 (or events NULL with n_events 0) switches the
 * recording off, which is the default.  Per-thread state, the library's only
 * mutable state; calls on other threads are unaffected.  Returns
 * MOE_ERR_INVALID_ARG for n_events < 0, or for events NULL with
 * n_events > 0. */
int moe_set_phase_events(void* const* events, int n_events);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
