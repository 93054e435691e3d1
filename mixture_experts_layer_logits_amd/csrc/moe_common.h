// Internal helpers of the HIP MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// bf16 is stored as its 16 raw bits.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// fp32 -> bf16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// The fp32 value of f rounded to bf16.
__device__ __forceinline__ float bf16_round(float f) { return bf16_to_f32(f32_to_bf16(f)); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) |
         (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// silu(g) = g / (1 + exp(-g)).
__device__ __forceinline__ float silu_fast(float g) { return g / (1.0f + __expf(-g)); }
__device__ __forceinline__ float silu_precise(float g) { return g / (1.0f + expf(-g)); }

// Events the calling thread asked to have recorded around each MOE_PHASE_*
// (moe_set_phase_events): ev[2 p] before phase p's kernels, ev[2 p + 1]
// after them.
struct PhaseEvents {
  void* const* ev;
  int n;
};
extern thread_local PhaseEvents g_phase_events;

inline void phase_mark(int phase, int end, hipStream_t st) {
  const int i = 2 * phase + end;
  if (i < g_phase_events.n && g_phase_events.ev[i])
    (void)hipEventRecord(static_cast<hipEvent_t>(g_phase_events.ev[i]), st);
}

// ---------------------------------------------------------------------------
// Launchers implemented in the .hip files.  Each returns hipSuccess or the
// launch error.  Shapes were validated by the API layer.
// ---------------------------------------------------------------------------
// part: router_ksplit(s) * T * E fp32 partial sums when that is above 1.
int router_ksplit(const moe_shape& s);
hipError_t launch_router_logits(const moe_shape& s, const void* x, const void* w_router,
                                const float* router_bias, float* logits, float* part,
                                hipStream_t st);
hipError_t launch_topk(const moe_shape& s, const float* logits, const float* score_bias,
                       int32_t* topk_idx, float* topk_w, hipStream_t st);

struct PermuteWs {
  int32_t* blk_cnt;   // [E * nblk]
  int32_t* blk_base;  // [E * nblk]
};
int permute_nblk(const moe_shape& s);
// The fixed scratch of moe_permute_noalloc: at most this many (expert,
// block) entries, E * permute_nblk(s).
constexpr long long PERMUTE_NOALLOC_MAX_ENTRIES = 1LL << 18;
// Points ws at the current device's fixed scratch (looked up on first use).
hipError_t permute_noalloc_ws(PermuteWs& ws);
hipError_t launch_permute(const moe_shape& s, const void* x, const int32_t* topk_idx,
                          const float* topk_w, int32_t* offsets, int32_t* row_token,
                          int32_t* token_row, float* row_gate, void* x_perm,
                          const PermuteWs& ws, hipStream_t st);

struct FfnWs {
  int32_t* tiles1;  // [E + 1] tile prefix of FC1
  int32_t* tiles2;  // [E + 1] tile prefix of FC2
  void* h;          // [R, F] dtype
  void* h_shared;   // [T, Fs] dtype
  float* part;      // [ksplit, R, d] fp32 split-K partials of FC2
};
bool ffn_uses_mfma(const moe_shape& s);
int ffn_fc2_ksplit(const moe_shape& s);
// FC1 alone, as the forward runs it on x_perm (same kernels, same schedule):
// writes the rounded g | u (routed rows, then the shared expert's) to gu_out.
hipError_t launch_fc1_recompute(const moe_shape& s, const void* x_perm, const int32_t* offsets,
                                const void* w_gate, const void* w_up, const void* x,
                                const void* ws_gate, const void* ws_up, void* gu_out,
                                void* h_scratch, void* hs_scratch, int32_t* tiles,
                                hipStream_t st);
hipError_t launch_grouped_ffn(const moe_shape& s, const void* x_perm, const int32_t* row_token,
                              const int32_t* offsets,
                              const void* w_gate, const void* w_up, const void* w_down,
                              const void* x, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y_perm, void* y_shared,
                              void* gu_save, const FfnWs& ws, hipStream_t st);
hipError_t launch_grouped_ffn_combine(const moe_shape& s, const void* x_perm,
                                      const int32_t* row_token, const float* row_gate,
                                      const int32_t* offsets, const void* w_gate,
                                      const void* w_up, const void* w_down, const void* x,
                                      const void* ws_gate, const void* ws_up,
                                      const void* ws_down, float* y, const FfnWs& ws,
                                      hipStream_t st);

// MXFP8 (E4M3 codes with one E8M0 scale byte per 32 values along a row).
hipError_t launch_mx_quantize(const void* src, long long rows, int cols, uint8_t* q,
                              uint8_t* scales, hipStream_t st);
struct MxWeights {      // codes and scales of each weight matrix
  const uint8_t *gate_q, *gate_s, *up_q, *up_s, *down_q, *down_s;
  const uint8_t *sgate_q, *sgate_s, *sup_q, *sup_s, *sdown_q, *sdown_s;  // shared expert
};
struct MxFfnWs {
  int32_t* tiles1;  // [E + 1] tile prefix of FC1
  int32_t* tiles2;  // [E + 1] tile prefix of FC2
  uint8_t* hq;      // [R, F] E4M3 codes of h
  uint8_t* hs;      // [R, F / 32] scales of h
  uint8_t* shq;     // [T, Fs] the shared expert's h
  uint8_t* shs;     // [T, Fs / 32]
};
hipError_t launch_grouped_ffn_mxfp8(const moe_shape& s, const uint8_t* xq, const uint8_t* xs,
                                    const int32_t* row_token, const int32_t* offsets,
                                    const MxWeights& w, void* y_perm, void* y_shared,
                                    const MxFfnWs& ws, hipStream_t st,
                                    const float* row_gate = nullptr, float* y = nullptr);
// y[0 .. n) = 0 with a kernel (so that a captured graph replays it faithfully).
hipError_t launch_zero_f32(float* y, long long n, hipStream_t st);

hipError_t launch_mx_quantize_t(const void* src, long long batches, int rows, int cols, int ldq,
                                uint8_t* q, uint8_t* scales, hipStream_t st);
// The backward's MXFP8 data-gradient GEMMs over `rows` routed rows grouped
// by `offsets` (shape.E groups).
struct MxDgrad {
  int rows;
  const int32_t* offsets;
  int32_t* tiles1;               // [E + 1] tile prefix of dh
  int32_t* tiles2;               // [E + 1] tile prefix of dX
  const uint8_t *dyq, *dys;      // dY_perm quantised along d: [rows, d], [rows, d / 32]
  const uint8_t *wd_tq, *wd_ts;  // w_down quantised along d: [E, F, d], [E, F, d / 32]
  const void* gu;                // [rows, 2F] bf16, the saved g | u
  void* dgu;                     // [rows, 2F] bf16 out
  void* h;                       // [rows, F] bf16 out
  uint8_t *dguq, *dgus;          // dg | du quantised along F: [rows, 2F], [rows, 2F / 32]
  const uint8_t *wgu_tq, *wgu_ts;  // [w_gate; w_up] quantised along F: [E, d, 2F], [E, d, 2F / 32]
  void* dX;                      // [rows, d] bf16 out
};
hipError_t launch_mx_dgrad(const moe_shape& s, const MxDgrad& g, hipStream_t st);
// The weight-gradient GEMM dW[e] = A_e^T . B_e over each group's rows on
// MXFP8 operands quantised along the rows (padded per group to 128 rows):
// A [rows, M] and B [rows, N] bf16, row-grouped by `offsets` (E groups);
// output rows m < wsplit go to w0 [E][wsplit][N], the rest to w1
// [E][M - wsplit][N], fp32 or bf16 (wbf16).  poffs [E + 1] receives the
// padded offsets; qa/sa and qb/sb hold the quantised operands (wrows padded
// rows each).
struct MxWgrad {
  int E, M, N;
  const int32_t* offsets;
  int32_t* poffs;
  const void* A;
  const void* B;
  uint8_t *qa, *sa, *qb, *sb;
  long long wrows;
  void* w0;
  void* w1;
  int wsplit, wbf16;
};
hipError_t launch_mx_wgrad(const MxWgrad& g, hipStream_t st);

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* token_row,
                          const float* topk_w, const void* y_shared, float* y,
                          hipStream_t st);

struct BwdWs {
  int32_t* tiles;   // [E + 1] tile prefix of the row-tiled data-gradient GEMMs
  int32_t* tiles2;  // [E + 1] second prefix (FC1 data gradient)
  void* dY;         // [R, d]  dtype: w * dy scattered to permuted rows
  void* dgu;        // [R, 2F] dtype: dg | du
  void* h;          // [R, F]  dtype: h recomputed from the saved g, u
  void* dX;         // [R, d]  dtype
  // the shared expert (F_shared > 0): one group of all T tokens
  int32_t* s_offsets;  // [2]
  int32_t* s_tiles;    // [2]
  int32_t* s_tiles2;   // [2]
  void* s_dgu;         // [T, 2 F_shared] dtype
  void* s_h;           // [T, F_shared] dtype
  void* s_dX;          // [T, d] dtype
  // MXFP8 data gradients only: the quantised GEMM inputs
  uint8_t *dyq, *dys;       // [R, d], [R, d / 32]
  uint8_t *dguq, *dgus;     // [R, 2F], [R, 2F / 32]
  uint8_t *s_dyq, *s_dys;   // [T, d], [T, d / 32]: dy for the shared expert
  uint8_t *s_dguq, *s_dgus; // [T, 2 F_shared], [T, 2 F_shared / 32]
  // MXFP8 weight gradients (shape.wgrad_mx) only: padded row offsets of
  // the routed experts and of the shared expert's one group, and the two
  // operands of one weight-gradient GEMM quantised along the padded rows
  // ([rows of the output, wrows] codes and [.., wrows / 32] scales)
  int32_t* poffs;           // [E + 1]
  int32_t* s_poffs;         // [E + 1] (two used)
  uint8_t *wqa, *wsa;       // A operand
  uint8_t *wqb, *wsb;       // B operand
  long long wrows;          // padded rows allocated (a multiple of 128)
};
// The quantised weights the MXFP8 data gradients read.
struct MxBwdWeights {
  const uint8_t *wd_tq, *wd_ts, *wgu_tq, *wgu_ts;      // routed
  const uint8_t *swd_tq, *swd_ts, *swgu_tq, *swgu_ts;  // shared expert
};
bool backward_supported(const moe_shape& s);
hipError_t launch_backward(const moe_shape& s, const void* dy, const void* x_perm,
                           const void* gu_save, const void* y_perm, const int32_t* offsets,
                           const int32_t* row_token, const int32_t* token_row,
                           const int32_t* topk_idx, const float* topk_w,
                           const float* logits, const void* w_gate, const void* w_up,
                           const void* w_down, const void* x, const void* ws_gate,
                           const void* ws_up, const void* ws_down, float* dx, void* dw_gate,
                           void* dw_up, void* dw_down, void* dws_gate, void* dws_up,
                           void* dws_down, float* d_gate, float* d_logits,
                           const BwdWs& ws, hipStream_t st,
                           const MxBwdWeights* mx = nullptr);

}  // namespace moe
