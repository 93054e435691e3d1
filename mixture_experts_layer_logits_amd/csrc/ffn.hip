// Grouped SwiGLU expert FFN (Primus blog, MegaMoE section: FC1 (gate/up) ->
// SwiGLU -> FC2 (down), as two grouped GEMMs over ragged expert groups; the
// DeepSeek-V3 memory-model page gives the three matrices h x h_E, h x h_E,
// h_E x h).  The shared expert, applied to every token, rides along as one dense group of
// all T tokens in the same two launches.
//
//   schedule:  tile prefixes of FC1 and FC2 from the device offsets
//   FC1:       h = silu(x_perm . w_gate^T) * (x_perm . w_up^T)  -> bf16, and
//              optionally the rounded g | u for the backward
//   FC2:       y_perm = h . w_down^T                            -> bf16
//
// The combining form folds the unpermute-and-scale into FC2's epilogue (the
// blog's MegaMoE combine fused into the second grouped GEMM): each fp32 FC2
// row, scaled by its gate, is added into its token's row of the fp32 output,
// so y_perm is never written.
//
// bf16 with K and N multiples of 64 runs on MFMA; everything else (the fp32
// layer, odd widths) runs on the generic fp32-FMA tile kernel.
#include <algorithm>

#include "gemm_tiles.h"

namespace moe {

// FC1: 256 rows x (128 gate + 128 up) columns per workgroup of 8 waves
// (tail tiles: 128 rows x (256 + 256)).
constexpr int FC1_BM = 256, FC1_BN = 128;
// FC2: 256 rows x 256 columns (tail tiles: 128 x 512).
constexpr int FC2_BM = 256, FC2_BN = 256;
constexpr int GEN_BM = 64, GEN_BN = 64;

bool ffn_uses_mfma(const moe_shape& s);

// Split-K for FC2 when its tiles are too few to fill the GPU for several
// rounds (few experts with long K = F): a pure function of the shape, so
// results do not depend on the device.  At most 4 slices.
int ffn_fc2_ksplit(const moe_shape& s) {
  if (!ffn_uses_mfma(s) || s.F_shared > 0) return 1;
  const long long R = (long long)s.T * s.k;
  const long long tiles = (cdiv((int)R, FC2_BM) + s.E) * (long long)cdiv(s.d, FC2_BN);
  for (int ks = 1; ks <= 4; ++ks) {
    if (s.F % (ks * 32) != 0) continue;
    if (tiles * ks >= 4 * 256 || ks == 4) return ks;
  }
  return 1;
}

// Sums the split-K partial slices in slice order and rounds to bf16.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, long long stride, int ks, long long n4,
                     bf16_t* __restrict__ out) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    float4 acc = reinterpret_cast<const float4*>(part)[i];
    for (int sl = 1; sl < ks; ++sl) {
      const float4 v = reinterpret_cast<const float4*>(part + sl * stride)[i];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    reinterpret_cast<uint2*>(out)[i] = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

// y = 0 before the combining FC2 adds into it (a kernel, not a memset, so
// that a captured graph replays it faithfully).
__global__ void __launch_bounds__(256)
zero_f32_kernel(float* __restrict__ p, long long n) {
  const long long n4 = n / 4;
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n4; i += (long long)gridDim.x * 256)
    reinterpret_cast<float4*>(p)[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (long long i = n4 * 4 + blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    p[i] = 0.0f;
}

hipError_t launch_zero_f32(float* y, long long n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  zero_f32_kernel<<<(int)std::min<long long>((n / 4 + 255) / 256 + 1, 4096), 256, 0, st>>>(y, n);
  return hipGetLastError();
}

bool ffn_uses_mfma(const moe_shape& s) {
  return s.dtype == MOE_DTYPE_BF16 && s.d % 64 == 0 && s.F % 64 == 0 &&
         (s.F_shared == 0 || s.F_shared % 64 == 0);
}

template <typename T, int EPI2>
static hipError_t run_generic(const moe_shape& s, GemmArgs& a1, GemmArgs& a2, int R,
                              const FfnWs& ws, hipStream_t st) {
  if (s.E > 0) {
    schedule_tiles_kernel<<<1, 1024, 0, st>>>(a1.offsets, s.E, GEN_BM, cdiv(s.F, GEN_BN),
                                              ws.tiles1, GEN_BM, cdiv(s.d, GEN_BN), ws.tiles2, 0);
  }
  phase_mark(MOE_PHASE_FC1, 0, st);
  int g1 = grid_upper_bound(a1, GEN_BM, GEN_BN, R);
  if (g1 > 0) gemm_generic_kernel<T, 2, EPI_SWIGLU><<<g1, 256, 0, st>>>(a1);
  phase_mark(MOE_PHASE_FC1, 1, st);
  phase_mark(MOE_PHASE_FC2, 0, st);
  int g2 = grid_upper_bound(a2, GEN_BM, GEN_BN, R);
  if (g2 > 0) gemm_generic_kernel<T, 1, EPI2><<<g2, 256, 0, st>>>(a2);
  phase_mark(MOE_PHASE_FC2, 1, st);
  return hipGetLastError();
}

// FC1's arguments (routed groups, and the shared expert as the dense group).
static GemmArgs fc1_args(const moe_shape& s, const void* x_perm, const int32_t* row_token,
                         const int32_t* offsets, const void* w_gate, const void* w_up,
                         const void* x, const void* ws_gate, const void* ws_up, void* h,
                         void* h_shared, void* gu_save, int32_t* tiles) {
  const int R = s.T * s.k;
  const bool shared = s.F_shared > 0 && s.T > 0;
  // FC1: x_perm [R, d] x w_gate/w_up [E, F, d] -> h [R, F]
  GemmArgs a1 = {};
  a1.E = R > 0 ? s.E : 0;
  a1.offsets = offsets;
  a1.tiles = tiles;
  // without x_perm, FC1 gathers each routed row from x[row_token[r]]
  a1.A = x_perm ? x_perm : x;
  a1.gather = x_perm ? nullptr : row_token;
  a1.lda = s.d;
  a1.B0 = w_gate;
  a1.B1 = w_up;
  a1.strideB = (long long)s.F * s.d;
  a1.N = s.F;
  a1.K = s.d;
  a1.C = h;
  a1.ldc = s.F;
  a1.GU = gu_save;
  a1.ldgu = 2LL * s.F;
  if (shared) {
    a1.Td = s.T;
    a1.Ad = x;
    a1.ldad = s.d;
    a1.Bd0 = ws_gate;
    a1.Bd1 = ws_up;
    a1.Nd = s.F_shared;
    a1.Kd = s.d;
    a1.Cd = h_shared;
    a1.ldcd = s.F_shared;
    if (gu_save) {   // the shared expert's g | u follow the routed rows
      a1.GUd = static_cast<char*>(gu_save) +
               (size_t)R * 2 * s.F * (s.dtype == MOE_DTYPE_BF16 ? 2 : 4);
      a1.ldgud = 2LL * s.F_shared;
    }
  }
  return a1;
}

// FC2's arguments: h [R, F] x w_down [E, d, F] -> y_perm [R, d], and the
// shared expert's h_shared [T, Fs] x ws_down [d, Fs] -> y_shared [T, d].
static GemmArgs fc2_args(const moe_shape& s, int E, const int32_t* offsets, const void* w_down,
                         const void* ws_down, void* y_perm, void* y_shared, const FfnWs& ws) {
  GemmArgs a2 = {};
  a2.E = E;
  a2.offsets = offsets;
  a2.tiles = ws.tiles2;
  a2.A = ws.h;
  a2.lda = s.F;
  a2.B0 = w_down;
  a2.B1 = nullptr;
  a2.strideB = (long long)s.d * s.F;
  a2.N = s.d;
  a2.K = s.F;
  a2.C = y_perm;
  a2.ldc = s.d;
  if (s.F_shared > 0 && s.T > 0) {
    a2.Td = s.T;
    a2.Ad = ws.h_shared;
    a2.ldad = s.F_shared;
    a2.Bd0 = ws_down;
    a2.Bd1 = nullptr;
    a2.Nd = s.d;
    a2.Kd = s.F_shared;
    a2.Cd = y_shared;
    a2.ldcd = s.d;
  }
  return a2;
}

static hipError_t launch_fc1(const moe_shape& s, GemmArgs& a1, int R, hipStream_t st) {
  if (!ffn_uses_mfma(s)) {
    const int g1 = grid_upper_bound(a1, GEN_BM, GEN_BN, R);
    if (g1 == 0) return hipSuccess;
    if (s.dtype == MOE_DTYPE_BF16)
      gemm_generic_kernel<bf16_t, 2, EPI_SWIGLU><<<g1, 256, 0, st>>>(a1);
    else
      gemm_generic_kernel<float, 2, EPI_SWIGLU><<<g1, 256, 0, st>>>(a1);
    return hipGetLastError();
  }
  a1.tail = 1;
  return launch_mfma_gemm<FC1_BM, FC1_BN, 2, EPI_SWIGLU, 4, 2, 1>(a1, R, st);
}

hipError_t launch_fc1_recompute(const moe_shape& s, const void* x_perm, const int32_t* offsets,
                                const void* w_gate, const void* w_up, const void* x,
                                const void* ws_gate, const void* ws_up, void* gu_out,
                                void* h_scratch, void* hs_scratch, int32_t* tiles,
                                hipStream_t st) {
  const int R = s.T * s.k;
  GemmArgs a1 = fc1_args(s, x_perm, nullptr, offsets, w_gate, w_up, x, ws_gate, ws_up,
                         h_scratch, hs_scratch, gu_out, tiles);
  if (a1.E == 0 && a1.Td == 0) return hipSuccess;
  if (a1.E > 0) {
    const bool mfma = ffn_uses_mfma(s);
    const int bm = mfma ? FC1_BM : GEN_BM;   // (the second prefix is not written)
    schedule_tiles_kernel<<<1, 1024, 0, st>>>(offsets, s.E, bm, cdiv(s.F, mfma ? FC1_BN : GEN_BN),
                                              tiles, bm, 1, nullptr, mfma ? 1 : 0);
  }
  return launch_fc1(s, a1, R, st);
}

hipError_t launch_grouped_ffn(const moe_shape& s, const void* x_perm, const int32_t* row_token,
                              const int32_t* offsets,
                              const void* w_gate, const void* w_up, const void* w_down,
                              const void* x, const void* ws_gate, const void* ws_up,
                              const void* ws_down, void* y_perm, void* y_shared,
                              void* gu_save, const FfnWs& ws, hipStream_t st) {
  const int R = s.T * s.k;
  const bool shared = s.F_shared > 0 && s.T > 0;
  GemmArgs a1 = fc1_args(s, x_perm, row_token, offsets, w_gate, w_up, x, ws_gate, ws_up, ws.h,
                         ws.h_shared, gu_save, ws.tiles1);
  GemmArgs a2 = fc2_args(s, a1.E, offsets, w_down, ws_down, y_perm, y_shared, ws);
  if (a1.E == 0 && !shared) return hipSuccess;

  if (!ffn_uses_mfma(s)) {
    if (s.dtype == MOE_DTYPE_BF16) return run_generic<bf16_t, EPI_STORE>(s, a1, a2, R, ws, st);
    return run_generic<float, EPI_STORE>(s, a1, a2, R, ws, st);
  }
  if (a1.E > 0) {
    schedule_tiles_kernel<<<1, 1024, 0, st>>>(offsets, s.E, FC1_BM, cdiv(s.F, FC1_BN),
                                              ws.tiles1, FC2_BM, cdiv(s.d, FC2_BN), ws.tiles2, 1);
  }
  a1.tail = a2.tail = 1;
  phase_mark(MOE_PHASE_FC1, 0, st);
  hipError_t e = launch_mfma_gemm<FC1_BM, FC1_BN, 2, EPI_SWIGLU, 4, 2, 1>(a1, R, st);
  phase_mark(MOE_PHASE_FC1, 1, st);
  if (e != hipSuccess) return e;
  const int ks = ffn_fc2_ksplit(s);
  if (ks > 1 && a2.E > 0) {
    a2.ksplit = ks;
    a2.Cpart = ws.part;
    a2.part_stride = (long long)R * s.d;
  }
  phase_mark(MOE_PHASE_FC2, 0, st);
  e = launch_mfma_gemm<FC2_BM, FC2_BN, 1, EPI_STORE, 4, 2, 1>(a2, R, st);
  if (e == hipSuccess && a2.ksplit > 1) {
    const long long n4 = (long long)R * s.d / 4;
    const int grid = (int)std::min<long long>((n4 + 255) / 256, 4096);
    splitk_reduce_kernel<<<grid, 256, 0, st>>>(ws.part, a2.part_stride, ks, n4,
                                               static_cast<bf16_t*>(y_perm));
    e = hipGetLastError();
  }
  phase_mark(MOE_PHASE_FC2, 1, st);
  return e;
}

// The FFN with the combine in FC2's epilogue: y = 0, then FC1 as above, then
// FC2 adding row_gate[r] * (h[r] . w_down[e]^T) into y[row_token[r]] (and
// the shared expert's rows with gate 1).  Split-K slices (same rule as the
// storing FC2) add their partial sums directly, so no partials are kept.
hipError_t launch_grouped_ffn_combine(const moe_shape& s, const void* x_perm,
                                      const int32_t* row_token, const float* row_gate,
                                      const int32_t* offsets, const void* w_gate,
                                      const void* w_up, const void* w_down, const void* x,
                                      const void* ws_gate, const void* ws_up,
                                      const void* ws_down, float* y, const FfnWs& ws,
                                      hipStream_t st) {
  const int R = s.T * s.k;
  const bool shared = s.F_shared > 0 && s.T > 0;
  const long long ny = (long long)s.T * s.d;
  if (ny == 0) return hipSuccess;
  hipError_t e0 = launch_zero_f32(y, ny, st);
  if (e0 != hipSuccess) return e0;
  GemmArgs a1 = fc1_args(s, x_perm, row_token, offsets, w_gate, w_up, x, ws_gate, ws_up, ws.h,
                         ws.h_shared, nullptr, ws.tiles1);
  GemmArgs a2 = fc2_args(s, a1.E, offsets, w_down, ws_down, nullptr, nullptr, ws);
  a2.comb_token = row_token;
  a2.comb_gate = row_gate;
  a2.Y = y;
  a2.ldy = s.d;
  if (a1.E == 0 && !shared) return hipGetLastError();

  if (!ffn_uses_mfma(s)) {
    if (s.dtype == MOE_DTYPE_BF16) return run_generic<bf16_t, EPI_COMBINE>(s, a1, a2, R, ws, st);
    return run_generic<float, EPI_COMBINE>(s, a1, a2, R, ws, st);
  }
  if (a1.E > 0) {
    schedule_tiles_kernel<<<1, 1024, 0, st>>>(offsets, s.E, FC1_BM, cdiv(s.F, FC1_BN),
                                              ws.tiles1, FC2_BM, cdiv(s.d, FC2_BN), ws.tiles2, 1);
  }
  a1.tail = a2.tail = 1;
  hipError_t e = launch_mfma_gemm<FC1_BM, FC1_BN, 2, EPI_SWIGLU, 4, 2, 1>(a1, R, st);
  if (e != hipSuccess) return e;
  const int ks = ffn_fc2_ksplit(s);
  if (ks > 1 && a2.E > 0) a2.ksplit = ks;
  return launch_mfma_gemm<FC2_BM, FC2_BN, 1, EPI_COMBINE, 4, 2, 1>(a2, R, st);
}

}  // namespace moe
