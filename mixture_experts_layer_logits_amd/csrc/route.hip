// Router scoring and top-k gating.
//
// Router logits are one dense GEMM (x . w_router^T, fp32 accumulate, plus an
// optional per-expert router bias).  Top-k runs one wavefront per token: each
// lane holds the keys of experts lane, lane + 64, ...; k passes of a 64-lane
// arg-max reduction pick the largest remaining key, the lower expert index
// winning ties.  Sigmoid scoring first keeps the topk_groups best groups of
// contiguous experts (group score: fp32 sum of the group's two largest keys),
// then searches only those.  (Primus blog, MegaMoE section: a router scores
// every token against each expert and keeps the k best; the sigmoid scores
// with a per-expert selection bias and group limit follow DeepSeek-V3, whose
// bias-based load balancing the Piper podcast page refers to.)
#include <float.h>
#include <limits.h>

#include <algorithm>

#include "gemm_tiles.h"

namespace moe {

// The router GEMM is as long in K (d) as the expert GEMMs but has few
// output tiles.  With up to 128 experts it runs 64 x 64 tiles (64 of them at
// T = 4096, E = 8), whose K loops are latency-bound with only three slices
// in flight, so it is split in K until there are 512 work items (2 per CU).
// With more experts, 64-wide tiles would re-read x once per 64 experts (4
// times at E = 256), so it runs 256 x 256 tiles split in K up to 8 ways
// towards one item per CU.  Each slice is at least one 32-wide K step.  The
// split is a pure function of the shape, so results do not depend on the
// device; slices write fp32 partial sums that a second kernel adds in slice
// order (then the bias): deterministic.  Measured per router GEMM (+ the
// partial-sum pass): T = 4096, E = 8: 47 -> 19 us; T = 8192, E = 256, d =
// 7168: 99 -> 73 us; T = 16384, E = 128, d = 2048 (512 tiles): unsplit, 35 us.
static bool router_big_tiles(const moe_shape& s) { return s.E > 128; }

int router_ksplit(const moe_shape& s) {
  if (!(s.dtype == MOE_DTYPE_BF16 && s.d % 64 == 0) || s.T == 0) return 1;
  const bool big = router_big_tiles(s);
  const int bm = big ? 256 : 64, bn = big ? 256 : 64;
  const long long tiles = (long long)cdiv(s.T, bm) * cdiv(s.E, bn);
  const long long want = big ? 256 : 512;
  const int most = big ? 8 : 16;
  int ks = 1;
  while (ks < most && tiles * ks < want && s.d % (2 * ks * 32) == 0) ks *= 2;
  return ks;
}

__global__ void __launch_bounds__(256)
router_reduce_kernel(const float* __restrict__ part, int ks, long long n, int E,
                     const float* __restrict__ bias, float* __restrict__ logits) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    float acc = part[i];
    for (int sl = 1; sl < ks; ++sl) acc += part[sl * n + i];
    logits[i] = acc + (bias ? bias[i % E] : 0.0f);
  }
}

hipError_t launch_router_logits(const moe_shape& s, const void* x, const void* w_router,
                                const float* router_bias, float* logits, float* part,
                                hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  GemmArgs a = {};
  a.E = 0;
  a.Td = s.T;
  a.Ad = x;
  a.ldad = s.d;
  a.Bd0 = w_router;
  a.Bd1 = nullptr;
  a.Nd = s.E;
  a.Kd = s.d;
  a.Cd = logits;
  a.ldcd = s.E;
  a.bias = router_bias;
  if (s.dtype == MOE_DTYPE_BF16 && s.d % 64 == 0) {
    const int ks = router_ksplit(s);
    if (ks > 1) {
      a.ksplit = ks;
      a.Cpart = part;
      a.part_stride = (long long)s.T * s.E;
    }
    hipError_t e = router_big_tiles(s)
                       ? launch_mfma_gemm<256, 256, 1, EPI_F32_BIAS, 4, 2, 0>(a, 0, st)
                       : launch_mfma_gemm<64, 64, 1, EPI_F32_BIAS, 2, 2, 0>(a, 0, st);
    if (e != hipSuccess || ks == 1) return e;
    const long long n = (long long)s.T * s.E;
    const int grid = (int)std::min<long long>((n + 255) / 256, 2048);
    router_reduce_kernel<<<grid, 256, 0, st>>>(part, ks, n, s.E, router_bias, logits);
    return hipGetLastError();
  } else if (s.dtype == MOE_DTYPE_BF16) {
    const int grid = grid_upper_bound(a, 64, 64, 0);
    gemm_generic_kernel<bf16_t, 1, EPI_F32_BIAS><<<grid, 256, 0, st>>>(a);
  } else {
    const int grid = grid_upper_bound(a, 64, 64, 0);
    gemm_generic_kernel<float, 1, EPI_F32_BIAS><<<grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

// Arg-max order: the larger key wins, the lower index on equal keys; lanes
// without a candidate carry idx == INT_MAX and never win.  The order is
// total, so any reduction tree finds the same winner.
__device__ __forceinline__ void argmax_take(float& v, int& i, float ov, int oi) {
  const bool take = (oi != INT_MAX) && (i == INT_MAX || ov > v || (ov == v && oi < i));
  if (take) {
    v = ov;
    i = oi;
  }
}

// One step against the lane that the DPP pattern CTRL names (every lane of a
// row has a source under the patterns used here).
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float& v, int& i) {
  const float ov =
      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
  const int oi = __builtin_amdgcn_update_dpp(0, i, CTRL, 0xf, 0xf, false);
  argmax_take(v, i, ov, oi);
}

// Wave-wide arg-max, the result in every lane.  Within each 16-lane row the
// pairs move by DPP (lane ^ 1 and lane ^ 2 by quad permutes, then rotations
// of the row by 4 and 8), so every lane ends with its row's winner; the four
// row winners are then read as wave-uniform values.  No LDS traffic, unlike
// a shuffle through ds_bpermute.  Must be called with every lane active.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_dpp<0xB1>(v, i);    // quad_perm [1, 0, 3, 2]
  argmax_dpp<0x4E>(v, i);    // quad_perm [2, 3, 0, 1]
  argmax_dpp<0x124>(v, i);   // row_ror:4
  argmax_dpp<0x128>(v, i);   // row_ror:8
  float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int ri = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r)
    argmax_take(rv, ri, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r)),
                __builtin_amdgcn_readlane(i, 16 * r));
  v = rv;
  i = ri;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// One wavefront per token, 4 tokens per workgroup.  NQ = experts per lane.
template <int NQ>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ logits, const float* __restrict__ score_bias, int T,
            int E, int k, int score, int renorm, int n_groups, int topk_groups,
            int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  __shared__ float s_key[4][64 * NQ];
  __shared__ int s_keep[4][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t_raw = blockIdx.x * 4 + wave;
  const bool live = t_raw < T;
  const int t = live ? t_raw : T - 1;  // idle waves mirror the last token, store nothing

  float key[NQ], sc[NQ];
  bool avail[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int e = lane + 64 * q;
    const bool valid = e < E;
    const float l = valid ? logits[(long long)t * E + e] : 0.0f;
    if (score == MOE_SCORE_SOFTMAX) {
      sc[q] = l;
      key[q] = l;
    } else {
      const float sg = (float)(1.0 / (1.0 + exp(-(double)l)));
      sc[q] = sg;
      key[q] = score_bias ? __fadd_rn(sg, valid ? score_bias[e] : 0.0f) : sg;
    }
    avail[q] = valid;
  }

  if (n_groups > 1) {  // uniform over the launch
    const int G = E / n_groups;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      if (e < E) s_key[wave][e] = key[q];
    }
    __syncthreads();
    float gs = 0.0f;
    int gi = INT_MAX;
    if (lane < n_groups) {
      float b1 = -FLT_MAX, b2 = -FLT_MAX;
      bool have1 = false, have2 = false;
      for (int e = lane * G; e < lane * G + G; ++e) {
        const float v = s_key[wave][e];
        if (!have1 || v > b1) {
          if (have1) { b2 = b1; have2 = true; }
          b1 = v;
          have1 = true;
        } else if (!have2 || v > b2) {
          b2 = v;
          have2 = true;
        }
      }
      gs = (G >= 2) ? __fadd_rn(b1, b2) : b1;
      gi = lane;
    }
    bool kept = false;
    for (int p = 0; p < topk_groups; ++p) {
      float v = gi != INT_MAX ? gs : 0.0f;
      int i = gi;
      wave_argmax(v, i);
      if (lane == i) {
        kept = true;
        gi = INT_MAX;
      }
    }
    s_keep[wave][lane] = kept ? 1 : 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = lane + 64 * q;
      if (e < E) avail[q] = s_keep[wave][e / G] != 0;
    }
  }

  int my_e = 0;
  float my_s = 0.0f;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = INT_MAX;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (avail[q] && (bi == INT_MAX || key[q] > bv)) {
        bv = key[q];
        bi = lane + 64 * q;
      }
    }
    wave_argmax(bv, bi);
    float mine = 0.0f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (lane + 64 * q == bi) {
        avail[q] = false;
        mine = sc[q];
      }
    }
    const float win_s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), bi & 63));
    if (lane == j) {
      my_e = bi;
      my_s = win_s;
    }
  }

  float w = 0.0f;
  if (score == MOE_SCORE_SOFTMAX) {
    const float m = __shfl(my_s, 0, 64);  // the first pick holds the largest logit
    if (renorm) {
      const float z = lane < k ? expf(my_s - m) : 0.0f;
      w = z / wave_sum(z);
    } else {
      float part = 0.0f;
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (lane + 64 * q < E) part += expf(sc[q] - m);
      w = expf(my_s - m) / wave_sum(part);
    }
  } else {
    if (renorm) {
      const double tot = wave_sum_f64(lane < k ? (double)my_s : 0.0);
      w = (float)((double)my_s / tot);
    } else {
      w = my_s;
    }
  }
  if (live && lane < k) {
    topk_idx[(long long)t * k + lane] = my_e;
    topk_w[(long long)t * k + lane] = w;
  }
}

hipError_t launch_topk(const moe_shape& s, const float* logits, const float* score_bias,
                       int32_t* topk_idx, float* topk_w, hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const int grid = cdiv(s.T, 4);
  const float* sb = (s.score == MOE_SCORE_SIGMOID) ? score_bias : nullptr;
#define MOE_TOPK(NQ)                                                                    \
  topk_kernel<NQ><<<grid, 256, 0, st>>>(logits, sb, s.T, s.E, s.k, s.score, s.renorm, \
                                        s.n_groups, s.topk_groups, topk_idx, topk_w)
  if (s.E <= 64) MOE_TOPK(1);
  else if (s.E <= 128) MOE_TOPK(2);
  else if (s.E <= 256) MOE_TOPK(4);
  else if (s.E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK
  return hipGetLastError();
}

}  // namespace moe
