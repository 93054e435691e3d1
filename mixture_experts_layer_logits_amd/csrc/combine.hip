// Unpermute-and-scale (Primus blog, MegaMoE section: the last stage weights
// each token's k expert outputs by its gates and sums them into its row):
//   y[t] = y_shared[t] + sum_{j=0..k-1} w[t, j] * y_perm[token_row[t, j]]
// as a per-token gather in fp32, in that fixed order.  Each token's sum is
// owned by one workgroup, so no atomics are needed and the result is bitwise
// deterministic.  HBM-bound: reads R*d + T*d (shared) elements, writes T*d
// fp32.
#include "gemm_tiles.h"

namespace moe {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One workgroup per token; each thread owns runs of 8 columns (d % 8 == 0).
// The k gathered rows are loaded in batches of JB before any of them is
// accumulated, so a thread keeps up to JB row loads in flight; the
// accumulation order stays j = 0, 1, ..., k-1.
template <typename T>
__global__ void __launch_bounds__(256)
combine_vec_kernel(const T* __restrict__ y_perm, const int32_t* __restrict__ token_row,
                   const float* __restrict__ topk_w, const T* __restrict__ y_shared, int d,
                   int k, float* __restrict__ y) {
  constexpr int JB = 8;
  const int t = blockIdx.x;
  const int32_t* rows = token_row + (long long)t * k;
  const float* w = topk_w + (long long)t * k;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8];
    if (y_shared) {
      load8<T>(y_shared + (long long)t * d + c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    for (int j0 = 0; j0 < k; j0 += JB) {
      float v[JB][8];
      float wj[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = j0 + jj;
        const int r = j < k ? rows[j] : -1;
        wj[jj] = r >= 0 ? w[j] : 0.0f;
        if (r >= 0) {
          load8<T>(y_perm + (long long)r * d + c, v[jj]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[jj][i] = 0.0f;
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (j0 + jj >= k || rows[j0 + jj] < 0) continue;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[jj], v[jj][i], acc[i]);
      }
    }
    float* dst = y + (long long)t * d + c;
    *reinterpret_cast<float4*>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

template <typename T>
__global__ void __launch_bounds__(256)
combine_scalar_kernel(const T* __restrict__ y_perm, const int32_t* __restrict__ token_row,
                      const float* __restrict__ topk_w, const T* __restrict__ y_shared, int d,
                      int k, float* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x; c < d; c += 256) {
    float acc = y_shared ? to_f32<T>(y_shared[(long long)t * d + c]) : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = token_row[(long long)t * k + j];
      if (r < 0) continue;
      acc = fmaf(topk_w[(long long)t * k + j], to_f32<T>(y_perm[(long long)r * d + c]), acc);
    }
    y[(long long)t * d + c] = acc;
  }
}

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const int32_t* token_row,
                          const float* topk_w, const void* y_shared, float* y,
                          hipStream_t st) {
  if (s.T == 0) return hipSuccess;
  const void* ys = s.F_shared > 0 ? y_shared : nullptr;
  if (s.dtype == MOE_DTYPE_BF16) {
    if (s.d % 8 == 0)
      combine_vec_kernel<bf16_t><<<s.T, 256, 0, st>>>(
          static_cast<const bf16_t*>(y_perm), token_row, topk_w,
          static_cast<const bf16_t*>(ys), s.d, s.k, y);
    else
      combine_scalar_kernel<bf16_t><<<s.T, 256, 0, st>>>(
          static_cast<const bf16_t*>(y_perm), token_row, topk_w,
          static_cast<const bf16_t*>(ys), s.d, s.k, y);
  } else {
    if (s.d % 8 == 0)
      combine_vec_kernel<float><<<s.T, 256, 0, st>>>(
          static_cast<const float*>(y_perm), token_row, topk_w,
          static_cast<const float*>(ys), s.d, s.k, y);
    else
      combine_scalar_kernel<float><<<s.T, 256, 0, st>>>(
          static_cast<const float*>(y_perm), token_row, topk_w,
          static_cast<const float*>(ys), s.d, s.k, y);
  }
  return hipGetLastError();
}

}  // namespace moe
