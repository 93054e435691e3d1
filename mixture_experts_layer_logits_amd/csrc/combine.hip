// Unpermute-and-scale (Primus blog, MegaMoE section: the last stage weights
// each token's k expert outputs by its gates and sums them into its row):
//   y[t] = y_shared[t] + sum_{j=0..k-1} w[t, j] * y_perm[token_row[t, j]]
// as a per-token gather in fp32, in that fixed order.  Each token's sum is
// owned by one workgroup, so no atomics are needed and the result is bitwise
// deterministic.  HBM-bound: reads R*d + T*d (shared) elements, writes T*d
// fp32.
#include "gemm_tiles.h"

namespace moe {

// 8 consecutive elements of a row, loaded as raw bits and converted to fp32
// separately, so that a batch of row loads can be issued before any of them
// is waited for.
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { uint4 q; };
template <> struct Raw8<float> { float4 a, b; };

template <typename T>
__device__ __forceinline__ Raw8<T> load_raw8(const T* p);
template <>
__device__ __forceinline__ Raw8<bf16_t> load_raw8<bf16_t>(const bf16_t* p) {
  return {*reinterpret_cast<const uint4*>(p)};
}
template <>
__device__ __forceinline__ Raw8<float> load_raw8<float>(const float* p) {
  return {*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
}

__device__ __forceinline__ void cvt8(const Raw8<bf16_t>& r, float (&v)[8]) {
  const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void cvt8(const Raw8<float>& r, float (&v)[8]) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
  v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}

// One workgroup per token; each thread owns runs of 8 columns (d % 8 == 0).
// The k gathered rows go in batches of JB (1, 2, 4 or 8, the largest not
// above k).  A batch is straight-line code: its JB row loads are issued
// unconditionally (a slot past k, or one without a row, reads row 0, and
// its value is not used), then converted, then accumulated in the order
// j = 0, 1, ..., k-1.  Loads under a branch, or converted where they were
// loaded, were each waited for on their own.  A token's rows are uniform
// over the workgroup.
template <typename T, int JB>
__global__ void __launch_bounds__(256)
combine_vec_kernel(const T* __restrict__ y_perm, const int32_t* __restrict__ token_row,
                   const float* __restrict__ topk_w, const T* __restrict__ y_shared, int d,
                   int k, float* __restrict__ y) {
  const int t = blockIdx.x;
  const int32_t* rows = token_row + (long long)t * k;
  const float* w = topk_w + (long long)t * k;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8];
    if (y_shared) {
      cvt8(load_raw8<T>(y_shared + (long long)t * d + c), acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    }
    for (int j0 = 0; j0 < k; j0 += JB) {
      Raw8<T> raw[JB];
      int r[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        r[jj] = j0 + jj < k ? rows[j0 + jj] : -1;
        raw[jj] = load_raw8<T>(y_perm + (long long)(r[jj] < 0 ? 0 : r[jj]) * d + c);
      }
      float v[JB][8];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) cvt8(raw[jj], v[jj]);
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (r[jj] < 0) continue;
        const float wj = w[j0 + jj];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[jj][i], acc[i]);
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
      with_gather_batch(s.k, [&](auto jb) {
        combine_vec_kernel<bf16_t, decltype(jb)::value><<<s.T, 256, 0, st>>>(
            static_cast<const bf16_t*>(y_perm), token_row, topk_w,
            static_cast<const bf16_t*>(ys), s.d, s.k, y);
      });
    else
      combine_scalar_kernel<bf16_t><<<s.T, 256, 0, st>>>(
          static_cast<const bf16_t*>(y_perm), token_row, topk_w,
          static_cast<const bf16_t*>(ys), s.d, s.k, y);
  } else {
    if (s.d % 8 == 0)
      with_gather_batch(s.k, [&](auto jb) {
        combine_vec_kernel<float, decltype(jb)::value><<<s.T, 256, 0, st>>>(
            static_cast<const float*>(y_perm), token_row, topk_w,
            static_cast<const float*>(ys), s.d, s.k, y);
      });
    else
      combine_scalar_kernel<float><<<s.T, 256, 0, st>>>(
          static_cast<const float*>(y_perm), token_row, topk_w,
          static_cast<const float*>(ys), s.d, s.k, y);
  }
  return hipGetLastError();
}

}  // namespace moe
