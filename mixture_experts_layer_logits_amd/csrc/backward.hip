// Backward of the routed MoE layer (Primus blog, MegaMoE section: the
// backward mirrors the forward through dispatch/combine duality, with the
// FC2 and FC1 data-gradient GEMMs, and weight-gradient GEMMs that contract over
// each expert's rows, so their K varies by expert).
//
//   b1+b7  per token: dY_perm[row] = rnd(w dy[t]), d_gate = <dy[t], y_perm[row]>,
//          d_logits through the gate function
//   b2     dh = dY_perm . w_down[e]; epilogue: dg = rnd(dh u silu'(g)),
//          du = rnd(dh silu(g)), h = rnd(silu(g) u) from the saved g, u
//   b3     dw_down[e] = dY_perm^T . h          (K = rows of expert e)
//   b4     dX_perm = [dg | du] . [w_gate[e]; w_up[e]]
//   b5     [dw_gate[e]; dw_up[e]] = [dg | du]^T . x_perm   (K = rows of e)
//   b6     dx[t] = sum_j dX_perm[token_row[t, j]]
//
// The GEMMs take each operand either K-contiguous ("row" operands, as in the
// forward) or M-contiguous ("column" operands: a weight read against its
// storage order, or activations contracted over rows).  The direct-to-LDS
// kernels (d and F multiples of 256: bwd_dma_kernel for dh and dX, the
// persistent bwd_wgrad_kernel for the weight gradients) keep column
// operands in storage order in LDS and build their MFMA fragments with the
// transposing LDS read (ds_read_b64_tr_b16).  The MFMA kernel for other
// shapes transposes them in registers on their way to LDS and reads 16-byte
// rows as the forward kernel does.  Weight-gradient tiles of experts without
// rows run zero K steps and store exact zeros.
#include <float.h>

#include <algorithm>

#include "gemm_tiles.h"

namespace moe {

bool backward_supported(const moe_shape&) { return true; }

// ---------------------------------------------------------------------------
// b1 + b7: one workgroup per token.
// ---------------------------------------------------------------------------
template <typename T, int JB>
__global__ void __launch_bounds__(256)
bwd_dispatch_kernel(const T* __restrict__ dy, const T* __restrict__ y_perm,
                    const int32_t* __restrict__ token_row, const int32_t* __restrict__ topk_idx,
                    const float* __restrict__ topk_w, const float* __restrict__ logits, int d,
                    int E, int k, int score, int renorm, T* __restrict__ dY,
                    float* __restrict__ d_gate, float* __restrict__ d_logits) {
  __shared__ float red[256];
  __shared__ float s_dg[64];
  __shared__ float s_stat[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const T* dyt = dy + (long long)t * d;
  const int lane = tid & 63, wave = tid >> 6;
  __shared__ float s_part[64][4];
  const bool vec = (sizeof(T) == 2) && (d % 8 == 0);
  if (vec) {
    // The token's rows in batches of JB (the largest of 1, 2, 4, 8 not above
    // k).  Per 8-column run a thread loads dy once and the batch's y_perm
    // rows unconditionally (a slot past k reads row 0, unused), then forms
    // each row's products and its 16-byte store of w * dy: the loads of a
    // run are not waited for one by one, nor behind the previous row's
    // stores.  Each row's partial dot product runs over the thread's runs in
    // ascending order, as it would one row at a time.
    const bf16_t* dyb = reinterpret_cast<const bf16_t*>(dyt);
    for (int j0 = 0; j0 < k; j0 += JB) {
      int r[JB];
      float w[JB], part[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const bool in = j0 + jj < k;
        r[jj] = in ? token_row[(long long)t * k + j0 + jj] : -1;
        w[jj] = in ? topk_w[(long long)t * k + j0 + jj] : 0.0f;
        part[jj] = 0.0f;
      }
      for (int c = tid * 8; c < d; c += 256 * 8) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(dyb + c);
        u32x4_t yv[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
          yv[jj] = *reinterpret_cast<const u32x4_t*>(
              reinterpret_cast<const bf16_t*>(y_perm) + (long long)(r[jj] < 0 ? 0 : r[jj]) * d + c);
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          if (r[jj] < 0) continue;
          u32x4_t o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float g0 = __uint_as_float(a[q] << 16), g1 = __uint_as_float(a[q] & 0xffff0000u);
            const float y0 = __uint_as_float(yv[jj][q] << 16), y1 = __uint_as_float(yv[jj][q] & 0xffff0000u);
            part[jj] = fmaf(g0, y0, part[jj]);
            part[jj] = fmaf(g1, y1, part[jj]);
            o[q] = pack_bf16x2(w[jj] * g0, w[jj] * g1);
          }
          *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(dY) + (long long)r[jj] * d + c) = o;
        }
      }
      // wave reductions (fixed butterfly order), partials combined below
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (j0 + jj >= k) continue;
        float pv = part[jj];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) pv += __shfl_xor(pv, off, 64);
        if (lane == 0) s_part[j0 + jj][wave] = pv;
      }
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int r = token_row[(long long)t * k + j];
      const float w = topk_w[(long long)t * k + j];
      float part = 0.0f;
      if (r >= 0) {
        for (int c = tid; c < d; c += 256) {
          const float g = to_f32<T>(dyt[c]);
          dY[(long long)r * d + c] = from_f32<T>(w * g);
          part = fmaf(g, to_f32<T>(y_perm[(long long)r * d + c]), part);
        }
      }
      // wave reduction (fixed butterfly order), partials combined below
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
      if (lane == 0) s_part[j][wave] = part;
    }
  }
  __syncthreads();
  if (tid < k) {
    const float v = (s_part[tid][0] + s_part[tid][1]) + (s_part[tid][2] + s_part[tid][3]);
    s_dg[tid] = v;
    d_gate[(long long)t * k + tid] = v;
  }
  __syncthreads();
  // d_logits[t, :]
  const float* lt = logits + (long long)t * E;
  const int32_t* it = topk_idx + (long long)t * k;
  const float* wt = topk_w + (long long)t * k;
  if (tid == 0) {
    float dot = 0.0f, ssum = 0.0f;
    for (int j = 0; j < k; ++j) {
      dot += wt[j] * s_dg[j];
      if (score == MOE_SCORE_SIGMOID) ssum += 1.0f / (1.0f + expf(-lt[it[j]]));
    }
    s_stat[0] = dot;
    s_stat[1] = ssum;
  }
  float mx = -FLT_MAX, z = 0.0f;
  if (score == MOE_SCORE_SOFTMAX && !renorm) {
    float m = -FLT_MAX;
    for (int e = tid; e < E; e += 256) m = fmaxf(m, lt[e]);
    red[tid] = m;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] = fmaxf(red[tid], red[tid + off]);
      __syncthreads();
    }
    mx = red[0];
    __syncthreads();
    float zs = 0.0f;
    for (int e = tid; e < E; e += 256) zs += expf(lt[e] - mx);
    red[tid] = zs;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
      if (tid < off) red[tid] += red[tid + off];
      __syncthreads();
    }
    z = red[0];
    // sum_j dg_j p_{e_j}
    if (tid == 0) {
      float q = 0.0f;
      for (int j = 0; j < k; ++j) q += s_dg[j] * (expf(lt[it[j]] - mx) / z);
      s_stat[2] = q;
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    int jsel = -1;
    for (int j = 0; j < k; ++j)
      if (it[j] == e) jsel = j;
    float v = 0.0f;
    if (score == MOE_SCORE_SOFTMAX) {
      if (renorm) {
        if (jsel >= 0) v = wt[jsel] * (s_dg[jsel] - s_stat[0]);
      } else {
        const float p = expf(lt[e] - mx) / z;
        v = -p * s_stat[2] + (jsel >= 0 ? p * s_dg[jsel] : 0.0f);
      }
    } else if (jsel >= 0) {
      const float sg = 1.0f / (1.0f + expf(-lt[e]));
      const float ds = renorm ? (s_dg[jsel] - s_stat[0]) / s_stat[1] : s_dg[jsel];
      v = ds * sg * (1.0f - sg);
    }
    d_logits[(long long)t * E + e] = v;
  }
}

// ---------------------------------------------------------------------------
// b6: dx[t] = sum_j dX_perm[token_row[t, j]] (fp32, fixed order), then
// + dX_shared[t] when the layer has a shared expert (dXs non-null).
// ---------------------------------------------------------------------------
template <typename T, int JB>
__global__ void __launch_bounds__(256)
bwd_gather_kernel(const T* __restrict__ dX, const int32_t* __restrict__ token_row, int d, int k,
                  const T* __restrict__ dXs, float* __restrict__ dx) {
  const int t = blockIdx.x;
  const int32_t* rows = token_row + (long long)t * k;
  if (sizeof(T) == 2 && d % 8 == 0) {
    // batches of JB rows as straight-line code: the row loads unconditional
    // (a slot past k reads row 0, unused), then the sums in the order j = 0,
    // 1, ..., k-1; a load under a branch, or added where it was loaded, was
    // waited for on its own.  A token's rows are uniform over the workgroup.
    const bf16_t* X = reinterpret_cast<const bf16_t*>(dX);
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
      float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int j0 = 0; j0 < k; j0 += JB) {
        u32x4_t raw[JB];
        int r[JB];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          r[jj] = j0 + jj < k ? rows[j0 + jj] : -1;
          raw[jj] = *reinterpret_cast<const u32x4_t*>(X + (long long)(r[jj] < 0 ? 0 : r[jj]) * d + c);
        }
        float v[JB][8];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v[jj][2 * q] = __uint_as_float(raw[jj][q] << 16);
            v[jj][2 * q + 1] = __uint_as_float(raw[jj][q] & 0xffff0000u);
          }
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) {
          if (r[jj] < 0) continue;
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += v[jj][i];
        }
      }
      if (dXs) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(
            reinterpret_cast<const bf16_t*>(dXs) + (long long)t * d + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += __uint_as_float(v[q] << 16);
          acc[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
        }
      }
      float* o = dx + (long long)t * d + c;
      *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      *reinterpret_cast<float4*>(o + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
    }
    return;
  }
  for (int c = threadIdx.x; c < d; c += 256) {
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r >= 0) acc += to_f32<T>(dX[(long long)r * d + c]);
    }
    if (dXs) acc += to_f32<T>(dXs[(long long)t * d + c]);
    dx[(long long)t * d + c] = acc;
  }
}

// ---------------------------------------------------------------------------
// Backward GEMM problems.  C[m, n] = sum_k A(m, k) B(n, k) with
//   row operand:    X(i, k) at base[i * ld + k]
//   column operand: X(i, k) at base[k * ld + i]
// ---------------------------------------------------------------------------
enum { BWD_DH = 0, BWD_DX = 1, BWD_WD = 2, BWD_WGU = 3 };

struct BwdArgs {
  int E, F, d;
  const int32_t* offsets;
  const int32_t* tiles;    // row-grouped modes: tile prefix per expert
  const void* dY;          // [R, d]
  const void* gu;          // [R, 2F] saved g | u
  const void* dgu;         // [R, 2F]
  const void* h;           // [R, F]
  const void* x_perm;      // [R, d]
  const void* w_gate;      // [E, F, d]
  const void* w_up;        // [E, F, d]
  const void* w_down;      // [E, d, F]
  void* out_dgu;           // BWD_DH: dg | du
  void* out_h;             // BWD_DH: h
  void* out_dX;            // BWD_DX
  void* dw_down;           // BWD_WD
  void* dw_gate;           // BWD_WGU
  void* dw_up;
  int wgrad_bf16;          // weight gradients stored as bf16 (else fp32)
};

// Element offset of weight-gradient entry (m, n) of expert e (BWD_WD: of
// dw_down [E, d, F]; BWD_WGU: rows m < F of dw_gate, then dw_up), and the
// base pointer it belongs to.
template <int MODE>
__device__ __forceinline__ long long wgrad_offset(const BwdArgs& a, int e, int m, int n,
                                                  void*& base) {
  if (MODE == BWD_WD) {
    base = a.dw_down;
    return ((long long)e * a.d + m) * a.F + n;
  }
  base = (m < a.F) ? a.dw_gate : a.dw_up;
  return ((long long)e * a.F + (m < a.F ? m : m - a.F)) * a.d + n;
}

// The operands of one tile, resolved from the mode.
template <typename T>
struct BwdJob {
  const T* A; long long lda; bool a_col;
  const T* B0; const T* B1; long long ldb; bool b_col; int kswitch;  // B1 for k >= kswitch
  int M_valid, N_valid, K;    // rows of A valid in this tile's group (row modes)
  int m0, n0;
  int row0, e;
  int cls;                    // 0: BM x BN tile, 1: BM/2 x 2BN tail tile (TAIL decode)
};

// TAIL (dh and dX of the direct-to-LDS kernel): the tile list was built
// with tail tiles (schedule_tiles_kernel, tail = 1).  As in the forward's
// decode, column tiles go in pairs: the expert's full row tiles of columns
// 2p and 2p + 1, then its tail tile (the last <= BM/2 rows) over the same
// 2 BN columns, which finds that weight strip still in L2.
template <int MODE, int BM, int BN, typename T, bool TAIL = false>
__device__ __forceinline__ bool bwd_decode(const BwdArgs& a, BwdJob<T>& j) {
  const int bid = blockIdx.x;
  j.cls = 0;
  if (MODE == BWD_DH || MODE == BWD_DX) {
    const int total = a.tiles[a.E];
    const int per = (total + 7) >> 3, slot = bid >> 3;
    if (slot >= per) return false;
    const int lid = (bid & 7) * per + slot;
    if (lid >= total) return false;
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tiles[mid] <= lid) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int row0 = a.offsets[g], rows = a.offsets[g + 1] - row0;
    const int r = lid - a.tiles[g];
    if (!TAIL) {
      const int mt = cdiv(rows, BM);
      j.m0 = (r % mt) * BM;
      j.n0 = (r / mt) * BN;
    } else {
      const int mt = group_full_rows(rows, BM, 1);
      const int ht = (mt * BM < rows) ? 1 : 0;
      const int nt = cdiv(MODE == BWD_DH ? a.F : a.d, BN);
      const int per = 2 * mt + ht;
      const int p = r / per, q = r - p * per;
      const int pair_cols = (nt - 2 * p) < 2 ? (nt - 2 * p) : 2;
      if (q < pair_cols * mt) {
        j.m0 = (q % mt) * BM;
        j.n0 = (2 * p + q / mt) * BN;
      } else {
        j.cls = 1;
        j.m0 = mt * BM;
        j.n0 = p * 2 * BN;
      }
    }
    j.row0 = row0;
    j.e = g;
    j.M_valid = rows;
    if (MODE == BWD_DH) {
      j.A = static_cast<const T*>(a.dY) + (long long)row0 * a.d; j.lda = a.d; j.a_col = false;
      j.B0 = static_cast<const T*>(a.w_down) + (long long)g * a.d * a.F;
      j.B1 = j.B0; j.ldb = a.F; j.b_col = true; j.kswitch = 1 << 30;
      j.N_valid = a.F; j.K = a.d;
    } else {
      j.A = static_cast<const T*>(a.dgu) + (long long)row0 * 2 * a.F; j.lda = 2LL * a.F; j.a_col = false;
      j.B0 = static_cast<const T*>(a.w_gate) + (long long)g * a.F * a.d;
      j.B1 = static_cast<const T*>(a.w_up) + (long long)g * a.F * a.d - (long long)a.F * a.d;
      j.ldb = a.d; j.b_col = true; j.kswitch = a.F;   // rows k >= F come from w_up[k - F]
      j.N_valid = a.d; j.K = 2 * a.F;
    }
    return true;
  }
  // per-expert weight gradients: fixed tile grid, K = rows of the expert
  const int Mtot = (MODE == BWD_WD) ? a.d : 2 * a.F;
  const int Ntot = (MODE == BWD_WD) ? a.F : a.d;
  const int mt = cdiv(Mtot, BM), nt = cdiv(Ntot, BN);
  const int total = a.E * mt * nt;
  const int per = (total + 7) >> 3, slot = bid >> 3;
  if (slot >= per) return false;
  const int lid = (bid & 7) * per + slot;
  if (lid >= total) return false;
  const int g = lid / (mt * nt), r = lid - g * mt * nt;
  j.m0 = (r % mt) * BM;
  j.n0 = (r / mt) * BN;
  j.e = g;
  j.row0 = a.offsets[g];
  j.K = a.offsets[g + 1] - j.row0;
  j.M_valid = Mtot;
  j.N_valid = Ntot;
  if (MODE == BWD_WD) {
    j.A = static_cast<const T*>(a.dY) + (long long)j.row0 * a.d; j.lda = a.d; j.a_col = true;
    j.B0 = static_cast<const T*>(a.h) + (long long)j.row0 * a.F; j.ldb = a.F; j.b_col = true;
  } else {
    j.A = static_cast<const T*>(a.dgu) + (long long)j.row0 * 2 * a.F; j.lda = 2LL * a.F; j.a_col = true;
    j.B0 = static_cast<const T*>(a.x_perm) + (long long)j.row0 * a.d; j.ldb = a.d; j.b_col = true;
  }
  j.B1 = j.B0;
  j.kswitch = 1 << 30;
  return true;
}

// Epilogue for one output element group of 4 consecutive columns.
template <int MODE, typename T>
__device__ __forceinline__ void bwd_store4(const BwdArgs& a, const BwdJob<T>& j, int m, int n,
                                           const float (&v)[4], bool precise) {
  if (MODE == BWD_DH) {
    // bf16 only (the MFMA path): 8-byte loads of 4 g and 4 u, 8-byte stores
    const long long r = (long long)(j.row0 + m);
    const bf16_t* gu = static_cast<const bf16_t*>(a.gu) + r * 2 * a.F;
    bf16_t* dgu = static_cast<bf16_t*>(a.out_dgu) + r * 2 * a.F;
    bf16_t* h = static_cast<bf16_t*>(a.out_h) + r * a.F;
    const uint2 gq = *reinterpret_cast<const uint2*>(gu + n);
    const uint2 uq = *reinterpret_cast<const uint2*>(gu + a.F + n);
    const uint32_t gw[2] = {gq.x, gq.y}, uw[2] = {uq.x, uq.y};
    float dg[4], du[4], hh[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t gb = gw[q >> 1], ub = uw[q >> 1];
      const float g = __uint_as_float((q & 1) ? (gb & 0xffff0000u) : (gb << 16));
      const float u = __uint_as_float((q & 1) ? (ub & 0xffff0000u) : (ub << 16));
      const float sg = 1.0f / (1.0f + (precise ? expf(-g) : __expf(-g)));
      const float sl = g * sg;
      dg[q] = v[q] * u * sg * (1.0f + g * (1.0f - sg));
      du[q] = v[q] * sl;
      hh[q] = sl * u;
    }
    *reinterpret_cast<uint2*>(dgu + n) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
    *reinterpret_cast<uint2*>(dgu + a.F + n) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
    *reinterpret_cast<uint2*>(h + n) = make_uint2(pack_bf16x2(hh[0], hh[1]), pack_bf16x2(hh[2], hh[3]));
  } else if (MODE == BWD_DX) {
    bf16_t* o = static_cast<bf16_t*>(a.out_dX) + (long long)(j.row0 + m) * a.d + n;
    *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  } else {
    void* base;
    const long long o = wgrad_offset<MODE>(a, j.e, m, n, base);
    if (a.wgrad_bf16)
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(base) + o) =
          make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    else
      *reinterpret_cast<float4*>(static_cast<float*>(base) + o) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA backward tile kernel: 4 waves (2 x 2), 128 x 128 tile, K slices
// of 32 through two padded LDS stages, next slice prefetched into registers.
// Row operands: each thread moves two 16-byte chunks (row c/4, k-chunk c%4).
// Column operands: each thread loads two k-rows x 8 columns and writes them
// transposed as eight (k, k+1) pairs, one per column.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(256)
bwd_mfma_kernel(const BwdArgs args) {
  constexpr int BM = 128, BN = 128, BK = 32, LDK = BK + 8;
  constexpr int WTM = 64, WTN = 64, MI = 2, NJ = 2;
  constexpr int STAGE = (BM + BN) * LDK;
  __shared__ __attribute__((aligned(16))) bf16_t smem[2 * STAGE];

  BwdJob<bf16_t> job;
  if (!bwd_decode<MODE, BM, BN>(args, job)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // row-operand chunk mapping
  const int rc_row = tid >> 2, rc_k = (tid & 3) * 8;
  // column-operand mapping: k pair kp, 8-column chunk mc
  const int kp = tid & 15, mc = tid >> 4;
  const bool row_modes = (MODE == BWD_DH || MODE == BWD_DX);

  u32x4_t ra[2], rb[2];
  // Loads slice k0 of one operand into registers.
  auto load_row = [&](const bf16_t* base, long long ld, int r0, int rvalid, int k0, u32x4_t (&reg)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int r = r0 + rc_row + 64 * i;
      r = r < rvalid ? r : rvalid - 1;
      reg[i] = *reinterpret_cast<const u32x4_t*>(base + (long long)r * ld + k0 + rc_k);
    }
  };
  auto load_col = [&](const bf16_t* base, long long ld, int c0, int k0, int kvalid, u32x4_t (&reg)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int kk = k0 + 2 * kp + q;
      if (kk < kvalid)
        reg[q] = *reinterpret_cast<const u32x4_t*>(base + (long long)kk * ld + c0 + mc * 8);
      else
        reg[q] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  auto store_row = [&](bf16_t* s, const u32x4_t (&reg)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      *reinterpret_cast<u32x4_t*>(&s[(rc_row + 64 * i) * LDK + rc_k]) = reg[i];
  };
  auto store_col = [&](bf16_t* s, const u32x4_t (&reg)[2]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = reg[0][w], b = reg[1][w];
      const uint32_t lo = (a & 0xffffu) | (b << 16);
      const uint32_t hi = (a >> 16) | (b & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(&s[(mc * 8 + 2 * w) * LDK + 2 * kp]) = lo;
      *reinterpret_cast<uint32_t*>(&s[(mc * 8 + 2 * w + 1) * LDK + 2 * kp]) = hi;
    }
  };
  const int K = job.K;
  auto gload = [&](int k0) {
    if (row_modes) load_row(job.A, job.lda, job.m0, job.M_valid, k0, ra);
    else load_col(job.A, job.lda, job.m0, k0, K, ra);
    const bf16_t* B = (k0 >= job.kswitch) ? job.B1 : job.B0;
    load_col(B, job.ldb, job.n0, k0, K, rb);
  };
  auto lstore = [&](int stage) {
    bf16_t* sA = smem + stage * STAGE;
    bf16_t* sB = sA + BM * LDK;
    if (row_modes) store_row(sA, ra); else store_col(sA, ra);
    store_col(sB, rb);
  };

  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.0f;

  const int KT = cdiv(K, BK);
  const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
  if (KT > 0) {
    gload(0);
    lstore(0);
    __syncthreads();
  }
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload((kt + 1) * BK);
    const bf16_t* sA = smem + cur * STAGE;
    const bf16_t* sB = sA + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t af[MI], bfr[NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&sA[(wm * WTM + i * 32 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj)
        bfr[jj] = *reinterpret_cast<const bf16x8_t*>(&sB[(wn * WTN + jj * 32 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[i], acc[i][jj], 0, 0, 0);
    }
    if (kt + 1 < KT) lstore(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = job.m0 + wm * WTM + i * 32 + frag_row;
    if (row_modes && m >= job.M_valid) continue;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = job.n0 + wn * WTN + jj * 32 + 8 * q + 4 * (lane >> 5);
        const float v[4] = {acc[i][jj][4 * q], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2],
                            acc[i][jj][4 * q + 3]};
        bwd_store4<MODE, bf16_t>(args, job, m, n, v, false);
      }
  }
}

// ---------------------------------------------------------------------------
// Generic backward tile kernel (any shape, fp32 or bf16 storage, fp32 FMA):
// 64 x 64 tiles, K slices of 16, strided operand access.
// ---------------------------------------------------------------------------
template <int MODE, typename T>
__global__ void __launch_bounds__(256)
bwd_generic_kernel(const BwdArgs args) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[BK][BN + 4];
  BwdJob<T> job;
  if (!bwd_decode<MODE, BM, BN>(args, job)) return;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < job.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / BK, kk = e % BK;
      const int m = job.m0 + r, k = k0 + kk;
      float va = 0.0f;
      const bool mv = (MODE == BWD_DH || MODE == BWD_DX) ? (m < job.M_valid) : (m < job.M_valid);
      if (mv && k < job.K)
        va = to_f32<T>(job.a_col ? job.A[(long long)k * job.lda + m] : job.A[(long long)m * job.lda + k]);
      sA[kk][r] = va;
      const int n = job.n0 + r;
      float vb = 0.0f;
      if (n < job.N_valid && k < job.K) {
        const T* B = (k >= job.kswitch) ? job.B1 : job.B0;
        vb = to_f32<T>(job.b_col ? B[(long long)k * job.ldb + n] : B[(long long)n * job.ldb + k]);
      }
      sB[kk][r] = vb;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) bv[jj] = sB[kk][tx * 4 + jj];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = fmaf(av[i], bv[jj], acc[i][jj]);
    }
    __syncthreads();
  }
  for (int i = 0; i < 4; ++i) {
    const int m = job.m0 + ty * 4 + i;
    if (m >= job.M_valid) continue;
    for (int jj = 0; jj < 4; ++jj) {
      const int n = job.n0 + tx * 4 + jj;
      if (n >= job.N_valid) continue;
      const float v = acc[i][jj];
      if (MODE == BWD_DH) {
        const long long r = (long long)(job.row0 + m);
        const T* gu = static_cast<const T*>(args.gu) + r * 2 * args.F;
        const float g = to_f32<T>(gu[n]), u = to_f32<T>(gu[args.F + n]);
        const float sg = 1.0f / (1.0f + expf(-g));
        const float sl = g * sg;
        static_cast<T*>(args.out_dgu)[r * 2 * args.F + n] = from_f32<T>(v * u * sg * (1.0f + g * (1.0f - sg)));
        static_cast<T*>(args.out_dgu)[r * 2 * args.F + args.F + n] = from_f32<T>(v * sl);
        static_cast<T*>(args.out_h)[r * args.F + n] = from_f32<T>(sl * u);
      } else if (MODE == BWD_DX) {
        static_cast<T*>(args.out_dX)[(long long)(job.row0 + m) * args.d + n] = from_f32<T>(v);
      } else {
        void* base;
        const long long o = wgrad_offset<MODE>(args, job.e, m, n, base);
        if (args.wgrad_bf16) static_cast<bf16_t*>(base)[o] = f32_to_bf16(v);
        else static_cast<float*>(base)[o] = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dh and dX on the forward kernel's structure (256 x 256 tiles, 8 waves of
// 64 x 128, direct global->LDS loads into a 4-stage ring of 32-wide K
// slices).  The row operand (dY_perm for dh, dg | du for dX) is read as the
// forward reads its rows.  The weights are the column operand: stored
// N-contiguous, they keep that order in LDS, 32 k-rows of 512 bytes (256
// columns), 16-byte chunk c of k-row r at position c ^ 4 (r mod 4), so the
// four k-rows one transposing read touches fill all 64 banks (with
// c ^ 2 (r mod 4), rows r and r + 1 shared 16 banks).  Its MFMA fragments
// come from two transposing LDS reads (ds_read_b64_tr_b16): within each
// 16-lane group, lane j points at k-row kb + j / 4, columns mb + 4 (j mod 4);
// lane i then receives the four k-values of column mb + i, the k-contiguous
// fragment a row operand gives with one 16-byte read.
//
// Tail tiles, as in the forward: an expert whose last t rows number at most
// 128 gets 128-row x 512-column tiles for them instead of half-empty
// 256-row tiles (Qwen3-235B shape: 23% of the MFMA work was padding rows
// with 256-row tiles only, 12% with tail tiles).  Their waves are laid out
// 2 x 4, each keeping its 64 x 128 block; a stage then holds the two
// 256-column halves of the weights (16 KiB each) and 128 operand rows
// (8 KiB), 40 KiB, and each wave loads 5 blocks of 1 KiB instead of 4.
// Columns past N (an odd number of 256-column tiles) are clamped on load
// and never stored.
// ---------------------------------------------------------------------------
typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ void __launch_bounds__(512)
bwd_dma_kernel(const BwdArgs args) {
  static_assert(MODE == BWD_DH || MODE == BWD_DX, "dh and dX only");
  constexpr int BM = 256, BN = 256, BK = 32, WTM = 64, WTN = 128;
  constexpr int MI = WTM / 32, NJ = WTN / 32;
  constexpr int OPB = BM * BK * 2;              // bytes of 256 rows or columns per stage (16 KiB)
  constexpr int STAGE_B = OPB * 5 / 2;          // bytes per stage: 40 KiB (a tail tile's)
  constexpr int STAGE = STAGE_B / 2;            // ... in bf16 elements
  constexpr int BPWX = 5;                       // 1 KiB load blocks per wave per stage, at most
  __shared__ __attribute__((aligned(1024))) bf16_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[STAGE];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[STAGE];

  BwdJob<bf16_t> job;
  if (!bwd_decode<MODE, BM, BN, bf16_t, true>(args, job)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool tail = __builtin_amdgcn_readfirstlane(job.cls) != 0;
  const int wn_count = tail ? 4 : 2;
  const int wm = wave / wn_count, wn = wave % wn_count;
  const int K = job.K;
  const int KT = cdiv(K, BK);
  // byte offsets within a stage: full tiles hold A (256 rows) then B (256
  // columns); tail tiles B's two halves, then A (128 rows)
  const int bpw = tail ? 5 : 4;
  const int a_off = tail ? 2 * OPB : 0;
  const int b_off = tail ? (wn >> 1) * OPB : OPB;
  const int bcol0 = (tail ? (wn & 1) : wn) * WTN;   // this wave's first column within its B half

  // ---- loads: block gb = wave * bpw + j of the stage ----------------------
  // full: gb < 16 A rows 16 gb.., else B block gb - 16; tail: gb < 8 A rows
  // 16 gb.., else B half (gb - 8) / 16, block (gb - 8) % 16.  A row blocks
  // hold 16 rows x 64 bytes, B blocks two k-rows x 512 bytes.
  const int n_a = tail ? 8 : 16;
  uint32_t g_off[BPWX];                         // byte offsets, k-independent part
  int krow_l[BPWX];                             // B blocks: k-row of this lane (-1: an A block)
  uint32_t lds_b[BPWX];                         // byte offset of the block in a stage
  // A blocks: the block's first row folded into a 64-bit base, so a lane's
  // 32-bit offset spans at most 16 rows whatever the group's size
  const char* a_base[BPWX];
#pragma unroll
  for (int j = 0; j < BPWX; ++j) {
    const int gb = wave * bpw + (j < bpw ? j : bpw - 1);
    if (gb < n_a) {
      const int rb = job.m0 + 16 * gb;
      const int r0 = rb < job.M_valid ? rb : job.M_valid - 1;
      int r = rb + (lane >> 2);
      r = r < job.M_valid ? r : job.M_valid - 1;
      const int c = (lane & 3) ^ swz(lane >> 2);
      krow_l[j] = -1;
      g_off[j] = (uint32_t)((r - r0) * (int)job.lda + c * 8) * 2u;
      a_base[j] = uniform_ptr(job.A + (long long)r0 * job.lda);
      lds_b[j] = (uint32_t)(a_off + gb * 1024);
    } else {
      const int bb = gb - n_a;                   // 0..15 (full) or 0..31 (tail)
      const int half = bb >> 4, blk = bb & 15;
      const int kr = 2 * blk + (lane >> 5);
      const int c = (lane & 31) ^ (4 * (kr & 3));
      int col = job.n0 + half * BN + c * 8;
      col = col < job.N_valid - 8 ? col : job.N_valid - 8;   // never stored
      krow_l[j] = kr;
      g_off[j] = (uint32_t)col * 2u;
      a_base[j] = nullptr;
      lds_b[j] = (uint32_t)((tail ? 0 : OPB) + bb * 1024);
    }
  }
  auto dma = [&](bf16_t* stage, int k0, auto nblk_c) {
    constexpr int NBLK = decltype(nblk_c)::value;
    const bf16_t* srcb = (k0 >= job.kswitch) ? job.B1 : job.B0;
    const char* base_b = reinterpret_cast<const char*>(srcb);
    const uint32_t st_lds = (uint32_t)(uintptr_t)MOE_AS_LDS(reinterpret_cast<char*>(stage));
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const uint32_t lds = st_lds + lds_b[j];
      if (krow_l[j] < 0) {
        const char* base_a = a_base[j] + (size_t)k0 * 2;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(lds), "v"(g_off[j]), "s"(base_a) : "memory");
      } else {
        int kr = k0 + krow_l[j];
        kr = kr < K ? kr : K - 1;
        const uint32_t off = g_off[j] + (uint32_t)(kr * (int)job.ldb) * 2u;
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(lds), "v"(off), "s"(base_b) : "memory");
      }
    }
  };

  // ---- fragments ----------------------------------------------------------
  const int frag_row = lane & 31;
  const int sw = swz(frag_row);
  const int kpos0 = ((0 + (lane >> 5)) ^ sw) << 3;
  const int kpos1 = ((2 + (lane >> 5)) ^ sw) << 3;
  // column operand, per lane: k-row part and chunk part of the transposing read
  const int tr_row = (8 * (lane >> 5) + ((lane & 15) >> 2)) * 512;
  const int tr_swz = 4 * ((lane & 15) >> 2);
  const int tr_c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = (lane & 1) * 8;
  auto col_frag = [&](const char* op, int kk, int mcol0) -> bf16x8_t {
    const int c = (tr_c + (mcol0 >> 3)) ^ tr_swz;
    const char* p = op + kk * 16 * 512 + tr_row + (c << 4) + tr_half;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)MOE_AS_LDS(p));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)MOE_AS_LDS(p + 4 * 512));
    const auto v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  };
  auto load_frags = [&](const bf16_t* stage, int kk, bf16x8_t (&af)[MI], bf16x8_t (&bfr)[NJ]) {
    const char* sa = reinterpret_cast<const char*>(stage) + a_off;
    const char* sb = reinterpret_cast<const char*>(stage) + b_off;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int off = (wm * WTM + i * 32 + frag_row) * BK + (kk ? kpos1 : kpos0);
      af[i] = *reinterpret_cast<const bf16x8_t*>(reinterpret_cast<const bf16_t*>(sa) + off);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[j] = col_frag(sb, kk, bcol0 + j * 32);
  };
  f32x16_t acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  auto mma = [&](const bf16x8_t (&af)[MI], const bf16x8_t (&bfr)[NJ]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Fragment reads spread between the MFMAs of each half-step (the first
  // reads of a half go ahead of its first MFMA, then one read per MFMA).
  // The last step also reads the (unused) next stage so that reads and
  // MFMAs stay in one block.
  constexpr int NREAD = MI + 2 * NJ;            // LDS reads per half-step
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD - (MI * NJ - 1), 0);
#pragma unroll
    for (int r = 0; r < MI * NJ - 1; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };
  // The K loop exists once per load-block count (4 or 5 per wave): the
  // vmcnt waits count this wave's loads per slice.
  auto k_loop = [&](auto nblk_c) {
    constexpr int NBLK = decltype(nblk_c)::value;
    auto wait_slice = [&](int ready, int issued) {
      const int younger = issued - 1 - ready;
      if (younger >= 2) wait_vmcnt<2 * NBLK>();
      else if (younger == 1) wait_vmcnt<NBLK>();
      else wait_vmcnt<0>();
    };
    bf16x8_t af0[MI], af1[MI], bf0[NJ], bf1[NJ];
    auto step = [&](const bf16_t* cur, const bf16_t* next, bf16_t* refill, int s) {
      __builtin_amdgcn_sched_barrier(0);
      load_frags(cur, 1, af1, bf1);
      mma(af0, bf0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < KT) wait_slice(s + 1, s + 3 < KT ? s + 3 : KT);
      barrier();
      if (s + 3 < KT) dma(refill, (s + 3) * BK, nblk_c);
      __builtin_amdgcn_sched_barrier(0);
      load_frags(next, 0, af0, bf0);
      mma(af1, bf1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (KT > 0) {
      dma(st0, 0, nblk_c);
      if (KT > 1) dma(st1, BK, nblk_c);
      if (KT > 2) dma(st2, 2 * BK, nblk_c);
      wait_slice(0, KT < 3 ? KT : 3);
      barrier();
      load_frags(st0, 0, af0, bf0);
      int kt = 0;
      for (; kt + 4 <= KT; kt += 4) {
        step(st0, st1, st3, kt);
        step(st1, st2, st0, kt + 1);
        step(st2, st3, st1, kt + 2);
        step(st3, st0, st2, kt + 3);
      }
      if (kt < KT) step(st0, st1, st3, kt);
      if (kt + 1 < KT) step(st1, st2, st0, kt + 1);
      if (kt + 2 < KT) step(st2, st3, st1, kt + 2);
    }
  };
  if (tail) k_loop(std::integral_constant<int, 5>{});
  else k_loop(std::integral_constant<int, 4>{});

  {
    // Outputs go out through LDS: in the accumulator layout a store
    // instruction scatters 16-byte pieces over 32 rows (which cost several
    // times their bytes in write traffic); re-read row-contiguous, every 16
    // (DX) or 32 (DH) lanes write whole runs of one row.  The ring is free
    // once every wave has passed this barrier; each wave stages through its
    // own 16 KiB (the first 32 KiB of each stage).
    barrier();
    char* buf = reinterpret_cast<char*>((wave >> 1) == 0 ? st0 : (wave >> 1) == 1 ? st1
                                        : (wave >> 1) == 2 ? st2 : st3) + (wave & 1) * 16384;
    const int rbase = job.m0 + wm * WTM;          // first row of this wave (within the group)
    const int cbase = job.n0 + wn * WTN;          // first column of this wave
    if (cbase >= job.N_valid) return;             // a tail tile's columns past N
    if constexpr (MODE == BWD_DX) {
      // 64 rows x 128 bf16 columns; 16-byte chunk c of row r at c ^ (r mod 16)
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = i * 32 + frag_row;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = j * 32 + 8 * q + 4 * (lane >> 5);
            const uint2 pk = make_uint2(pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                                        pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]));
            *reinterpret_cast<uint2*>(buf + r * 256 + (((c >> 3) ^ (r & 15)) << 4) + (c & 4) * 2) = pk;
          }
      }
      bf16_t* out = static_cast<bf16_t*>(args.out_dX) + (long long)job.row0 * args.d + cbase;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int r = 4 * t + (lane >> 4), ch = lane & 15;
        const uint4 v = *reinterpret_cast<const uint4*>(buf + r * 256 + ((ch ^ (r & 15)) << 4));
        if (rbase + r < job.M_valid)
          *reinterpret_cast<uint4*>(out + (long long)(rbase + r) * args.d + ch * 8) = v;
      }
    } else {
      // dh in fp32, 32 rows x 128 columns per block; 16-byte chunk c of row r
      // at c ^ r.  Each lane then owns 4 consecutive columns of one row per
      // pass and applies the SwiGLU backward with coalesced g, u loads and
      // dg, du, h stores.  The 32 passes go in groups of 4, and a group's g, u
      // loads are issued before the previous group's stores: vmcnt counts
      // loads and stores in issue order, so a load issued after a store
      // would wait for that store too.
      // GR passes per group, GPB groups per 32-row block, MI blocks
      constexpr int GR = 4, GPB = 16 / GR, NGRP = MI * GPB;
      static_assert(MI == 2, "the second block is staged halfway");
      const int ch = lane & 31;
      const long long F = args.F;
      const bf16_t* gu_e = static_cast<const bf16_t*>(args.gu) + (long long)job.row0 * 2 * F;
      bf16_t* dgu_e = static_cast<bf16_t*>(args.out_dgu) + (long long)job.row0 * 2 * F;
      bf16_t* h_e = static_cast<bf16_t*>(args.out_h) + (long long)job.row0 * F;
      auto stage_block = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = j * 8 + 2 * q + (lane >> 5);
            *reinterpret_cast<float4*>(buf + frag_row * 512 + ((c ^ frag_row) << 4)) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
          }
      };
      // pass t of block i: row 2 t + lane / 32 of the block
      auto row_of = [&](int grp, int u) {
        return rbase + (grp / GPB) * 32 + 2 * ((grp % GPB) * GR + u) + (lane >> 5);
      };
      uint2 gq[2][GR], uq[2][GR];
      auto load_gu = [&](int grp, uint2 (&g)[GR], uint2 (&uu)[GR]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < GR; ++u) {
          const int m = row_of(grp, u);
          const int mc = m < job.M_valid ? m : job.M_valid - 1;   // read a valid row, store none
          const bf16_t* pg = gu_e + (long long)mc * 2 * F + cbase + 4 * ch;
          g[u] = *reinterpret_cast<const uint2*>(pg);
          uu[u] = *reinterpret_cast<const uint2*>(pg + F);
        }
      };
      stage_block(0);
      load_gu(0, gq[0], uq[0]);
      static_for<NGRP>([&](auto gc) __attribute__((always_inline)) {
        constexpr int grp = decltype(gc)::value;
        if constexpr (grp + 1 < NGRP) load_gu(grp + 1, gq[(grp + 1) & 1], uq[(grp + 1) & 1]);
        float4 d4[GR];
#pragma unroll
        for (int u = 0; u < GR; ++u) {
          const int r = 2 * ((grp % GPB) * GR + u) + (lane >> 5);
          d4[u] = *reinterpret_cast<const float4*>(buf + r * 512 + ((ch ^ r) << 4));
        }
        // the next block reuses the staging buffer after this group's reads
        if constexpr (grp == GPB - 1) stage_block(1);
#pragma unroll
        for (int u = 0; u < GR; ++u) {
          const int m = row_of(grp, u);
          if (m < job.M_valid) {
            const float v[4] = {d4[u].x, d4[u].y, d4[u].z, d4[u].w};
            const uint32_t gw[2] = {gq[grp & 1][u].x, gq[grp & 1][u].y};
            const uint32_t uw[2] = {uq[grp & 1][u].x, uq[grp & 1][u].y};
            float dg[4], du[4], hh[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const uint32_t gb = gw[q >> 1], ub = uw[q >> 1];
              const float g = __uint_as_float((q & 1) ? (gb & 0xffff0000u) : (gb << 16));
              const float uv = __uint_as_float((q & 1) ? (ub & 0xffff0000u) : (ub << 16));
              const float sg = 1.0f / (1.0f + __expf(-g));
              const float sl = g * sg;
              dg[q] = v[q] * uv * sg * (1.0f + g * (1.0f - sg));
              du[q] = v[q] * sl;
              hh[q] = sl * uv;
            }
            const long long o = (long long)m * 2 * F + cbase + 4 * ch;
            *reinterpret_cast<uint2*>(dgu_e + o) =
                make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(dgu_e + o + F) =
                make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
            *reinterpret_cast<uint2*>(h_e + (long long)m * F + cbase + 4 * ch) =
                make_uint2(pack_bf16x2(hh[0], hh[1]), pack_bf16x2(hh[2], hh[3]));
          }
        }
      });
    }
  }
}

// Tile r of an expert's mt x nt weight-gradient grid: m-tiles go in groups
// of gm (the last may be smaller); within a group m runs fastest, then n, and
// the n direction alternates from group to group.  The tiles that run
// together on an XCD then form a gm x (slots / gm) block of the grid, and
// consecutive blocks share one operand's columns (a serpentine), which the
// XCD's L2 still holds.
__device__ __forceinline__ void wgrad_tile_mn(int r, int mt, int nt, int gm, int& mi, int& ni) {
  const int gi = r / (gm * nt);
  const int q = r - gi * gm * nt;
  const int gsz = min(gm, mt - gi * gm);
  const int nq = q / gsz;
  mi = gi * gm + (q - nq * gsz);
  ni = (gi & 1) ? nt - 1 - nq : nq;
}

// ---------------------------------------------------------------------------
// Weight gradients as a persistent kernel.  Each expert's tiles have a short
// K (its row count: about 512 rows in a Qwen3-235B-shape step), so a
// workgroup per tile spent more time starting, waiting for its first slice
// and draining its epilogue than in its K loop (per-tile timestamps: 3.7 us
// to the first slice, a 15 us K loop, a 4.6 us epilogue, 1.7 us between
// workgroups).  Here one workgroup per CU walks a run of tiles, and the
// stream of K slices continues across tiles: the next tile's first slices
// load during the current tile's last steps and its epilogue.
//
// The epilogue therefore cannot stage its results in the ring (which holds
// those slices): each wave has 4 KiB of its own, one 32 x 32 fp32 block at a
// time, rows of 128 bytes with 16-byte chunk c of row r at c ^ ((r >> 1) & 7),
// which is conflict-free for both the accumulator-layout writes and the
// row-contiguous reads; each store instruction covers 8 rows x 128 bytes.
//
// vmcnt counts loads and stores in issue order, so a wait for a slice
// issued before an epilogue's stores need not wait for them, while a wait
// for one issued after them does: each wave counts the memory operations it
// issued after the slice it waits for.
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(512)
bwd_wgrad_kernel(const BwdArgs args) {
  static_assert(MODE == BWD_WD || MODE == BWD_WGU, "weight gradients only");
  constexpr int BM = 256, BN = 256, BK = 32, WN = 2;
  constexpr int WTM = 64, WTN = 128, MI = WTM / 32, NJ = WTN / 32;
  constexpr int OPB = BM * BK * 2;              // bytes of one operand per stage (16 KiB)
  constexpr int STAGE = OPB;                    // bf16 elements per stage (A then B)
  constexpr int BPW = 4;                        // 1 KiB load blocks per wave per slice
  constexpr int NST = MI * NJ * 4;              // global stores per wave per epilogue
  __shared__ __attribute__((aligned(1024))) bf16_t ring[4 * STAGE];
  __shared__ __attribute__((aligned(1024))) float stg[8][32 * 32];

  const int Mtot = MODE == BWD_WD ? args.d : 2 * args.F;
  const int Ntot = MODE == BWD_WD ? args.F : args.d;
  const int mt = cdiv(Mtot, BM), nt = cdiv(Ntot, BN);
  const int total = args.E * mt * nt;
  // XCD x (workgroups are dealt to the 8 XCDs round-robin) takes a contiguous
  // range of the tile list; its workgroups interleave over that range, so
  // the tiles running at one time on an XCD are neighbours sharing operands
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslot = gridDim.x >> 3;
  // m-groups: mt split evenly into the group count nearest mt / sqrt(nslot
  // mt / nt), which makes the block of concurrent tiles about as wide in m
  // as in n (Qwen3-235B shape: groups of 6 of dW_gate|up's 12 m-tiles, 2.36
  // -> 2.33 ms against the 4 of a power-of-two rule; 8 of dW_down's 16)
  const float gm_target = sqrtf((float)nslot * (float)mt / (float)nt);
  const int n_groups = max(1, (int)lrintf((float)mt / gm_target));
  const int gm = (mt + n_groups - 1) / n_groups;
  const int per = (total + 7) >> 3;
  const int t_begin = xcd * per + slot;
  const int t_end = min(total, (xcd + 1) * per);
  if (t_begin >= t_end) return;                 // uniform: no tiles for this workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const bool load_a = wave < 4;
  const int blk0 = (wave & 3) * BPW;
  const int lds_op = load_a ? 0 : OPB;
  const long long lda = MODE == BWD_WD ? args.d : 2LL * args.F;   // A: dY or dg | du rows
  const long long ldb = MODE == BWD_WD ? args.F : (long long)args.d;   // B: h or x_perm rows
  const long long ld = load_a ? lda : ldb;
  const bf16_t* opnd = static_cast<const bf16_t*>(
      load_a ? (MODE == BWD_WD ? args.dY : args.dgu) : (MODE == BWD_WD ? args.h : args.x_perm));
  // per lane, block j of a slice holds k-row 2 (blk0 + j) + lane / 32 and the
  // 16-byte column chunk (lane % 32) ^ 4 (k-row % 4) (computed where used:
  // arrays of them indexed in a loop the compiler keeps rolled go to scratch)

  // ---- the slice stream: tile t_begin + i nslot, its K slices in order,
  // tiles without rows skipped -------------------------------------------
  // The expert offsets are read through the constant address space with a
  // scalar index: scalar loads, counted by lgkmcnt.  As vector loads the
  // compiler's own wait for them would be a vmcnt(0) that drains every DMA
  // in flight (it cannot see the loads issued in inline assembly).
  const __attribute__((address_space(4))) int32_t* offs =
      (const __attribute__((address_space(4))) int32_t*)args.offsets;
  auto offset_of = [&](int e) { return offs[__builtin_amdgcn_readfirstlane(e)]; };
  // The issue cursor: tile is_t (decoded only when the cursor reaches it),
  // slice is_s of its is_KT.  Within a tile a lane's DMA offsets stay fixed
  // (column chunk and k-row within the slice) and the scalar base advances
  // by one slice per issue; only a last, partial slice clamps its k-rows.
  int is_t = t_begin, is_s = 0, is_K = 0, is_KT = 0;
  const char* is_base = nullptr;                // k-row 32 is_s of the tile's operand block
  uint32_t goff0 = 0, goff1 = 0, goff2 = 0, goff3 = 0;
  int is_mn0 = 0;
  const uint32_t slice_bytes = (uint32_t)(BK * ld * 2);
  auto lane_off = [&](int j, int mn0, int kmax) {
    const int krs = 2 * (blk0 + j) + (lane >> 5);
    const int ccol = (lane & 31) ^ (4 * (krs & 3));
    const int kr = krs < kmax ? krs : kmax - 1;
    return (uint32_t)(mn0 + ccol * 8) * 2u + (uint32_t)(kr * (int)ld) * 2u;
  };
  auto load_issue_tile = [&]() {                // from is_t on, the next tile with rows
    for (; is_t < t_end; is_t += nslot) {
      const int e = is_t / (mt * nt), r = is_t - e * (mt * nt);
      const int row0 = offset_of(e);
      is_K = offset_of(e + 1) - row0;
      if (is_K == 0) continue;
      is_KT = cdiv(is_K, BK);
      int mi, ni;
      wgrad_tile_mn(r, mt, nt, gm, mi, ni);
      is_mn0 = load_a ? mi * BM : ni * BN;
      // wave-uniform values the compiler cannot prove uniform: scalar copies
      is_base = uniform_ptr(opnd + (long long)row0 * ld);
      goff0 = lane_off(0, is_mn0, BK);
      goff1 = lane_off(1, is_mn0, BK);
      goff2 = lane_off(2, is_mn0, BK);
      goff3 = lane_off(3, is_mn0, BK);
      return;
    }
  };
  load_issue_tile();
  int issued = 0;                               // slices issued so far
  // `issued` at the last three epilogues (-1: none): an epilogue's stores
  // are younger than slice g exactly when it ran with issued > g
  int ep0 = -1, ep1 = -1, ep2 = -1;
  const uint32_t lds_wave = (uint32_t)(uintptr_t)MOE_AS_LDS(reinterpret_cast<char*>(ring)) +
                            (uint32_t)(lds_op + blk0 * 1024);
  auto issue_one = [&]() {
    if (is_t >= t_end) return;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_wave + (uint32_t)(issued & 3) * (STAGE * 2));
    uint32_t o0 = goff0, o1 = goff1, o2 = goff2, o3 = goff3;
    if (__builtin_amdgcn_readfirstlane((is_s + 1) * BK > is_K)) {
      // a partial last slice: k-rows past the tile's end read its last row
      // (their A values are zeroed before use)
      const int kmax = is_K - is_s * BK;
      o0 = lane_off(0, is_mn0, kmax);
      o1 = lane_off(1, is_mn0, kmax);
      o2 = lane_off(2, is_mn0, kmax);
      o3 = lane_off(3, is_mn0, kmax);
    }
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds0), "v"(o0), "s"(is_base) : "memory");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds0 + 1024), "v"(o1), "s"(is_base) : "memory");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds0 + 2048), "v"(o2), "s"(is_base) : "memory");
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :: "s"(lds0 + 3072), "v"(o3), "s"(is_base) : "memory");
    ++issued;
    if (++is_s == is_KT) {
      is_s = 0;
      is_t += nslot;
      load_issue_tile();
    } else {
      is_base = is_base + slice_bytes;
    }
  };
  // waits until this wave's loads of slice g have landed, leaving every
  // younger operation in flight: the slices issued after it, and the stores
  // of the epilogues since (counting at most three: a smaller count than
  // the true one only waits longer)
  auto wait_for = [&](int g) {
    const int ys = issued - 1 - g;
    const int ye = (ep0 > g ? 1 : 0) + (ep1 > g ? 1 : 0) + (ep2 > g ? 1 : 0);
    if (ye == 0) {                              // inside a tile: the common case
      if (ys >= 2) wait_vmcnt<2 * BPW>();
      else if (ys == 1) wait_vmcnt<BPW>();
      else wait_vmcnt<0>();
      return;
    }
    const int y = ys * BPW + ye * NST;
    if (y >= NST + 3 * BPW) wait_vmcnt<NST + 3 * BPW>();
    else if (y >= NST + 2 * BPW) wait_vmcnt<NST + 2 * BPW>();
    else if (y >= NST + BPW) wait_vmcnt<NST + BPW>();
    else if (y >= NST) wait_vmcnt<NST>();
    else if (y >= 2 * BPW) wait_vmcnt<2 * BPW>();
    else if (y >= BPW) wait_vmcnt<BPW>();
    else wait_vmcnt<0>();
  };

  // ---- fragments: both operands are column operands (read transposed) ---
  const int frag_row = lane & 31;
  const int tr_row = (8 * (lane >> 5) + ((lane & 15) >> 2)) * 512;
  const int tr_swz = 4 * ((lane & 15) >> 2);
  const int tr_c = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tr_half = (lane & 1) * 8;
  auto col_frag = [&](const char* op, int kk, int mcol0) -> bf16x8_t {
    const int c = (tr_c + (mcol0 >> 3)) ^ tr_swz;
    const char* p = op + kk * 16 * 512 + tr_row + (c << 4) + tr_half;
    const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)MOE_AS_LDS(p));
    const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)MOE_AS_LDS(p + 4 * 512));
    const auto v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  };
  auto load_frags = [&](const bf16_t* stage, int kk, bf16x8_t (&af)[MI], bf16x8_t (&bfr)[NJ]) {
    const char* sa = reinterpret_cast<const char*>(stage);
    const char* sb = sa + OPB;
#pragma unroll
    for (int i = 0; i < MI; ++i) af[i] = col_frag(sa, kk, wm * WTM + i * 32);
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[j] = col_frag(sb, kk, wn * WTN + j * 32);
  };
  f32x16_t acc[MI][NJ];
  auto mma = [&](const bf16x8_t (&af)[MI], const bf16x8_t (&bfr)[NJ]) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
  };
  auto mask_tail = [&](bf16x8_t (&af)[MI], int s, int kk, int K) {
    const int k0 = s * BK + kk * 16 + 8 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k0 + e >= K) af[i][e] = (__bf16)0.0f;
  };
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  constexpr int NREAD = 2 * MI + 2 * NJ;        // LDS reads per half-step
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD - (MI * NJ - 1), 0);
#pragma unroll
    for (int r = 0; r < MI * NJ - 1; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
  };

  // ---- the epilogue: one 32 x 32 block at a time through the wave's 4 KiB
  float* sw = stg[wave];
  auto epilogue = [&](int e_, int m0_, int n0_) {
    // The tile's output block, from scalars the compiler cannot see through:
    // otherwise it hoists the 32 store addresses out of the K loop and keeps
    // them live across it (spilling).  Tiles never straddle dW_gate and
    // dW_up (F is a multiple of 256 here).
    uint32_t e = __builtin_amdgcn_readfirstlane(e_);
    uint32_t m0 = __builtin_amdgcn_readfirstlane(m0_);
    uint32_t n0 = __builtin_amdgcn_readfirstlane(n0_);
    asm volatile("" : "+s"(e), "+s"(m0), "+s"(n0));
    const bool up = MODE == BWD_WGU && (int)m0 >= args.F;
    const long long per_e = (long long)(MODE == BWD_WD ? args.d : args.F) * Ntot;
    const long long blk = (long long)e * per_e +
                          (long long)((int)m0 - (up ? args.F : 0) + wm * WTM) * Ntot +
                          (int)n0 + wn * WTN;
    void* const wbase = MODE == BWD_WD ? args.dw_down : (up ? args.dw_up : args.dw_gate);
    // Per 32 x 32 block: the four staging writes, then the four row reads,
    // then the four global stores, so the reads return together and each
    // store waits only for its own.  The staging buffer is reused by the
    // next block without a wait (a wave's LDS operations complete in order).
    // The output type is one uniform branch around the whole loop.
    auto blocks = [&](auto store4) __attribute__((always_inline)) {
      static_for<MI * NJ>([&](auto ijc) __attribute__((always_inline)) {
          constexpr int i = decltype(ijc)::value / NJ, j = decltype(ijc)::value % NJ;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = 2 * q + (lane >> 5);
            const int pos = ch ^ ((frag_row >> 1) & 7);
            *reinterpret_cast<float4*>(sw + frag_row * 32 + pos * 4) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
          }
          float4 v4[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = (lane >> 3) + 8 * t, ch = lane & 7;
            v4[t] = *reinterpret_cast<const float4*>(sw + r * 32 + ((ch ^ ((r >> 1) & 7)) * 4));
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = (lane >> 3) + 8 * t, ch = lane & 7;
            store4(blk + (long long)(i * 32 + r) * Ntot + j * 32 + ch * 4, v4[t]);
          }
      });
    };
    if (args.wgrad_bf16) {
      // bf16 gradients: half the bytes, and faster through L2 than around it
      blocks([&](long long o, const float4& v) __attribute__((always_inline)) {
        *reinterpret_cast<uint2*>(static_cast<bf16_t*>(wbase) + o) =
            make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      });
    } else {
      // fp32 gradients (the largest write of the backward) bypass L2 so they
      // do not evict the operand slices other tiles still read
      blocks([&](long long o, const float4& v) __attribute__((always_inline)) {
        typedef float f4_t __attribute__((ext_vector_type(4)));
        const f4_t q = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(q, reinterpret_cast<f4_t*>(static_cast<float*>(wbase) + o));
      });
    }
    ep2 = ep1;
    ep1 = ep0;
    ep0 = issued;
  };

  // ---- the tiles ----------------------------------------------------------
  for (int j = 0; j < 3; ++j) issue_one();
  int consumed = 0;                             // slices consumed so far
  bf16x8_t af0[MI], af1[MI], bf0[NJ], bf1[NJ];
  for (int t = t_begin; t < t_end; t += nslot) {
    const int e = t / (mt * nt), r = t - e * (mt * nt);
    int mi, ni;
    wgrad_tile_mn(r, mt, nt, gm, mi, ni);
    const int m0 = mi * BM, n0 = ni * BN;
    const int K = offset_of(e + 1) - offset_of(e);
    const int KT = cdiv(K, BK);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j2 = 0; j2 < NJ; ++j2)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j2][v] = 0.0f;
    if (KT > 0) {
      // the tile's first slice: landed and visible to every wave
      wait_for(consumed);
      barrier();
      load_frags(ring + (consumed & 3) * STAGE, 0, af0, bf0);
      const bool tail = (K % BK) != 0;
      for (int s = 0; s < KT; ++s, ++consumed) {
        const bf16_t* cur = ring + (consumed & 3) * STAGE;
        const bf16_t* nxt = ring + ((consumed + 1) & 3) * STAGE;
        const bool last = s == KT - 1;
        const bool tail_step = __builtin_amdgcn_readfirstlane(tail && last);
        if (tail_step) mask_tail(af0, s, 0, K);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, 1, af1, bf1);
        mma(af0, bf0);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
        if (consumed + 1 < issued) wait_for(consumed + 1);
        barrier();
        issue_one();                            // slice consumed + 3, of this tile or a later one
        if (tail_step) mask_tail(af1, s, 1, K);
        __builtin_amdgcn_sched_barrier(0);
        // (in the tile's last step these read the next slice in the stream,
        // or a stale stage: one code path for every step, since a branch
        // here made the compiler copy the accumulators through scratch; the
        // next tile reads its first fragments again after its barrier)
        load_frags(nxt, 0, af0, bf0);
        mma(af1, bf1);
        interleave();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    epilogue(e, m0, n0);
  }
  wait_vmcnt<0>();
}

static bool bwd_uses_dma(const moe_shape& s) {
  return s.dtype == MOE_DTYPE_BF16 && s.d % 256 == 0 && s.F % 256 == 0;
}

static bool bwd_uses_mfma(const moe_shape& s) {
  return s.dtype == MOE_DTYPE_BF16 && s.d % 128 == 0 && s.F % 128 == 0;
}

// Compute units of the current device (cached per device; the persistent
// weight-gradient kernel launches one workgroup per CU).
static int device_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// FLAVOR: 0 generic, 1 MFMA with register transposes, 2 direct-to-LDS MFMA
// (the weight gradients persistent, one workgroup per CU)
template <int MODE, typename T, int FLAVOR>
static void launch_bwd_gemm(const moe_shape& s, const BwdArgs& a, hipStream_t st) {
  if constexpr (FLAVOR == 2 && (MODE == BWD_WD || MODE == BWD_WGU)) {
    if (s.E > 0) {
      const long long tiles = MODE == BWD_WD ? (long long)s.E * cdiv(s.d, 256) * cdiv(s.F, 256)
                                             : (long long)s.E * cdiv(2 * s.F, 256) * cdiv(s.d, 256);
      const long long cap = ((tiles + 7) / 8) * 8;
      const int grid = (int)std::min<long long>(cap, device_cus() / 8 * 8);
      bwd_wgrad_kernel<MODE><<<grid, 512, 0, st>>>(a);
    }
  } else {
    constexpr int BM = FLAVOR == 2 ? 256 : FLAVOR == 1 ? 128 : 64;
    constexpr int BN = BM;
    const long long R = (long long)s.T * s.k;
    // (with tail tiles a group's tiles are at most its 256-row tiles' count)
    long long tiles;
    if (MODE == BWD_DH) tiles = (cdiv((int)R, BM) + s.E) * (long long)cdiv(s.F, BN);
    else if (MODE == BWD_DX) tiles = (cdiv((int)R, BM) + s.E) * (long long)cdiv(s.d, BN);
    else if (MODE == BWD_WD) tiles = (long long)s.E * cdiv(s.d, BM) * cdiv(s.F, BN);
    else tiles = (long long)s.E * cdiv(2 * s.F, BM) * cdiv(s.d, BN);
    const int grid = (int)(((tiles + 7) / 8) * 8);
    if (grid == 0) return;
    if constexpr (FLAVOR == 2) bwd_dma_kernel<MODE><<<grid, 512, 0, st>>>(a);
    else if constexpr (FLAVOR == 1) bwd_mfma_kernel<MODE><<<grid, 256, 0, st>>>(a);
    else bwd_generic_kernel<MODE, T><<<grid, 256, 0, st>>>(a);
  }
}

// One backward GEMM launch, bracketed by its phase events when `marks`.
template <int MODE, typename T, int FLAVOR>
static void launch_bwd_phase(const moe_shape& s, const BwdArgs& a, hipStream_t st, bool marks) {
  constexpr int PHASE = MODE == BWD_DH ? MOE_PHASE_BWD_DH : MODE == BWD_WD ? MOE_PHASE_BWD_DW_DOWN
                        : MODE == BWD_DX ? MOE_PHASE_BWD_DX : MOE_PHASE_BWD_DW_GATE_UP;
  if (marks) phase_mark(PHASE, 0, st);
  launch_bwd_gemm<MODE, T, FLAVOR>(s, a, st);
  if (marks) phase_mark(PHASE, 1, st);
}

template <typename T, int FLAVOR>
static hipError_t run_backward(const moe_shape& s, BwdArgs& a, const BwdWs& ws, hipStream_t st,
                               bool marks) {
  constexpr int BM = FLAVOR == 2 ? 256 : FLAVOR == 1 ? 128 : 64, BN = BM;
  // tile prefixes of the two row-grouped GEMMs (N = F for dh, N = d for dX)
  schedule_tiles_kernel<<<1, 1024, 0, st>>>(a.offsets, s.E, BM, cdiv(s.F, BN), ws.tiles, BM,
                                            cdiv(s.d, BN), ws.tiles2, FLAVOR == 2 ? 1 : 0);
  a.tiles = ws.tiles;
  launch_bwd_phase<BWD_DH, T, FLAVOR>(s, a, st, marks);
  launch_bwd_phase<BWD_WD, T, FLAVOR>(s, a, st, marks);
  a.tiles = ws.tiles2;
  launch_bwd_phase<BWD_DX, T, FLAVOR>(s, a, st, marks);
  launch_bwd_phase<BWD_WGU, T, FLAVOR>(s, a, st, marks);
  return hipGetLastError();
}

// Zeroes n 16-bit elements (bf16 weight gradients with no tokens to sum).
__global__ void __launch_bounds__(256) zero_u16_kernel(uint16_t* __restrict__ p, long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
    p[i] = 0;
}

// A weight gradient summed over no tokens: zero, in fp32 or bf16.
static hipError_t zero_wgrad(void* p, long long n, bool bf16, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (!bf16) return launch_zero_f32(static_cast<float*>(p), n, st);
  zero_u16_kernel<<<(int)std::min<long long>((n + 255) / 256, 4096), 256, 0, st>>>(
      static_cast<uint16_t*>(p), n);
  return hipGetLastError();
}

// {0, n}: the row offsets of a single group of n rows.
__global__ void one_group_offsets_kernel(int32_t* offsets, int n) {
  if (threadIdx.x == 0) {
    offsets[0] = 0;
    offsets[1] = n;
  }
}

// marks: bracket the kernels with the phase events (the routed group only).
static hipError_t run_backward_any(const moe_shape& s, BwdArgs& a, const BwdWs& ws,
                                   hipStream_t st, bool marks) {
  const bool bf = s.dtype == MOE_DTYPE_BF16;
  if (bf && bwd_uses_dma(s)) return run_backward<bf16_t, 2>(s, a, ws, st, marks);
  if (bf && bwd_uses_mfma(s)) return run_backward<bf16_t, 1>(s, a, ws, st, marks);
  if (bf) return run_backward<bf16_t, 0>(s, a, ws, st, marks);
  return run_backward<float, 0>(s, a, ws, st, marks);
}

// The weight-gradient GEMMs alone (bf16), after data gradients computed
// elsewhere (the MXFP8 path) have written h and dg | du.
static hipError_t run_wgrad_any(const moe_shape& s, const BwdArgs& a, hipStream_t st,
                                bool marks) {
  if (bwd_uses_dma(s)) {
    launch_bwd_phase<BWD_WD, bf16_t, 2>(s, a, st, marks);
    launch_bwd_phase<BWD_WGU, bf16_t, 2>(s, a, st, marks);
  } else if (bwd_uses_mfma(s)) {
    launch_bwd_phase<BWD_WD, bf16_t, 1>(s, a, st, marks);
    launch_bwd_phase<BWD_WGU, bf16_t, 1>(s, a, st, marks);
  } else {
    launch_bwd_phase<BWD_WD, bf16_t, 0>(s, a, st, marks);
    launch_bwd_phase<BWD_WGU, bf16_t, 0>(s, a, st, marks);
  }
  return hipGetLastError();
}

// The two weight-gradient GEMMs on MXFP8 operands quantised along each
// group's rows (the shape's wgrad_mx): dW_down = dY^T . h, then
// [dW_gate | dW_up] = [dg | du]^T . x, reusing the quantised-operand buffers.
static hipError_t run_mx_wgrad(const moe_shape& s, const BwdArgs& a, const BwdWs& ws, int groups,
                               const int32_t* offsets, hipStream_t st, bool marks) {
  MxWgrad g = {};
  g.E = groups;
  g.offsets = offsets;
  g.poffs = groups == 1 ? ws.s_poffs : ws.poffs;
  g.qa = ws.wqa;
  g.sa = ws.wsa;
  g.qb = ws.wqb;
  g.sb = ws.wsb;
  g.wrows = ws.wrows;
  g.wbf16 = a.wgrad_bf16;
  g.M = a.d;
  g.N = a.F;
  g.A = a.dY;
  g.B = a.h;
  g.w0 = a.dw_down;
  g.w1 = a.dw_down;
  g.wsplit = a.d;
  if (marks) phase_mark(MOE_PHASE_BWD_DW_DOWN, 0, st);
  hipError_t e = launch_mx_wgrad(g, st);
  if (marks) phase_mark(MOE_PHASE_BWD_DW_DOWN, 1, st);
  if (e != hipSuccess) return e;
  g.M = 2 * a.F;
  g.N = a.d;
  g.A = a.dgu;
  g.B = a.x_perm;
  g.w0 = a.dw_gate;
  g.w1 = a.dw_up;
  g.wsplit = a.F;
  if (marks) phase_mark(MOE_PHASE_BWD_DW_GATE_UP, 0, st);
  e = launch_mx_wgrad(g, st);
  if (marks) phase_mark(MOE_PHASE_BWD_DW_GATE_UP, 1, st);
  return e;
}

hipError_t launch_backward(const moe_shape& s, const void* dy, const void* x_perm,
                           const void* gu_save, const void* y_perm, const int32_t* offsets,
                           const int32_t* row_token, const int32_t* token_row,
                           const int32_t* topk_idx, const float* topk_w,
                           const float* logits, const void* w_gate, const void* w_up,
                           const void* w_down, const void* x, const void* ws_gate,
                           const void* ws_up, const void* ws_down, float* dx, void* dw_gate,
                           void* dw_up, void* dw_down, void* dws_gate, void* dws_up,
                           void* dws_down, float* d_gate, float* d_logits,
                           const BwdWs& ws, hipStream_t st, const MxBwdWeights* mx) {
  (void)row_token;
  const bool bf = s.dtype == MOE_DTYPE_BF16;
  phase_mark(MOE_PHASE_BWD_DISPATCH, 0, st);
  if (s.T > 0) {
    if (bf)
      with_gather_batch(s.k, [&](auto jb) {
        bwd_dispatch_kernel<bf16_t, decltype(jb)::value><<<s.T, 256, 0, st>>>(
            static_cast<const bf16_t*>(dy), static_cast<const bf16_t*>(y_perm), token_row,
            topk_idx, topk_w, logits, s.d, s.E, s.k, s.score, s.renorm,
            static_cast<bf16_t*>(ws.dY), d_gate, d_logits);
      });
    else
      bwd_dispatch_kernel<float, 1><<<s.T, 256, 0, st>>>(
          static_cast<const float*>(dy), static_cast<const float*>(y_perm), token_row, topk_idx,
          topk_w, logits, s.d, s.E, s.k, s.score, s.renorm, static_cast<float*>(ws.dY), d_gate,
          d_logits);
  }
  phase_mark(MOE_PHASE_BWD_DISPATCH, 1, st);
  BwdArgs a = {};
  a.E = s.E;
  a.F = s.F;
  a.d = s.d;
  a.offsets = offsets;
  a.dY = ws.dY;
  a.gu = gu_save;
  a.dgu = ws.dgu;
  a.h = ws.h;
  a.x_perm = x_perm;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  a.out_dgu = ws.dgu;
  a.out_h = ws.h;
  a.out_dX = ws.dX;
  a.dw_down = dw_down;
  a.dw_gate = dw_gate;
  a.wgrad_bf16 = s.wgrad_dtype == MOE_DTYPE_BF16;
  a.dw_up = dw_up;
  const int R = s.T * s.k;
  hipError_t e;
  if (mx) {
    // MXFP8 data gradients: dY_perm quantised along d, then dh (with the
    // SwiGLU backward) and dX on the quantised operands; bf16 weight gradients
    if ((e = launch_mx_quantize(ws.dY, R, s.d, ws.dyq, ws.dys, st)) != hipSuccess) return e;
    MxDgrad g = {R, offsets, ws.tiles, ws.tiles2, ws.dyq, ws.dys, mx->wd_tq, mx->wd_ts,
                 gu_save, ws.dgu, ws.h, ws.dguq, ws.dgus, mx->wgu_tq, mx->wgu_ts, ws.dX};
    if ((e = launch_mx_dgrad(s, g, st)) != hipSuccess) return e;
    e = s.wgrad_mx ? run_mx_wgrad(s, a, ws, s.E, offsets, st, true)
                   : run_wgrad_any(s, a, st, true);
  } else {
    e = run_backward_any(s, a, ws, st, true);
  }
  if (e != hipSuccess) return e;
  const bool shared = s.F_shared > 0 && s.T > 0;
  if (s.F_shared > 0 && s.T == 0) {
    // no tokens: the shared expert's weight gradients are empty sums
    const long long n = (long long)s.F_shared * s.d;
    if ((e = zero_wgrad(dws_gate, n, a.wgrad_bf16, st)) != hipSuccess) return e;
    if ((e = zero_wgrad(dws_up, n, a.wgrad_bf16, st)) != hipSuccess) return e;
    if ((e = zero_wgrad(dws_down, n, a.wgrad_bf16, st)) != hipSuccess) return e;
  }
  if (shared) {
    // The shared expert: one group of all T tokens with gate 1, so dY = dy,
    // its input is x and its saved g | u follow the routed rows in gu_save.
    one_group_offsets_kernel<<<1, 64, 0, st>>>(ws.s_offsets, s.T);
    moe_shape s2 = s;
    s2.E = 1;
    s2.k = 1;
    s2.F = s.F_shared;
    s2.F_shared = 0;
    const size_t es = bf ? 2 : 4;
    BwdArgs b = {};
    b.E = 1;
    b.F = s.F_shared;
    b.d = s.d;
    b.offsets = ws.s_offsets;
    b.dY = dy;
    b.gu = static_cast<const char*>(gu_save) + (size_t)s.T * s.k * 2 * s.F * es;
    b.dgu = ws.s_dgu;
    b.h = ws.s_h;
    b.x_perm = x;
    b.w_gate = ws_gate;
    b.w_up = ws_up;
    b.w_down = ws_down;
    b.out_dgu = ws.s_dgu;
    b.out_h = ws.s_h;
    b.out_dX = ws.s_dX;
    b.dw_down = dws_down;
    b.dw_gate = dws_gate;
    b.dw_up = dws_up;
    b.wgrad_bf16 = a.wgrad_bf16;
    BwdWs w2 = ws;
    w2.tiles = ws.s_tiles;
    w2.tiles2 = ws.s_tiles2;
    if (mx) {
      if ((e = launch_mx_quantize(dy, s.T, s.d, ws.s_dyq, ws.s_dys, st)) != hipSuccess) return e;
      MxDgrad g = {s.T, ws.s_offsets, ws.s_tiles, ws.s_tiles2, ws.s_dyq, ws.s_dys,
                   mx->swd_tq, mx->swd_ts, b.gu, ws.s_dgu, ws.s_h, ws.s_dguq, ws.s_dgus,
                   mx->swgu_tq, mx->swgu_ts, ws.s_dX};
      if ((e = launch_mx_dgrad(s2, g, st)) != hipSuccess) return e;
      if ((e = s.wgrad_mx ? run_mx_wgrad(s2, b, ws, 1, ws.s_offsets, st, false)
                          : run_wgrad_any(s2, b, st, false)) != hipSuccess)
        return e;
    } else if ((e = run_backward_any(s2, b, w2, st, false)) != hipSuccess) {
      return e;
    }
  }
  phase_mark(MOE_PHASE_BWD_GATHER, 0, st);
  if (s.T > 0) {
    if (bf)
      with_gather_batch(s.k, [&](auto jb) {
        bwd_gather_kernel<bf16_t, decltype(jb)::value><<<s.T, 256, 0, st>>>(
            static_cast<const bf16_t*>(ws.dX), token_row, s.d, s.k,
            shared ? static_cast<const bf16_t*>(ws.s_dX) : nullptr, dx);
      });
    else
      bwd_gather_kernel<float, 1><<<s.T, 256, 0, st>>>(
          static_cast<const float*>(ws.dX), token_row, s.d, s.k,
          shared ? static_cast<const float*>(ws.s_dX) : nullptr, dx);
  }
  phase_mark(MOE_PHASE_BWD_GATHER, 1, st);
  return hipGetLastError();
}

}  // namespace moe
