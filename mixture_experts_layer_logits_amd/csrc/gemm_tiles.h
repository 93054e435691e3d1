// Grouped "NT" GEMM tiles for the expert FFN and the router (gfx950).
//
//   C[m, n] = sum_k A[m, k] * B[n, k]      (both operands K-contiguous)
//
// over a list of groups: the routed experts, whose row ranges live in a
// device array of offsets (so the host never learns the per-expert counts),
// and at most one dense group whose row count is known on the host (the
// shared expert, or the router GEMM).  A small schedule kernel turns the
// offsets into a prefix of tile counts; each workgroup finds its tile with a
// binary search over that prefix.  The grid is sized from the host-side upper
// bound ceil(R / BM) + E row tiles per column tile, and surplus workgroups
// exit at once.
//
// Tile order: within a group, the row tiles of one column tile are adjacent,
// so workgroups that share a weight tile run together.  The workgroup id is
// remapped so that each XCD (workgroups are dealt to the 8 XCDs round-robin)
// walks a contiguous range of the tile list, keeping those neighbours in one
// L2.
#pragma once

#include <type_traits>

#include "moe_common.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_F32_BIAS = 2 };

struct GemmArgs {
  // routed groups (E == 0: none)
  int E;
  const int32_t* offsets;  // [E + 1] row offsets of the groups
  const int32_t* tiles;    // [E + 1] exclusive prefix of the groups' tile counts
  const void* A;           // group g owns rows offsets[g] .. offsets[g+1]-1
  long long lda;
  const void* B0;          // [E][N][K]
  const void* B1;          // second B (FC1 up), same layout, or null
  long long strideB;       // elements between experts
  int N, K;
  void* C;                 // rows as A
  long long ldc;
  void* GU;                // FC1 only, or null: g saved at column n, u at N + n
  long long ldgu;
  // dense group (Td == 0: none)
  int Td;
  const void* Ad;
  long long ldad;
  const void* Bd0;
  const void* Bd1;
  int Nd, Kd;
  void* Cd;
  long long ldcd;
  const float* bias;       // EPI_F32_BIAS: added per column, or null
};

// One tile's work, with typed base pointers already offset to the group.
template <typename TIn, typename TOut>
struct TileJob {
  const TIn* A;
  long long lda;
  int rows;
  const TIn* B0;
  const TIn* B1;
  int N, K;
  TOut* C;
  long long ldc;
  TOut* GU;
  long long ldgu;
  int m0, n0;
};

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Upper bound of the tile count, known on the host (a multiple of 8).
inline int grid_upper_bound(const GemmArgs& a, int BM, int BN, int R) {
  long long t = 0;
  if (a.E > 0) t += (long long)(cdiv(R, BM) + a.E) * cdiv(a.N, BN);
  if (a.Td > 0) t += (long long)cdiv(a.Td, BM) * cdiv(a.Nd, BN);
  return (int)(((t + 7) / 8) * 8);
}

// Maps blockIdx.x to a tile.  Returns false for surplus workgroups.
template <int BM, int BN, typename TIn, typename TOut>
__device__ __forceinline__ bool decode_tile(const GemmArgs& a, TileJob<TIn, TOut>& j) {
  const int routed = (a.E > 0) ? a.tiles[a.E] : 0;
  const int dmt = cdiv(a.Td, BM);
  const int dense = (a.Td > 0) ? dmt * cdiv(a.Nd, BN) : 0;
  const int total = routed + dense;
  const int bid = blockIdx.x;
  const int per = (total + 7) >> 3;
  const int slot = bid >> 3;
  if (slot >= per) return false;
  const int lid = (bid & 7) * per + slot;
  if (lid >= total) return false;
  if (lid < routed) {
    // largest g with tiles[g] <= lid (empty groups share their start)
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tiles[mid] <= lid) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int row0 = a.offsets[g];
    const int rows = a.offsets[g + 1] - row0;
    const int mt = cdiv(rows, BM);
    const int r = lid - a.tiles[g];
    j.m0 = (r % mt) * BM;
    j.n0 = (r / mt) * BN;
    j.rows = rows;
    j.N = a.N;
    j.K = a.K;
    j.lda = a.lda;
    j.ldc = a.ldc;
    j.ldgu = a.ldgu;
    j.A = static_cast<const TIn*>(a.A) + (long long)row0 * a.lda;
    j.B0 = static_cast<const TIn*>(a.B0) + (long long)g * a.strideB;
    j.B1 = a.B1 ? static_cast<const TIn*>(a.B1) + (long long)g * a.strideB : nullptr;
    j.C = static_cast<TOut*>(a.C) + (long long)row0 * a.ldc;
    j.GU = a.GU ? static_cast<TOut*>(a.GU) + (long long)row0 * a.ldgu : nullptr;
    return true;
  }
  const int r = lid - routed;
  j.m0 = (r % dmt) * BM;
  j.n0 = (r / dmt) * BN;
  j.rows = a.Td;
  j.N = a.Nd;
  j.K = a.Kd;
  j.lda = a.ldad;
  j.ldc = a.ldcd;
  j.ldgu = 0;
  j.A = static_cast<const TIn*>(a.Ad);
  j.B0 = static_cast<const TIn*>(a.Bd0);
  j.B1 = static_cast<const TIn*>(a.Bd1);
  j.C = static_cast<TOut*>(a.Cd);
  j.GU = nullptr;
  return true;
}

// ---------------------------------------------------------------------------
// Schedule: tiles[g] = sum_{g' < g} ceil(rows_g' / BM) * NT, for two GEMMs at
// once.  One workgroup of 1024 threads (E <= 1024).
// ---------------------------------------------------------------------------
namespace {
__global__ void __launch_bounds__(1024)
schedule_tiles_kernel(const int32_t* __restrict__ offsets, int E, int bm1, int nt1,
                      int32_t* __restrict__ tiles1, int bm2, int nt2,
                      int32_t* __restrict__ tiles2) {
  __shared__ int s1[1024];
  __shared__ int s2[1024];
  const int g = threadIdx.x;
  int v1 = 0, v2 = 0;
  if (g < E) {
    const int rows = offsets[g + 1] - offsets[g];
    v1 = cdiv(rows, bm1) * nt1;
    v2 = tiles2 ? cdiv(rows, bm2) * nt2 : 0;
  }
  s1[g] = v1;
  s2[g] = v2;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a1 = (g >= off) ? s1[g - off] : 0;
    const int a2 = (g >= off) ? s2[g - off] : 0;
    __syncthreads();
    s1[g] += a1;
    s2[g] += a2;
    __syncthreads();
  }
  // inclusive -> exclusive, plus the total at index E
  if (g <= E) {
    tiles1[g] = (g == 0) ? 0 : s1[g - 1];
    if (tiles2) tiles2[g] = (g == 0) ? 0 : s2[g - 1];
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// bf16 MFMA tile kernel.
//
// WM x WN waves (64 threads each) tile the BM x BN output (per B matrix);
// each wave owns a (BM/WM) x (BN/WN) block made of 32 x 32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16, fp32 accumulators).  K advances 64 at a time
// through two LDS stages: while the waves consume stage s, the next K slice
// is fetched from global memory into registers and then written to stage
// s^1, so one barrier per K step suffices.  LDS rows are padded by 16 bytes
// so that the 16-byte fragment reads of consecutive rows fall in different
// banks.  The LDS is dynamic: 2 * (BM + NB*BN) * 72 * 2 bytes.
//
// The MFMA is issued with the weight fragment as its first operand, so each
// lane ends up owning one token row and runs of 4 consecutive output columns
// (8-byte stores of bf16, 16-byte stores of fp32).
// ---------------------------------------------------------------------------
template <int BM, int BN, int NB>
constexpr int mfma_lds_bytes() { return 2 * (BM + NB * BN) * (64 + 8) * 2; }

template <int BM, int BN, int NB, int EPI, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_bf16_mfma_kernel(const GemmArgs args) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BK = 64;
  constexpr int LDK = BK + 8;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NJ = WTN / 32;
  constexpr int RPP = NT / 8;                   // rows per pass of 16-byte chunks
  constexpr int A_CH = BM / RPP;                // chunks per thread
  constexpr int B_CH = NB * BN / RPP;
  constexpr int STAGE = (BM + NB * BN) * LDK;   // elements per LDS stage
  static_assert(A_CH >= 1 && B_CH >= 1 && MI >= 1 && NJ >= 1, "tile too small");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be whole passes");
  using TOut = typename std::conditional<EPI == EPI_F32_BIAS, float, bf16_t>::type;

  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];

  TileJob<bf16_t, TOut> job;
  if (!decode_tile<BM, BN>(args, job)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Global -> LDS mapping: chunk i of a thread covers row tid / 8 + RPP i and
  // columns (tid % 8) * 8 .. +7 of the BK-wide slice.  Out-of-range rows are
  // clamped to the last valid row (their results are never stored).
  const int kc = (tid & 7) * 8;
  const int r0 = tid >> 3;
  int a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    int m = job.m0 + r0 + RPP * i;
    m = m < job.rows ? m : job.rows - 1;
    a_off[i] = m * (int)job.lda + kc;
  }
  int b_off[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int r = r0 + RPP * i;
    int n = job.n0 + (r % BN);
    n = n < job.N ? n : job.N - 1;
    b_off[i] = n * job.K + kc;
  }
  const bf16_t* const A = job.A;
  const bf16_t* const B0 = job.B0;
  const bf16_t* const B1 = NB > 1 ? job.B1 : job.B0;

  u32x4_t ra[A_CH], rb[B_CH];
#define MOE_GLOAD(k0)                                                               \
  do {                                                                              \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                \
        ra[i] = *reinterpret_cast<const u32x4_t*>(A + a_off[i] + (k0));             \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                \
        rb[i] = *reinterpret_cast<const u32x4_t*>(((RPP * i) / BN == 0 ? B0 : B1) + \
                                                  b_off[i] + (k0));                 \
  } while (0)
#define MOE_LSTORE(stage)                                                           \
  do {                                                                              \
    bf16_t* sA_ = smem + (stage) * STAGE;                                           \
    bf16_t* sB_ = sA_ + BM * LDK;                                                   \
    _Pragma("unroll") for (int i = 0; i < A_CH; ++i)                                \
        *reinterpret_cast<u32x4_t*>(&sA_[(r0 + RPP * i) * LDK + kc]) = ra[i];       \
    _Pragma("unroll") for (int i = 0; i < B_CH; ++i)                                \
        *reinterpret_cast<u32x4_t*>(&sB_[(r0 + RPP * i) * LDK + kc]) = rb[i];       \
  } while (0)

  f32x16_t acc[NB][MI][NJ];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.0f;

  const int KT = job.K / BK;
  MOE_GLOAD(0);
  MOE_LSTORE(0);
  __syncthreads();
  const int frag_row = lane & 31;
  const int frag_k = (lane >> 5) * 8;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) MOE_GLOAD((kt + 1) * BK);
    const bf16_t* sA = smem + cur * STAGE;
    const bf16_t* sB = sA + BM * LDK;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8_t af[MI];
      bf16x8_t bfr[NB][NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            &sA[(wm * WTM + i * 32 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          bfr[b][j] = *reinterpret_cast<const bf16x8_t*>(
              &sB[(b * BN + wn * WTN + j * 32 + frag_row) * LDK + kk + frag_k]);
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
            acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b][j], af[i],
                                                                   acc[b][i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) MOE_LSTORE(cur ^ 1);
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_LSTORE

  // Epilogue.  Lane owns row m = .. + (lane % 32) and, for register v,
  // column n = .. + 8 (v / 4) + 4 (lane / 32) + v % 4.
#pragma unroll
  for (int i = 0; i < MI; ++i) {
    const int m = job.m0 + wm * WTM + i * 32 + frag_row;
    if (m >= job.rows) continue;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = job.n0 + wn * WTN + j * 32 + 8 * q + 4 * (lane >> 5);
        if constexpr (EPI == EPI_F32_BIAS) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o[r] = acc[0][i][j][4 * q + r] + ((args.bias && n + r < job.N) ? args.bias[n + r] : 0.0f);
          float* dst = job.C + (long long)m * job.ldc + n;
          if (n + 3 < job.N && (job.ldc & 3) == 0) {
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (n + r < job.N) dst[r] = o[r];
          }
        } else if constexpr (EPI == EPI_SWIGLU) {
          if (n >= job.N) continue;  // N is a multiple of 8 on this path
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = acc[0][i][j][4 * q + r];
            const float u = acc[NB - 1][i][j][4 * q + r];
            h[r] = silu_fast(g) * u;
          }
          uint2 pk = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          *reinterpret_cast<uint2*>(job.C + (long long)m * job.ldc + n) = pk;
          if (job.GU) {
            const f32x16_t& G = acc[0][i][j];
            const f32x16_t& U = acc[NB - 1][i][j];
            uint2 pg = make_uint2(pack_bf16x2(G[4 * q], G[4 * q + 1]),
                                  pack_bf16x2(G[4 * q + 2], G[4 * q + 3]));
            uint2 pu = make_uint2(pack_bf16x2(U[4 * q], U[4 * q + 1]),
                                  pack_bf16x2(U[4 * q + 2], U[4 * q + 3]));
            *reinterpret_cast<uint2*>(job.GU + (long long)m * job.ldgu + n) = pg;
            *reinterpret_cast<uint2*>(job.GU + (long long)m * job.ldgu + job.N + n) = pu;
          }
        } else {
          if (n >= job.N) continue;
          const f32x16_t& Cv = acc[0][i][j];
          uint2 pk = make_uint2(pack_bf16x2(Cv[4 * q], Cv[4 * q + 1]),
                                pack_bf16x2(Cv[4 * q + 2], Cv[4 * q + 3]));
          *reinterpret_cast<uint2*>(job.C + (long long)m * job.ldc + n) = pk;
        }
      }
    }
  }
}

// Host launcher of the MFMA kernel: sets the dynamic LDS limit (above the
// 64 KiB default) and sizes the grid from the host-side tile bound.
template <int BM, int BN, int NB, int EPI, int WM, int WN>
hipError_t launch_mfma_gemm(const GemmArgs& a, int R, hipStream_t st) {
  constexpr int lds = mfma_lds_bytes<BM, BN, NB>();
  const void* fn = reinterpret_cast<const void*>(&gemm_bf16_mfma_kernel<BM, BN, NB, EPI, WM, WN>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  const int grid = grid_upper_bound(a, BM, BN, R);
  if (grid == 0) return hipSuccess;
  gemm_bf16_mfma_kernel<BM, BN, NB, EPI, WM, WN><<<grid, 64 * WM * WN, lds, st>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Generic tile kernel: any shape, fp32 or bf16 storage, fp32 FMA.  Used for
// the fp32 layer and for shapes the MFMA kernel does not take (K or N not a
// multiple of 64 / 8).  64 x 64 tiles, K slices of 16 staged in LDS, 4 x 4
// outputs per thread per B matrix.
// ---------------------------------------------------------------------------
template <typename T, int NB, int EPI>
__global__ void __launch_bounds__(256)
gemm_generic_kernel(const GemmArgs args) {
  constexpr int BM = 64, BN = 64, BK = 16;
  using TOut = typename std::conditional<EPI == EPI_F32_BIAS, float, T>::type;
  __shared__ float sA[BK][BM + 4];
  __shared__ float sB[NB][BK][BN + 4];

  TileJob<T, TOut> job;
  if (!decode_tile<BM, BN>(args, job)) return;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;

  float acc[NB][4][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[b][i][jj] = 0.0f;

  const T* Bp[2] = {job.B0, NB > 1 ? job.B1 : job.B0};
  for (int k0 = 0; k0 < job.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int r = e / BK, kk = e % BK;
      const int m = job.m0 + r, k = k0 + kk;
      sA[kk][r] = (m < job.rows && k < job.K) ? to_f32<T>(job.A[(long long)m * job.lda + k]) : 0.0f;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + 256 * i;
        const int r = e / BK, kk = e % BK;
        const int n = job.n0 + r, k = k0 + kk;
        sB[b][kk][r] = (n < job.N && k < job.K) ? to_f32<T>(Bp[b][(long long)n * job.K + k]) : 0.0f;
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float bv[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) bv[jj] = sB[b][kk][tx * 4 + jj];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[b][i][jj] = fmaf(av[i], bv[jj], acc[b][i][jj]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = job.m0 + ty * 4 + i;
    if (m >= job.rows) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n = job.n0 + tx * 4 + jj;
      if (n >= job.N) continue;
      if constexpr (EPI == EPI_F32_BIAS) {
        job.C[(long long)m * job.ldc + n] = acc[0][i][jj] + (args.bias ? args.bias[n] : 0.0f);
      } else if constexpr (EPI == EPI_SWIGLU) {
        const float g = acc[0][i][jj], u = acc[NB - 1][i][jj];
        job.C[(long long)m * job.ldc + n] = from_f32<TOut>(silu_precise(g) * u);
        if (job.GU) {
          job.GU[(long long)m * job.ldgu + n] = from_f32<TOut>(g);
          job.GU[(long long)m * job.ldgu + job.N + n] = from_f32<TOut>(u);
        }
      } else {
        job.C[(long long)m * job.ldc + n] = from_f32<TOut>(acc[0][i][jj]);
      }
    }
  }
}

}  // namespace moe
