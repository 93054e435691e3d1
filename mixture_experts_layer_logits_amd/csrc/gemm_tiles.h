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
// Tail tiles: with the tail option, a routed group of n rows gets floor(n/BM)
// full BM x BN tiles, and its remaining t rows one more such tile when
// t > BM/2, else "tail" tiles of BM/2 rows x 2 BN columns.  Each wave keeps
// the same (BM/WM) x (BN/WN) block in both shapes, so a tail tile runs at the
// full tile's rate while executing half its rows; when the tail has at most
// BM/4 rows the waves past it skip their MFMAs, which leaves one busy wave per
// SIMD.  Under skewed expert loads most of the padding of the last row tile
// goes away.
//
// Tile order: within a group, the row tiles of one column tile are adjacent
// (and a tail tile follows the two column tiles whose columns it covers),
// so workgroups that share a weight tile run together.  The workgroup id is
// remapped so that each XCD (workgroups are dealt to the 8 XCDs round-robin)
// walks a contiguous range of the tile list, keeping those neighbours in one
// L2.
#pragma once

#include <type_traits>
#include <utility>

#include "moe_common.h"

namespace moe {

// fn(integral_constant<int, 0>{}), ..., fn(integral_constant<int, N - 1>{}):
// a loop the compiler cannot leave rolled (a rolled loop over accumulator
// blocks indexes them at run time and moves them to scratch memory).
template <typename Fn, int... I>
__device__ __forceinline__ void static_for_impl(Fn& fn, std::integer_sequence<int, I...>) {
  (fn(std::integral_constant<int, I>{}), ...);
}
template <int N, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  static_for_impl(fn, std::make_integer_sequence<int, N>{});
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// EPI_COMBINE: no C; each result row is scaled by its row's gate and added
// (fp32 atomics) into Y at its token's row.  EPI_DSWIGLU (MXFP8 kernel
// only): the SwiGLU backward of the result dh.  EPI_WGRAD (MXFP8 kernel
// only): a weight gradient, one fixed tile grid per group whose K is the
// group's padded row count.
enum { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_F32_BIAS = 2, EPI_COMBINE = 3, EPI_DSWIGLU = 4,
       EPI_WGRAD = 5 };

struct GemmArgs {
  // routed groups (E == 0: none)
  int E;
  const int32_t* offsets;  // [E + 1] row offsets of the groups
  const int32_t* tiles;    // [E + 1] exclusive prefix of the groups' tile counts
  const void* A;           // group g owns rows offsets[g] .. offsets[g+1]-1
  long long lda;
  const int32_t* gather;   // or null: routed row r is row gather[r] of A
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
  void* GUd;               // FC1 only, or null: the dense group's g | u
  long long ldgud;
  const float* bias;       // EPI_F32_BIAS: added per column, or null
  // Split-K (EPI_STORE on routed groups, EPI_F32_BIAS on the dense group):
  // K is cut into ksplit equal slices; slice s of every tile writes fp32
  // partials (no bias) to Cpart + s * part_stride + row * N + n, summed
  // later in slice order.
  int ksplit;
  float* Cpart;
  long long part_stride;
  int tail;                // routed groups use tail tiles (kernels built for them)
  // EPI_COMBINE: routed row r adds comb_gate[r] * C[r] into Y[comb_token[r]];
  // dense row t adds C[t] into Y[t].  With split-K every slice adds its part.
  const int32_t* comb_token;
  const float* comb_gate;
  float* Y;
  long long ldy;
  // EPI_WGRAD: rows of each group's output (the A operand's rows)
  int Mw;
};

// One tile's work, with typed base pointers already offset to the group.
template <typename TIn, typename TOut>
struct TileJob {
  const TIn* A;
  long long lda;
  const int32_t* gather;   // routed rows read from A row gather[m], or null
  int rows;
  const TIn* B0;
  const TIn* B1;
  int N, K;
  TOut* C;
  long long ldc;
  TOut* GU;
  long long ldgu;
  int m0, n0;
  int k0, klen;            // K range of this work item (split-K slice)
  float* P;                // split-K partial rows of the group, or null
  int cls;                 // 0: BM x BN tile, 1: BM/2 x 2BN tail tile
  int dense;               // 1: the dense group, 0: a routed group
  int row0;                // first row of the group (routed), else 0
  const int32_t* ctok;     // EPI_COMBINE: token of each routed row, or null (dense)
  const float* cgate;      // EPI_COMBINE: gate of each routed row, or null (gate 1)
};

// Tiles of one routed group of `rows` rows with NT = ceil(N / BN) column tiles.
__host__ __device__ inline int group_full_rows(int rows, int bm, int tail) {
  if (!tail) return (rows + bm - 1) / bm;
  const int nf = rows / bm, t = rows - nf * bm;
  return nf + (t > bm / 2 ? 1 : 0);
}

__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Batch size of a per-token gather over its k routed rows (combine, the
// dispatch gradient, dx):
// fn(integral_constant<int, B>) with B the largest of 1, 2, 4, 8 not above k.
template <typename Fn>
inline void with_gather_batch(int k, Fn&& fn) {
  if (k >= 8) fn(std::integral_constant<int, 8>{});
  else if (k >= 4) fn(std::integral_constant<int, 4>{});
  else if (k >= 2) fn(std::integral_constant<int, 2>{});
  else fn(std::integral_constant<int, 1>{});
}

// Upper bound of the tile count, known on the host (a multiple of 8).
inline int grid_upper_bound(const GemmArgs& a, int BM, int BN, int R) {
  long long t = 0;
  if (a.E > 0) t += (long long)(cdiv(R, BM) + a.E) * cdiv(a.N, BN);
  if (a.Td > 0) t += (long long)cdiv(a.Td, BM) * cdiv(a.Nd, BN);
  t *= (a.ksplit > 1 ? a.ksplit : 1);
  return (int)(((t + 7) / 8) * 8);
}

// Maps blockIdx.x to a tile.  Returns false for surplus workgroups.
template <int BM, int BN, typename TIn, typename TOut>
__device__ __forceinline__ bool decode_tile(const GemmArgs& a, TileJob<TIn, TOut>& j) {
  const int routed = (a.E > 0) ? a.tiles[a.E] : 0;
  const int dmt = cdiv(a.Td, BM);
  const int dense = (a.Td > 0) ? dmt * cdiv(a.Nd, BN) : 0;
  const int total = routed + dense;
  const int ks = a.ksplit > 1 ? a.ksplit : 1;
  const int bid = blockIdx.x;
  const int per = (total * ks + 7) >> 3;
  const int slot = bid >> 3;
  if (slot >= per) return false;
  const int item = (bid & 7) * per + slot;
  if (item >= total * ks) return false;
  // slice-major: concurrently running items share the slice's K range
  const int kslice = item / total;
  const int lid = item - kslice * total;
  j.P = nullptr;
  if (lid < routed) {
    // largest g with tiles[g] <= lid (empty groups share their start)
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tiles[mid] <= lid) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    j.dense = 0;
    const int row0 = a.offsets[g];
    j.row0 = row0;
    const int rows = a.offsets[g + 1] - row0;
    // Column tiles go in pairs: the full tiles of columns 2p and 2p+1 (row
    // tiles adjacent), then the group's tail tile over the same 2 BN columns,
    // which finds that weight strip still in L2.
    const int mt = group_full_rows(rows, BM, a.tail);
    const int ht = (mt * BM < rows) ? 1 : 0;           // only with tail tiles
    const int r = lid - a.tiles[g];
    const int per = 2 * mt + ht;
    const int p = r / per;
    const int q = r - p * per;
    const int nt = cdiv(a.N, BN);
    const int pair_cols = (nt - 2 * p) < 2 ? (nt - 2 * p) : 2;
    if (q < pair_cols * mt) {
      j.cls = 0;
      j.m0 = (q % mt) * BM;
      j.n0 = (2 * p + q / mt) * BN;
    } else {
      j.cls = 1;
      j.m0 = mt * BM;
      j.n0 = p * 2 * BN;
    }
    j.rows = rows;
    j.N = a.N;
    j.K = a.K;
    j.lda = a.lda;
    j.ldc = a.ldc;
    j.ldgu = a.ldgu;
    if (a.gather) {
      j.A = static_cast<const TIn*>(a.A);
      j.gather = a.gather + row0;
    } else {
      j.A = static_cast<const TIn*>(a.A) + (long long)row0 * a.lda;
      j.gather = nullptr;
    }
    j.B0 = static_cast<const TIn*>(a.B0) + (long long)g * a.strideB;
    j.B1 = a.B1 ? static_cast<const TIn*>(a.B1) + (long long)g * a.strideB : nullptr;
    j.C = static_cast<TOut*>(a.C) + (long long)row0 * a.ldc;
    j.GU = a.GU ? static_cast<TOut*>(a.GU) + (long long)row0 * a.ldgu : nullptr;
    j.klen = a.K / ks;
    j.k0 = kslice * j.klen;
    if (ks > 1 && a.Cpart) j.P = a.Cpart + kslice * a.part_stride + (long long)row0 * a.N;
    j.ctok = a.comb_token ? a.comb_token + row0 : nullptr;
    j.cgate = a.comb_gate ? a.comb_gate + row0 : nullptr;
    return true;
  }
  const int r = lid - routed;
  j.cls = 0;
  j.dense = 1;
  j.row0 = 0;
  j.m0 = (r % dmt) * BM;
  j.n0 = (r / dmt) * BN;
  j.rows = a.Td;
  j.N = a.Nd;
  j.K = a.Kd;
  j.lda = a.ldad;
  j.gather = nullptr;
  j.ldc = a.ldcd;
  j.A = static_cast<const TIn*>(a.Ad);
  j.B0 = static_cast<const TIn*>(a.Bd0);
  j.B1 = static_cast<const TIn*>(a.Bd1);
  j.C = static_cast<TOut*>(a.Cd);
  j.GU = static_cast<TOut*>(a.GUd);
  j.ldgu = a.ldgud;
  j.klen = a.Kd / ks;
  j.k0 = kslice * j.klen;
  if (ks > 1 && a.Cpart) j.P = a.Cpart + kslice * a.part_stride;
  j.ctok = nullptr;
  j.cgate = nullptr;
  return true;
}

// ---------------------------------------------------------------------------
// Schedule: tiles[g] = sum over groups g' < g of that group's tile count
// (ceil(rows / BM) * NT, or with tail tiles the full tiles times NT plus
// ceil(N / 2BN) tail tiles), for two GEMMs at once.  One workgroup of 1024
// threads (E <= 1024).
// ---------------------------------------------------------------------------
namespace {
__global__ void __launch_bounds__(1024)
schedule_tiles_kernel(const int32_t* __restrict__ offsets, int E, int bm1, int nt1,
                      int32_t* __restrict__ tiles1, int bm2, int nt2,
                      int32_t* __restrict__ tiles2, int tail) {
  __shared__ int s1[1024];
  __shared__ int s2[1024];
  const int g = threadIdx.x;
  int v1 = 0, v2 = 0;
  if (g < E) {
    const int rows = offsets[g + 1] - offsets[g];
    const int f1 = group_full_rows(rows, bm1, tail), f2 = group_full_rows(rows, bm2, tail);
    v1 = f1 * nt1 + (tail && f1 * bm1 < rows ? (nt1 + 1) / 2 : 0);
    v2 = tiles2 ? f2 * nt2 + (tail && f2 * bm2 < rows ? (nt2 + 1) / 2 : 0) : 0;
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
  // inclusive -> exclusive, plus the total at index E (E == 1024 puts that
  // entry one past the last thread, so the loop gives it to thread 0)
  for (int i = g; i <= E; i += 1024) {
    tiles1[i] = (i == 0) ? 0 : s1[i - 1];
    if (tiles2) tiles2[i] = (i == 0) ? 0 : s2[i - 1];
  }
}
}  // namespace

// ---------------------------------------------------------------------------
// bf16 MFMA tile kernel.
//
// WM x WN waves (64 threads each) tile the BM x BN output (per B matrix);
// each wave owns a (BM/WM) x (BN/WN) block made of 32 x 32 MFMA blocks
// (v_mfma_f32_32x32x16_bf16, fp32 accumulators).
//
// Operands reach LDS with the direct global->LDS load
// (global_load_lds_dwordx4): each wave instruction moves 16 rows x 64 bytes,
// lane l's 16 bytes landing at byte 16 l of a 1 KiB block, so the data never
// passes through registers.  K advances 32 at a time through a ring of four
// LDS stages with three slices in flight: a CU ingests only ~45-55 bytes per
// clock this way, close to what the MFMAs consume, so the loads must stream
// continuously rather than one slice ahead.  Each step waits only for its own
// slice (an explicit vmcnt that leaves the two younger slices in flight),
// then a barrier makes every wave's part of the slice visible.
//
// Rows are 64 bytes with no padding; 16-byte chunk c of row r sits at
// position c ^ f(r), f(r) = 2 r[2] + (r[1] ^ r[3]) (bits of r), which keeps
// the 16-byte fragment reads of 32 consecutive rows free of bank conflicts.
//
// The MFMA is issued with the weight fragment as its first operand, so each
// lane ends up owning one token row and runs of 4 consecutive output columns
// (8-byte stores of bf16, 16-byte stores of fp32).
// ---------------------------------------------------------------------------
#define MOE_AS_GLOBAL(p) ((const __attribute__((address_space(1))) void*)(p))
#define MOE_AS_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ int swz(int r) { return (((r >> 2) & 1) << 1) | (((r >> 1) ^ (r >> 3)) & 1); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Scalar copy of a pointer that is uniform across the wave.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const char*>(((unsigned long long)hi << 32) | lo);
}

template <int BM, int BN, int NB, int EPI, int WM, int WN, int TL>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_bf16_mfma_kernel(const GemmArgs args) {
  constexpr int NW = WM * WN;
  constexpr int BK = 32;                        // one 64-byte row per operand row
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NJ = WTN / 32;
  constexpr int ROWS0 = BM + NB * BN;           // operand rows per LDS stage
  constexpr int ROWS1 = BM / 2 + NB * 2 * BN;   // ... of a tail tile
  constexpr int ROWS = (TL && ROWS1 > ROWS0) ? ROWS1 : ROWS0;
  constexpr int BPW0 = ROWS0 / 16 / NW;         // 1 KiB blocks (loads) per wave
  constexpr int BPW1 = ROWS1 / 16 / NW;
  constexpr int BPWX = (TL && BPW1 > BPW0) ? BPW1 : BPW0;
  static_assert(MI >= 1 && NJ >= 1, "tile too small");
  static_assert(ROWS0 % (16 * NW) == 0 && (!TL || (ROWS1 % (16 * NW) == 0 && WM % 2 == 0)),
                "every wave loads the same number of 1 KiB blocks");
  using TOut = typename std::conditional<EPI == EPI_F32_BIAS, float, bf16_t>::type;

  __shared__ __attribute__((aligned(1024))) bf16_t st0[ROWS * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t st1[ROWS * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t st2[ROWS * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t st3[ROWS * BK];

  TileJob<bf16_t, TOut> job;
  if (!decode_tile<BM, BN>(args, job)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // Tile shape: BM x BN, or for a tail tile BM/2 x 2BN with the waves laid
  // out (WM/2) x (2WN); the per-wave block is the same.
  const bool tail = TL && __builtin_amdgcn_readfirstlane(job.cls) != 0;
  const int bmc = tail ? BM / 2 : BM;
  const int bnc = tail ? 2 * BN : BN;
  const int wnc = tail ? 2 * WN : WN;
  const int bpw = tail ? BPW1 : BPW0;      // blocks this wave loads per slice
  const int wm = wave / wnc, wn = wave % wnc;
  // Waves whose rows all lie past the group's end only load and sync.
  const bool live = job.m0 + wm * WTM < job.rows;

  // This wave loads blocks b = wave * bpw + j; lane l covers row 16 b + l / 4
  // of the operand that block belongs to and fetches the logical chunk that
  // belongs at position l % 4.
  const int dma_c = (lane & 3) ^ swz(lane >> 2);
  // Each block's first row is folded into its 64-bit base, so a lane's
  // 32-bit offset spans at most 16 rows whatever the operand's size.  Rows
  // gathered from x keep the absolute token row (T d < 2^31, checked by the
  // API).
  uint32_t g_off[BPWX];
  const char* g_base[BPWX];
#pragma unroll
  for (int j = 0; j < BPWX; ++j) {
    const int row = (wave * bpw + j) * 16;
    const bf16_t* src;
    int ld, rbase, rlimit;
    if (row < bmc) {
      src = job.A;
      ld = (int)job.lda;
      rbase = job.m0 + row;
      rlimit = job.rows;
    } else {
      const int rb = row - bmc;
      src = (rb < bnc) ? job.B0 : job.B1;
      ld = job.K;
      rbase = job.n0 + (rb < bnc ? rb : rb - bnc);
      rlimit = job.N;
    }
    int r = rbase + (lane >> 2);
    r = r < rlimit ? r : rlimit - 1;                    // clamp: never stored
    if (row < bmc && job.gather) {
      // fused permutation: a routed row comes straight from its token's row
      r = job.gather[r];
      g_off[j] = (uint32_t)(r * ld + dma_c * 8) * 2u;
      g_base[j] = uniform_ptr(src);
    } else {
      const int r0 = rbase < rlimit ? rbase : rlimit - 1;   // the block's first (clamped) row
      g_off[j] = (uint32_t)((r - r0) * ld + dma_c * 8) * 2u;
      g_base[j] = uniform_ptr(src + (long long)r0 * ld);
    }
  }
  // Issued as inline assembly so that only the explicit vmcnt waits below
  // order these loads (the compiler cannot tell the four stages apart across
  // the loop and would otherwise drain every load before some LDS reads).
  // M0 holds the wave-uniform LDS destination; nothing else in this kernel
  // uses M0.
  auto dma = [&](bf16_t* stage, int k0, auto nblk_c) {
    constexpr int NBLK = decltype(nblk_c)::value;
#pragma unroll
    for (int j = 0; j < NBLK; ++j) {
      const uint32_t lds = (uint32_t)(uintptr_t)MOE_AS_LDS(stage + (wave * bpw + j) * 512);
      const char* base = g_base[j] + (size_t)k0 * 2;
      const uint32_t off = g_off[j];
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                   :: "s"(lds), "v"(off), "s"(base) : "memory");
    }
  };

  f32x16_t acc[NB][MI][NJ];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.0f;

  // Fragment rows are lane % 32 plus multiples of 16, so the swizzle is a
  // per-lane constant; sub-step kk reads chunk 2 kk + lane / 32.
  const int frag_row = lane & 31;
  const int sw = swz(frag_row);
  const int kpos0 = ((0 + (lane >> 5)) ^ sw) << 3;
  const int kpos1 = ((2 + (lane >> 5)) ^ sw) << 3;
  const int a_row = (wm * WTM + frag_row) * BK;
  const int b_row = (bmc + wn * WTN + frag_row) * BK;
  const int b_blk = bnc * BK;
  auto load_frags = [&](const bf16_t* stage, int kpos, bf16x8_t (&af)[MI],
                        bf16x8_t (&bfr)[NB][NJ]) {
    const bf16_t* pa = stage + a_row + kpos;
    const bf16_t* pb = stage + b_row + kpos;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * BK);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[b][j] = *reinterpret_cast<const bf16x8_t*>(pb + b * b_blk + j * 32 * BK);
  };
  auto mma = [&](const bf16x8_t (&af)[MI], const bf16x8_t (&bfr)[NB][NJ]) {
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b][j], af[i],
                                                                 acc[b][i][j], 0, 0, 0);
  };
  // Barrier with compiler fences: the hardware barrier itself does not
  // order memory operations for the compiler.
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Waits until this wave's loads of slice `ready` are done, given the
  // slices issued so far (0 .. issued-1), leaving younger ones in flight.
  const int KT = job.klen / BK;
  const int kbeg = job.k0;
  auto wait_slice = [&](int ready, int issued, auto nblk_c) {
    constexpr int NBLK = decltype(nblk_c)::value;
    const int younger = issued - 1 - ready;
    if (younger >= 2) wait_vmcnt<2 * NBLK>();
    else if (younger == 1) wait_vmcnt<NBLK>();
    else wait_vmcnt<0>();
  };
  // Step s consumes stage s % 4 in two 16-wide sub-steps.  Its first
  // fragments were read during the previous step.  The barrier sits between
  // the two sub-steps: after it, slice s+1 is complete in LDS (each wave
  // waited for its own part), every wave has finished step s-1, so stage
  // (s+3) % 4 can be refilled and the first fragments of step s+1 read while
  // the second sub-step's MFMAs run.
  // The K loop exists twice, with and without the fragment reads and MFMAs,
  // so that no branch on `live` sits inside it (a branch there makes the
  // compiler drain outstanding LDS reads at every join).
  auto k_loop = [&](auto live_c, auto nblk_c) {
    constexpr bool LIVE = decltype(live_c)::value;
    bf16x8_t af0[MI], af1[MI];
    bf16x8_t bf0[NB][NJ], bf1[NB][NJ];
    // The fragment reads of each half-step are spread between its MFMAs
    // (one read, one MFMA, ...), which keeps both the LDS and the matrix
    // pipe busy; the last step reads the (unused) next stage as well, so
    // that reads and MFMAs stay in one block the scheduler can interleave.
    auto interleave = [&]() {
#pragma unroll
      for (int r = 0; r < 5; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    };
    auto step = [&](const bf16_t* cur, const bf16_t* next, bf16_t* refill, int s) {
      if constexpr (LIVE) {
        load_frags(cur, kpos1, af1, bf1);
        mma(af0, bf0);
        interleave();
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < KT) wait_slice(s + 1, s + 3 < KT ? s + 3 : KT, nblk_c);
      barrier();
      if (s + 3 < KT) dma(refill, kbeg + (s + 3) * BK, nblk_c);
      if constexpr (LIVE) {
        load_frags(next, kpos0, af0, bf0);
        mma(af1, bf1);
        interleave();
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    dma(st0, kbeg, nblk_c);
    if (KT > 1) dma(st1, kbeg + BK, nblk_c);
    if (KT > 2) dma(st2, kbeg + 2 * BK, nblk_c);
    wait_slice(0, KT < 3 ? KT : 3, nblk_c);
    barrier();
    if constexpr (LIVE) load_frags(st0, kpos0, af0, bf0);
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
  };
  // Each wave issues the same number of block loads per slice (4 or 5 with
  // the tail shape), which the vmcnt waits count on.
  using nb0 = std::integral_constant<int, BPW0>;
  using nb1 = std::integral_constant<int, BPW1>;
  // With g and u saved for the backward, the SwiGLU epilogue goes out
  // through LDS (below); every wave, idle or not, joins its barrier.
  const bool staged = (EPI == EPI_SWIGLU && job.GU != nullptr) || EPI == EPI_COMBINE;
  if (!live) {
    if (tail) k_loop(std::false_type{}, nb1{});
    else k_loop(std::false_type{}, nb0{});
    if (staged) barrier();
    return;
  }
  if (tail) k_loop(std::true_type{}, nb1{});
  else k_loop(std::true_type{}, nb0{});

  if constexpr (EPI == EPI_SWIGLU) {
    if (staged) {
      // In the accumulator layout a store instruction scatters 16-byte
      // pieces over 32 rows, which cost several times their bytes in write
      // traffic for the three outputs.  Per 32-row half, g and u (fp32) go
      // to this wave's 16 KiB of the ring (rows of 512 bytes, 16-byte chunk
      // c of row r at c ^ r: g in chunks 0-15, u in 16-31), and come back
      // with each lane holding 4 consecutive columns of one row, so 16 lanes
      // store 128 contiguous bytes of h, of g and of u.
      barrier();                                  // the ring is free
      char* buf = reinterpret_cast<char*>((wave >> 1) == 0 ? st0 : (wave >> 1) == 1 ? st1
                                          : (wave >> 1) == 2 ? st2 : st3) + (wave & 1) * 16384;
      const int cbase = job.n0 + wn * WTN;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = j * 8 + 2 * q + (lane >> 5);
            const f32x16_t& G = acc[0][i][j];
            const f32x16_t& U = acc[NB - 1][i][j];
            *reinterpret_cast<float4*>(buf + frag_row * 512 + ((ch ^ frag_row) << 4)) =
                make_float4(G[4 * q], G[4 * q + 1], G[4 * q + 2], G[4 * q + 3]);
            *reinterpret_cast<float4*>(buf + frag_row * 512 + (((16 + ch) ^ frag_row) << 4)) =
                make_float4(U[4 * q], U[4 * q + 1], U[4 * q + 2], U[4 * q + 3]);
          }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int r = 4 * t + (lane >> 4), cc = lane & 15;
          const float4 g4 = *reinterpret_cast<const float4*>(buf + r * 512 + ((cc ^ r) << 4));
          const float4 u4 = *reinterpret_cast<const float4*>(buf + r * 512 + (((16 + cc) ^ r) << 4));
          const int m = job.m0 + wm * WTM + i * 32 + r;
          const int n = cbase + 4 * cc;
          if (m < job.rows && n < job.N) {
            const uint2 ph = make_uint2(pack_bf16x2(silu_fast(g4.x) * u4.x, silu_fast(g4.y) * u4.y),
                                        pack_bf16x2(silu_fast(g4.z) * u4.z, silu_fast(g4.w) * u4.w));
            *reinterpret_cast<uint2*>(job.C + (long long)m * job.ldc + n) = ph;
            *reinterpret_cast<uint2*>(job.GU + (long long)m * job.ldgu + n) =
                make_uint2(pack_bf16x2(g4.x, g4.y), pack_bf16x2(g4.z, g4.w));
            *reinterpret_cast<uint2*>(job.GU + (long long)m * job.ldgu + job.N + n) =
                make_uint2(pack_bf16x2(u4.x, u4.y), pack_bf16x2(u4.z, u4.w));
          }
        }
      }
      return;
    }
  }

  if constexpr (EPI == EPI_COMBINE) {
    // Per 32-row half, this wave's 32 x 128 fp32 results go to its 16 KiB
    // of the ring (rows of 512 bytes, 16-byte chunk c of row r at c ^ r) and
    // come back one row at a time, lane l holding column l (+ 64), so each
    // atomic add instruction covers 256 contiguous bytes of one y row.
    static_assert(NB == 1 && WTN == 128, "combine epilogue: one B, 128 columns per wave");
    barrier();                                    // the ring is free
    char* buf = reinterpret_cast<char*>((wave >> 1) == 0 ? st0 : (wave >> 1) == 1 ? st1
                                        : (wave >> 1) == 2 ? st2 : st3) + (wave & 1) * 16384;
    const int cbase = job.n0 + wn * WTN;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = j * 8 + 2 * q + (lane >> 5);
          const f32x16_t& Cv = acc[0][i][j];
          *reinterpret_cast<float4*>(buf + frag_row * 512 + ((ch ^ frag_row) << 4)) =
              make_float4(Cv[4 * q], Cv[4 * q + 1], Cv[4 * q + 2], Cv[4 * q + 3]);
        }
      // lane r < 32 looks up row r's token and gate; rows past the group: -1
      const int mr = job.m0 + wm * WTM + i * 32 + frag_row;
      int tok = -1;
      float gw = 0.0f;
      if (mr < job.rows) {
        tok = job.ctok ? job.ctok[mr] : mr;
        gw = job.cgate ? job.cgate[mr] : 1.0f;
      }
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int t = __builtin_amdgcn_readlane(tok, r);
        const float g = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gw), r));
        if (t < 0) continue;
        float* yrow = args.Y + (long long)t * args.ldy + cbase;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = h * 64 + lane;
          const float v = *reinterpret_cast<const float*>(
              buf + r * 512 + ((((col >> 2) ^ r)) << 4) + (col & 3) * 4);
          if (cbase + col < job.N) atomicAdd(yrow + col, g * v);
        }
      }
    }
    return;
  }

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
            o[r] = acc[0][i][j][4 * q + r] +
                   ((!job.P && args.bias && n + r < job.N) ? args.bias[n + r] : 0.0f);
          // a split-K slice writes its partial sums (row pitch N), no bias
          float* dst = job.P ? job.P + (long long)m * job.N + n : job.C + (long long)m * job.ldc + n;
          const long long ld = job.P ? job.N : job.ldc;
          if (n + 3 < job.N && (ld & 3) == 0) {
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
          if (job.P) {
            *reinterpret_cast<float4*>(job.P + (long long)m * job.N + n) =
                make_float4(Cv[4 * q], Cv[4 * q + 1], Cv[4 * q + 2], Cv[4 * q + 3]);
          } else {
            uint2 pk = make_uint2(pack_bf16x2(Cv[4 * q], Cv[4 * q + 1]),
                                  pack_bf16x2(Cv[4 * q + 2], Cv[4 * q + 3]));
            *reinterpret_cast<uint2*>(job.C + (long long)m * job.ldc + n) = pk;
          }
        }
      }
    }
  }
}

// Host launcher of the MFMA kernel: sizes the grid from the host-side tile
// bound.
template <int BM, int BN, int NB, int EPI, int WM, int WN, int TL>
hipError_t launch_mfma_gemm(const GemmArgs& a, int R, hipStream_t st) {
  if (a.tail && !TL) return hipErrorInvalidValue;
  const int grid = grid_upper_bound(a, BM, BN, R);
  if (grid == 0) return hipSuccess;
  gemm_bf16_mfma_kernel<BM, BN, NB, EPI, WM, WN, TL><<<grid, 64 * WM * WN, 0, st>>>(a);
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
      float v = 0.0f;
      if (m < job.rows && k < job.K) {
        const long long src = job.gather ? job.gather[m] : m;
        v = to_f32<T>(job.A[src * job.lda + k]);
      }
      sA[kk][r] = v;
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
      } else if constexpr (EPI == EPI_COMBINE) {
        const int t = job.ctok ? job.ctok[m] : m;
        const float gw = job.cgate ? job.cgate[m] : 1.0f;
        atomicAdd(args.Y + (long long)t * args.ldy + n, gw * acc[0][i][jj]);
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
