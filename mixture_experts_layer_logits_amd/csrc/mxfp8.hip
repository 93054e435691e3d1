// MXFP8 grouped expert FFN (Primus blog, low-precision section: MXFP8 block
// scaling, E4M3 elements in blocks of 32 along the contraction dimension with
// one E8M0 power-of-two scale per block, on gfx950's scaled MFMA).
//
//   quantize:  bf16 [rows, cols] -> E4M3 codes [rows, cols] + E8M0 bytes
//              [rows, cols / 32].  Block scale 2^s, s = floor(log2 amax) - 8
//              (8 = exponent of E4M3's largest power of two), clipped to
//              [-127, 127]; an all-zero block gets s = -127.  Elements are
//              v / 2^s rounded to E4M3, nearest-even, saturating at +-448.
//   FC1:       h = silu(xq . wg^T) * (xq . wu^T) on the dequantised operands
//              (fp32 accumulate), quantised to MXFP8 along F in the epilogue
//   FC2:       y_perm = hq . wd^T -> bf16
//
// Backward (data gradients; the weight gradients stay bf16):
//   quantize_t: bf16 [B][rows, cols] -> codes [B][cols, rows] quantised
//              along rows (weights read against their storage order)
//   dh:        dYq . (w_down quantised along d)^T, epilogue: the SwiGLU
//              backward from the saved g, u -> dg, du, h in bf16, and dg | du
//              quantised along F for the next GEMM
//   dX:        (dg | du)q . ([w_gate; w_up] quantised along F)^T -> bf16
//
// Both GEMMs read routed rows through row_token from the quantised x (the
// permutation fused into FC1's operand load; quantising is row-wise, so
// quantise-then-gather equals gather-then-quantise exactly).
//
// Scaled MFMA operand layout (v_mfma_scale_f32_32x32x64_f8f6f4, fp8 e4m3 on
// both sides): lane l holds row l % 32 of its operand and 32 values of K,
// bytes 0-15 at k = 16 (l / 32) + q and bytes 16-31 at k = 32 + 16 (l / 32) + q;
// its scale operand (byte 0) applies to row l % 32 and K block l / 32 of the
// 64-wide step.  Each 64-byte LDS row of a stage therefore feeds one MFMA per
// fragment: chunks l / 32 and 2 + l / 32, the same two 16-byte chunks the
// bf16 kernel reads in its two sub-steps.
#include <utility>

#include "gemm_tiles.h"

namespace moe {

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// v, in a scalar register the compiler cannot see through.
__device__ __forceinline__ uint32_t opaque_u32(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// An empty use of an accumulator tile (in VGPRs): its MFMAs must have run
// by here.
__device__ __forceinline__ void use_acc(const f32x16_t& a) { asm volatile("" ::"v"(a)); }


// FC1: 256 rows x (128 gate + 128 up) columns; FC2: 256 x 256; 8 waves.
constexpr int MX_FC1_BM = 256, MX_FC1_BN = 128;
constexpr int MX_FC2_BM = 256, MX_FC2_BN = 256;

// ---------------------------------------------------------------------------
// E4M3 / E8M0 encoding
// ---------------------------------------------------------------------------

// Scale exponent s of a block with largest magnitude amax (>= 0, finite):
// floor(log2 amax) - 8 from amax's exponent field; zero and fp32-subnormal
// amax (floor(log2) <= -127) give the smallest scale, -127.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 255u);
  const int s = e - 127 - 8;
  return (e == 0 || s < -127) ? -127 : s;
}

// 2^-s for s in [-127, 119], exactly.
__device__ __forceinline__ float mx_inv_scale(int s) {
  return __uint_as_float((uint32_t)(127 - s) << 23);
}

// E4M3 code (1 sign, 4 exponent bits with bias 7, 3 mantissa bits) nearest
// to y, ties to even, magnitudes that round past 448 saturating to 448.
// Below 2^-6 the grid is the subnormal step 2^-9, whose integer multiples
// 0..8 are exactly the codes 0..8.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t c;
  if (!(a < 448.0f)) {
    c = 0x7eu;
  } else if (a < 0.015625f) {
    c = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 mantissa bits of the fp32 pattern, nearest-even; a carry moves
    // into the exponent, which is the correct next binade
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);
    c = (b >> 20) - (120u << 3);   // rebias the exponent from 127 to 7
  }
  return sign | c;
}

// ---------------------------------------------------------------------------
// Quantisation: 4 lanes per block of 32 values, 8 values (16 bytes) per lane.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
mx_quantize_kernel(const bf16_t* __restrict__ src, long long n8, uint8_t* __restrict__ q,
                   uint8_t* __restrict__ scales) {
  // n8 is a multiple of 4 and so is the stride: the 4 lanes of a block are
  // active together
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n8; i += (long long)gridDim.x * 256) {
    const uint4 raw = reinterpret_cast<const uint4*>(src)[i];
    float v[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      v[2 * p] = __uint_as_float(w[p] << 16);
      v[2 * p + 1] = __uint_as_float(w[p] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p) amax = fmaxf(amax, fabsf(v[p]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    const int s = mx_scale_exp(amax);
    const float inv = mx_inv_scale(s);
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      lo |= e4m3_code(v[p] * inv) << (8 * p);
      hi |= e4m3_code(v[4 + p] * inv) << (8 * p);
    }
    reinterpret_cast<uint2*>(q)[i] = make_uint2(lo, hi);
    if ((i & 3) == 0) scales[i >> 2] = (uint8_t)(s + 127);
  }
}

hipError_t launch_mx_quantize(const void* src, long long rows, int cols, uint8_t* q,
                              uint8_t* scales, hipStream_t st) {
  const long long n8 = rows * (cols / 8);
  if (n8 == 0) return hipSuccess;
  const long long want = (n8 + 255) / 256;
  const int grid = (int)(want < 8192 ? want : 8192);
  mx_quantize_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(src), n8, q, scales);
  return hipGetLastError();
}

// Transposed quantisation: element (r, c) of batch b of src [B][rows][cols]
// becomes code q[(b cols + c) ldq + r], quantised with the 31 other rows of
// its 32-row block, scale byte at sq[(b cols + c) (ldq / 32) + r / 32].  A
// workgroup takes 32 rows x 64 columns through LDS; 4 lanes per column
// quantise 8 rows each.
__global__ void __launch_bounds__(256)
mx_quantize_t_kernel(const bf16_t* __restrict__ src, int rows, int cols, int ldq,
                     uint8_t* __restrict__ q, uint8_t* __restrict__ sq) {
  __shared__ float tile[32][65];
  const long long b = blockIdx.z;
  const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 32 * 64; i += 256) {
    const int rr = i >> 6, cc = i & 63;
    const int c = c0 + cc;
    tile[rr][cc] = c < cols ? to_f32<bf16_t>(src[(b * rows + r0 + rr) * cols + c]) : 0.0f;
  }
  __syncthreads();
  const int cc = threadIdx.x >> 2, part = threadIdx.x & 3;
  float v[8];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    v[p] = tile[8 * part + p][cc];
    amax = fmaxf(amax, fabsf(v[p]));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  const int s = mx_scale_exp(amax);
  const float inv = mx_inv_scale(s);
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    lo |= e4m3_code(v[p] * inv) << (8 * p);
    hi |= e4m3_code(v[4 + p] * inv) << (8 * p);
  }
  const int c = c0 + cc;
  if (c < cols) {
    const long long orow = b * cols + c;
    *reinterpret_cast<uint2*>(q + orow * ldq + r0 + 8 * part) = make_uint2(lo, hi);
    if (part == 0) sq[orow * (ldq / 32) + r0 / 32] = (uint8_t)(s + 127);
  }
}

hipError_t launch_mx_quantize_t(const void* src, long long batches, int rows, int cols, int ldq,
                                uint8_t* q, uint8_t* scales, hipStream_t st) {
  if (batches == 0 || rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid(cdiv(cols, 64), rows / 32, (unsigned)batches);
  mx_quantize_t_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(src), rows, cols, ldq,
                                             q, scales);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scaled-MFMA grouped GEMM tile kernel.
//
// The tile machinery (groups, schedule, XCD-aware order) is the bf16
// kernel's, with bytes for elements.  Operand rows of a stage are 64 fp8
// values (one MFMA step), loaded straight into LDS with the same 16-byte
// chunk swizzle.  Scales ride in the same slices: per stage, each operand
// row's dword holding K blocks 4 (kt / 2) .. + 3 (row strides are K / 32
// bytes, K a multiple of 128, so the dword is aligned) lands in a dword
// array beside the stage, one global_load_lds_dword per 64 rows; a lane then
// reads its block's byte, 2 (kt % 2) + l / 32, with one byte read.
//
// Each step is split in two halves over the B fragments: the first half's
// MFMAs run while the second half's fragments are read; after the barrier
// the second half's MFMAs run while the next stage's token fragments and
// first-half weight fragments are read (token fragments double-buffered).
// ---------------------------------------------------------------------------
struct MxScales {
  const uint8_t* A;    // routed rows' operand scales (rows of the quantised x)
  const uint8_t* B0;   // [E][N][K / 32]
  const uint8_t* B1;   // FC1 up, or null
  uint8_t* C;          // FC1: h scales [R][F / 32]
  const uint8_t* Ad;   // the dense group
  const uint8_t* Bd0;
  const uint8_t* Bd1;
  uint8_t* Cd;
};

// The SwiGLU-backward epilogue's other tensors (routed rows, row-major):
// gu [R, 2F] the saved g | u, dgu [R, 2F] and h [R, F] bf16 outputs; the
// GEMM's own C is the quantised dg | du [R, 2F] with scales in MxScales::C.
struct MxBwd {
  const bf16_t* gu;
  bf16_t* dgu;
  bf16_t* h;
  int F;
  // EPI_WGRAD: rows m < wsplit of group g go to w0 + (g wsplit + m) N,
  // the others to w1 + (g (M - wsplit) + m - wsplit) N; fp32, or bf16 when
  // wbf16
  void* w0;
  void* w1;
  int wsplit, wbf16;
};

// The shape of one tile class: CLS 0 is BM x BN with WM x WN waves and a
// four-stage ring; CLS 1 (tail tiles) is BM/2 x 2BN with (WM/2) x (2WN) waves,
// so each wave keeps its (BM/WM) x (BN/WN) block and registers, and a
// three-stage ring (its 640-row stages do not fit four times beside the
// scales).
template <int BM, int BN, int NB, int WM, int WN, int SG, int CLS>
struct MxShape {
  static constexpr int NW = WM * WN;
  static constexpr int BMC = CLS ? BM / 2 : BM;
  static constexpr int BNC = CLS ? 2 * BN : BN;
  static constexpr int WMC = CLS ? WM / 2 : WM;
  static constexpr int WNC = CLS ? 2 * WN : WN;
  static constexpr int NS = CLS ? 3 : 4;            // LDS stages
  static constexpr int ROWS = BMC + NB * BNC;       // operand rows per stage
  static constexpr int BPW = ROWS / 16 / NW;        // 1 KiB data loads per wave per slice
  static constexpr int SB = ROWS / 64;              // 64-row scale blocks per scale slice
  static constexpr int SPW = (SB + NW - 1) / NW;    // scale loads per wave (surplus repeats the last)
  static constexpr int NLD = SG == 1 ? BPW + SPW : BPW;
  static constexpr int SSTR = SG == 1 ? 4 : 16;     // LDS bytes per row of a scale slice
  static constexpr int RING = NS * ROWS * 64;       // bytes of the operand ring
  static constexpr int SRING = (SG == 1 ? NS : 2) * ROWS * SSTR;
  static_assert(ROWS % (16 * NW) == 0 && BMC % 64 == 0 && BNC % 64 == 0, "load blocks");
};

template <int EPI>
using MxOut = typename std::conditional<EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU, uint8_t,
                                        bf16_t>::type;

template <int BM, int BN, int NB, int EPI, int WM, int WN, int SG, int CLS>
__device__ __forceinline__ void mx_tile(const GemmArgs& args, const MxScales& sc,
                                        const MxBwd& bw, const TileJob<uint8_t, MxOut<EPI>>& job,
                                        uint8_t* ring, uint8_t* sring) {
  using S = MxShape<BM, BN, NB, WM, WN, SG, CLS>;
  constexpr int NW = S::NW, BMC = S::BMC, BNC = S::BNC, WNC = S::WNC, NS = S::NS;
  constexpr int ROWS = S::ROWS, BPW = S::BPW, SB = S::SB, SPW = S::SPW, NLD = S::NLD;
  constexpr int SSTR = S::SSTR;
  constexpr int BK = 64;                        // fp8 values (bytes) per row per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MI = WTM / 32, NJ = WTN / 32;
  constexpr int NBJ = NB * NJ;                  // weight fragments per wave
  constexpr int H0 = NBJ / 2, H1 = NBJ - H0;    // ... in each half-step
  static_assert(MI >= 1 && NJ >= 1 && H0 >= 1 && H0 == H1, "tile too small or odd");
  static_assert(NW == 8, "the tail class pairs wave rows");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WNC, wn = wave % WNC;
  const bool live = job.m0 + wm * WTM < job.rows;
  // scale bytes per operand row: the rows of both operands are lda codes
  // long (lda = K except in the weight gradients, whose operand rows hold
  // every group's padded rows and each tile reads its group's K of them)
  const int kb = (int)(job.lda / 32);
  // SG = 8: scale group g covers K blocks 16 g .. 16 g + 15 (steps 8 g ..
  // 8 g + 7), read as the 16 bytes from sg_start(g); the last group's
  // window ends at the row's end (kb >= 16 here), so no read passes it.
  auto sg_start = [&](int g) { return min(16 * g, kb - 16); };

  // Scale bases of this job (the scale arrays mirror the code arrays with
  // one byte per 32 codes, so a code offset maps to offset / 32).
  const uint8_t* sA;
  const uint8_t* sB0;
  const uint8_t* sB1;
  uint8_t* sC;
  if (job.dense) {
    sA = sc.Ad;
    sB0 = sc.Bd0;
    sB1 = sc.Bd1;
    sC = sc.Cd;
  } else {
    sA = sc.A + (job.A - static_cast<const uint8_t*>(args.A)) / 32;
    sB0 = sc.B0 + (job.B0 - static_cast<const uint8_t*>(args.B0)) / 32;
    sB1 = NB > 1 ? sc.B1 + (job.B1 - static_cast<const uint8_t*>(args.B1)) / 32 : nullptr;
    sC = (EPI == EPI_SWIGLU || EPI == EPI_DSWIGLU)
             ? sc.C + (reinterpret_cast<const uint8_t*>(job.C) -
                       static_cast<const uint8_t*>(args.C)) / 32
             : nullptr;
  }

  // Data loads: block b = wave * BPW + j covers stage rows 16 b .. + 15; lane
  // l fetches row 16 b + l / 4, logical chunk (l % 4) ^ f(row), f the bf16
  // kernel's swizzle, which keeps the fragment reads free of bank conflicts.
  const int dma_c = (lane & 3) ^ swz(lane >> 2);
  uint32_t g_off[BPW];
  const char* g_base[BPW];
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int row = (wave * BPW + j) * 16;
    const uint8_t* src;
    int ld, rbase, rlimit;
    if (row < BMC) {
      src = job.A;
      ld = (int)job.lda;
      rbase = job.m0 + row;
      rlimit = job.rows;
    } else {
      const int rb = row - BMC;
      src = (rb < BNC) ? job.B0 : job.B1;
      ld = (int)job.lda;                                // both operands' row stride
      rbase = job.n0 + (rb < BNC ? rb : rb - BNC);
      rlimit = job.N;
    }
    int r = rbase + (lane >> 2);
    r = r < rlimit ? r : rlimit - 1;                    // clamp: never stored
    if (row < BMC && job.gather) {
      // gathered token rows keep their absolute offset (T d < 2^31)
      r = job.gather[r];
      g_off[j] = (uint32_t)(r * ld + dma_c * 16);
      g_base[j] = uniform_ptr(src);
    } else {
      // the block's first (clamped) row folded into the 64-bit base
      const int r0 = rbase < rlimit ? rbase : rlimit - 1;
      g_off[j] = (uint32_t)((r - r0) * ld + dma_c * 16);
      g_base[j] = uniform_ptr(src + (long long)r0 * ld);
    }
  }
  // Scale loads: block b = wave * SPW + j (the last block again where the
  // waves have more loads than there are blocks) covers stage rows 64 b ..
  // + 63, lane l fetching row 64 b + l.
  uint32_t s_off[SPW];
  uint32_t s_lds[SPW];
  const char* s_base[SPW];
#pragma unroll
  for (int j = 0; j < SPW; ++j) {
    const int blk = min(wave * SPW + j, SB - 1);        // wave-uniform
    const int blk0 = blk * 64;
    const int row = blk0 + lane;
    const uint8_t* src;
    int rbase, rlimit;
    if (blk0 < BMC) {
      src = sA;
      rbase = job.m0 + row;
      rlimit = job.rows;
    } else {
      const int rb = blk0 - BMC;
      src = (rb < BNC) ? sB0 : sB1;
      rbase = job.n0 + (row - BMC - (rb < BNC ? 0 : BNC));
      rlimit = job.N;
    }
    int r = rbase < rlimit ? rbase : rlimit - 1;
    s_lds[j] = (uint32_t)blk * 64 * SSTR;
    if (blk0 < BMC && job.gather) {
      r = job.gather[r];
      s_off[j] = (uint32_t)(r * kb);
      s_base[j] = uniform_ptr(src);
    } else {
      const int rb0 = blk0 < BMC ? job.m0 + blk0 : job.n0 + (blk0 - BMC - ((blk0 - BMC) < BNC ? 0 : BNC));
      const int r0 = rb0 < rlimit ? rb0 : rlimit - 1;   // the block's first (clamped) row
      s_off[j] = (uint32_t)((r - r0) * kb);
      s_base[j] = uniform_ptr(src + (long long)r0 * kb);
    }
  }
  // Slice kt: its scale loads (SG = 1, or the first slice of a group), then
  // its data loads (inline assembly, so that only the explicit vmcnt waits
  // order them; M0 holds the LDS destination).
  auto dma = [&](uint8_t* dst, uint8_t* sdst, int kt) {
    if (SG == 1 || (kt & 7) == 0) {
#pragma unroll
      for (int j = 0; j < SPW; ++j) {
        const uint32_t off = s_off[j];
        if constexpr (SG == 1) {
          const uint32_t lds = (uint32_t)(uintptr_t)MOE_AS_LDS(sdst + s_lds[j]);
          const char* base = s_base[j] + (size_t)(kt >> 1) * 4;
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                       :: "s"(lds), "v"(off), "s"(base) : "memory");
        } else {
          const uint32_t lds = (uint32_t)(uintptr_t)MOE_AS_LDS(
              sring + ((kt >> 3) & 1) * (ROWS * 16) + s_lds[j]);
          const char* base = s_base[j] + sg_start(kt >> 3);
          asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                       :: "s"(lds), "v"(off), "s"(base) : "memory");
        }
      }
    }
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const uint32_t lds = (uint32_t)(uintptr_t)MOE_AS_LDS(dst + (wave * BPW + j) * 1024);
      const char* base = g_base[j] + (size_t)kt * BK;
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

  const int frag_row = lane & 31;
  const int hsel = lane >> 5;
  const int c0 = ((0 + hsel) ^ swz(frag_row)) << 4;   // k = 16 hsel ..
  const int c1 = ((2 + hsel) ^ swz(frag_row)) << 4;   // k = 32 + 16 hsel ..
  const int a_row = wm * WTM + frag_row;                // stage row of A fragment 0
  const int b_row = BMC + wn * WTN + frag_row;          // ... of B fragment (0, 0)

  auto read_frag = [&](const uint8_t* stage, int row) -> i32x8_t {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t*>(stage + row * BK + c0);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t*>(stage + row * BK + c1);
    return (i32x8_t)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // Scale bytes of step s start at scale_base(s) + row * SSTR + hsel.
  auto scale_base = [&](int s, int rp) -> const uint8_t* {
    if constexpr (SG == 1) {
      return sring + opaque_u32((uint32_t)rp * (ROWS * 4)) + 2 * (s & 1);
    } else {
      return sring + ((s >> 3) & 1) * (ROWS * 16) + (2 * s - sg_start(s >> 3));
    }
  };
  auto read_scale = [&](const uint8_t* sbase, int row) -> int {
    return (int)sbase[row * SSTR + hsel];
  };
  // weight fragment f (0 .. NBJ-1) = (b, j) with b = f / NJ, j = f % NJ
  auto brow = [&](int f) { return b_row + (f / NJ) * BNC + (f % NJ) * 32; };

  const int KT = job.klen / BK;
  const int kbeg = job.k0 / BK;
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Waits until this wave's loads of slice `ready` are done, given that
  // slices 0 .. last are issued, leaving the younger ones in flight.
  auto wait_slice = [&](int ready, int last) {
    const int younger = last - ready;
    if (NS > 3 && younger >= 2) wait_vmcnt<2 * NLD>();
    else if (younger >= 1) wait_vmcnt<NLD>();
    else wait_vmcnt<0>();
  };

  // Stage rp of the ring.  Stages past 64 KiB are out of reach of the LDS
  // reads' immediate offset, so if the compiler saw constant stage addresses
  // it would keep one address register per fragment and stage live across
  // the loop; the opaque scalar offset makes it add the stage per step to a
  // few per-lane bases instead.
  auto stage = [&](int rp) -> uint8_t* { return ring + opaque_u32((uint32_t)rp * (ROWS * BK)); };

  // The MFMA builtins have no side effects, so without a use LLVM sinks
  // them past the wait/refill blocks of later steps to the loop's end,
  // keeping every fragment of four steps live.  An empty asm that reads a
  // half-step's accumulators pins its MFMAs inside that half-step.
  auto pin_half = [&](int f0) {
#pragma unroll
    for (int f = 0; f < H0; ++f)
#pragma unroll
      for (int i = 0; i < MI; ++i) use_acc(acc[(f0 + f) / NJ][i][(f0 + f) % NJ]);
  };
  auto k_loop = [&](auto live_c) {
    constexpr bool LIVE = decltype(live_c)::value;
    i32x8_t af[2][MI];
    int as[2][MI];
    i32x8_t bf0[H0], bf1[H1];
    int bs0[H0], bs1[H1];
    // Step s uses ring position RP = s % NS and token-fragment buffer
    // P = s % 2, both static: the loop runs in groups of lcm(NS, 2) steps.
    auto step = [&](auto rp_c, auto p_c, int s) {
      constexpr int RP = decltype(rp_c)::value;
      constexpr int P = decltype(p_c)::value;
      const uint8_t* cur = stage(RP);
      const uint8_t* scur = scale_base(s, RP);
      const uint8_t* nxt = stage((RP + 1) % NS);
      const uint8_t* snxt = scale_base(s + 1, (RP + 1) % NS);
      if constexpr (LIVE) {
#pragma unroll
        for (int f = 0; f < H1; ++f) {
          bf1[f] = read_frag(cur, brow(H0 + f));
          bs1[f] = read_scale(scur, brow(H0 + f));
        }
#pragma unroll
        for (int f = 0; f < H0; ++f)
#pragma unroll
          for (int i = 0; i < MI; ++i)
            acc[f / NJ][i][f % NJ] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf0[f], af[P][i], acc[f / NJ][i][f % NJ], 0, 0, 0, bs0[f], 0, as[P][i]);
        // reads spread between the MFMAs (two reads, one MFMA, ...)
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // LDS reads
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        pin_half(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < KT) wait_slice(s + 1, s + NS - 2 < KT - 1 ? s + NS - 2 : KT - 1);
      barrier();
      // stage (s - 1) % NS, read for the last time before this barrier,
      // takes slice s + NS - 1
      if (s + NS - 1 < KT)
        dma(ring + ((RP + NS - 1) % NS) * (ROWS * BK), sring + ((RP + NS - 1) % NS) * (ROWS * 4),
            kbeg + s + NS - 1);
      if constexpr (LIVE) {
        // the last step reads the (unused) next stage too, keeping one shape
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          af[1 - P][i] = read_frag(nxt, a_row + 32 * i);
          as[1 - P][i] = read_scale(snxt, a_row + 32 * i);
        }
#pragma unroll
        for (int f = 0; f < H0; ++f) {
          bf0[f] = read_frag(nxt, brow(f));
          bs0[f] = read_scale(snxt, brow(f));
        }
#pragma unroll
        for (int f = 0; f < H1; ++f)
#pragma unroll
          for (int i = 0; i < MI; ++i)
            acc[(H0 + f) / NJ][i][(H0 + f) % NJ] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf1[f], af[P][i], acc[(H0 + f) / NJ][i][(H0 + f) % NJ], 0, 0, 0, bs1[f], 0,
                as[P][i]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        pin_half(H0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    dma(ring, sring, kbeg);
    if (KT > 1) dma(ring + ROWS * BK, sring + ROWS * 4, kbeg + 1);
    if (NS > 3 && KT > 2) dma(ring + 2 * ROWS * BK, sring + 2 * ROWS * 4, kbeg + 2);
    wait_slice(0, KT - 1 < NS - 2 ? KT - 1 : NS - 2);
    barrier();
    if constexpr (LIVE) {
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        af[0][i] = read_frag(stage(0), a_row + 32 * i);
        as[0][i] = read_scale(scale_base(0, 0), a_row + 32 * i);
      }
#pragma unroll
      for (int f = 0; f < H0; ++f) {
        bf0[f] = read_frag(stage(0), brow(f));
        bs0[f] = read_scale(scale_base(0, 0), brow(f));
      }
    }
    using c0_ = std::integral_constant<int, 0>;
    using c1_ = std::integral_constant<int, 1>;
    using c2_ = std::integral_constant<int, 2>;
    using c3_ = std::integral_constant<int, 3>;
    int kt = 0;
    if constexpr (NS == 4) {
      for (; kt + 4 <= KT; kt += 4) {
        step(c0_{}, c0_{}, kt);
        step(c1_{}, c1_{}, kt + 1);
        step(c2_{}, c0_{}, kt + 2);
        step(c3_{}, c1_{}, kt + 3);
      }
      if (kt < KT) {   // KT is even (K is a multiple of 128)
        step(c0_{}, c0_{}, kt);
        step(c1_{}, c1_{}, kt + 1);
      }
    } else {
      for (; kt + 6 <= KT; kt += 6) {
        step(c0_{}, c0_{}, kt);
        step(c1_{}, c1_{}, kt + 1);
        step(c2_{}, c0_{}, kt + 2);
        step(c0_{}, c1_{}, kt + 3);
        step(c1_{}, c0_{}, kt + 4);
        step(c2_{}, c1_{}, kt + 5);
      }
      if (kt < KT) {   // 2 or 4 steps left
        step(c0_{}, c0_{}, kt);
        step(c1_{}, c1_{}, kt + 1);
        if (kt + 2 < KT) {
          step(c2_{}, c0_{}, kt + 2);
          step(c0_{}, c1_{}, kt + 3);
        }
      }
    }
  };
  // A weight gradient of a group without rows runs zero K steps and stores
  // exact zeros (KT is uniform over the workgroup: every wave skips the same
  // loop and its barriers).
  if (EPI != EPI_WGRAD || KT > 0) {
    if (!live) {
      k_loop(std::false_type{});
      if constexpr (EPI == EPI_DSWIGLU || EPI == EPI_COMBINE) barrier();   // the staged epilogue's
      return;
    }
    k_loop(std::true_type{});
  }

  if constexpr (EPI == EPI_COMBINE) {
    // The combine folded into FC2: per 32-row half, this wave's 32 x 128 fp32
    // results go through its 16 KiB of the freed ring and come back one row
    // at a time, lane l holding columns l and l + 64, so each atomic add
    // instruction covers 256 contiguous bytes of one y row; the row's gate
    // (1 for the shared expert's rows) scales it and its token picks the row.
    static_assert(NB == 1 && WTN == 128, "combine epilogue: one B, 128 columns per wave");
    barrier();                                    // the ring is free
    char* buf = reinterpret_cast<char*>(ring) + wave * 16384;
    const int cbase = job.n0 + wn * WTN;
    static_for<MI>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      static_for<NJ>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = j * 8 + 2 * q + hsel;
          const f32x16_t& Cv = acc[0][i][j];
          *reinterpret_cast<float4*>(buf + frag_row * 512 + ((ch ^ frag_row) << 4)) =
              make_float4(Cv[4 * q], Cv[4 * q + 1], Cv[4 * q + 2], Cv[4 * q + 3]);
        }
      });
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
              buf + r * 512 + (((col >> 2) ^ r) << 4) + (col & 3) * 4);
          if (cbase + col < job.N) atomicAdd(yrow + col, g * v);
        }
      }
    });
    return;
  }

  if constexpr (EPI == EPI_DSWIGLU) {
    // The SwiGLU backward of dh.  Per 32-row half, this wave's 32 x 128 fp32
    // dh go to its 16 KiB of the freed ring (rows of 512 bytes, 16-byte chunk
    // c of row r at c ^ r) and come back with lane l holding columns 4 (l % 32)
    // .. + 3 of one row, so g, u, dg, du and h move in contiguous runs of
    // that row.  With s = sigmoid(g): dg = dh u s (1 + g (1 - s)), du = dh g s,
    // h = g s u, each rounded to bf16; dg and du are then quantised per
    // 32-column block, which 8 neighbouring lanes hold, for the dX GEMM.
    // Compile-time loops keep every accumulator index constant (a rolled
    // loop would send the accumulators to scratch memory).
    static_assert(NB == 1 && WTN == 128, "dh epilogue: one B, 128 columns per wave");
    barrier();                                    // the ring is free
    char* buf = reinterpret_cast<char*>(ring) + wave * 16384;
    const int F = bw.F;
    const int cbase = job.n0 + wn * WTN;          // first dh column of this wave
    static_for<MI>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      static_for<NJ>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = j * 8 + 2 * q + hsel;
          const f32x16_t& D = acc[0][i][j];
          *reinterpret_cast<float4*>(buf + frag_row * 512 + ((ch ^ frag_row) << 4)) =
              make_float4(D[4 * q], D[4 * q + 1], D[4 * q + 2], D[4 * q + 3]);
        }
      });
      // The 16 passes go in groups of 4; a group's g, u loads are issued
      // before the previous group's stores (vmcnt counts loads and stores in
      // issue order: a load issued after a store would wait for it too).
      // Rows and columns past the tile read a valid element and store none.
      const int ch = lane & 31, n = cbase + 4 * ch;
      const int nc = n < job.N ? n : job.N - 4;   // N is a multiple of 32
      uint2 gqs[2][4], uqs[2][4];
      auto load_gu = [&](int grp, uint2 (&gq4)[4], uint2 (&uq4)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int m = job.m0 + wm * WTM + i * 32 + 2 * (4 * grp + u) + hsel;
          const long long rg = (long long)job.row0 + (m < job.rows ? m : job.rows - 1);
          gq4[u] = *reinterpret_cast<const uint2*>(bw.gu + rg * 2 * F + nc);
          uq4[u] = *reinterpret_cast<const uint2*>(bw.gu + rg * 2 * F + F + nc);
        }
      };
      load_gu(0, gqs[0], uqs[0]);
      static_for<4>([&](auto gc) __attribute__((always_inline)) {
        constexpr int grp = decltype(gc)::value;
        if constexpr (grp + 1 < 4) load_gu(grp + 1, gqs[(grp + 1) & 1], uqs[(grp + 1) & 1]);
#pragma unroll
        for (int pu = 0; pu < 4; ++pu) {
          const int r = 2 * (4 * grp + pu) + hsel;
          const float4 d4 = *reinterpret_cast<const float4*>(buf + r * 512 + ((ch ^ r) << 4));
          const int m = job.m0 + wm * WTM + i * 32 + r;
          const bool ok = m < job.rows && n < job.N;
          const long long rg = (long long)job.row0 + m;
          const uint2 gq = gqs[grp & 1][pu], uq = uqs[grp & 1][pu];
          const float dh[4] = {d4.x, d4.y, d4.z, d4.w};
          const uint32_t gw[2] = {gq.x, gq.y}, uw[2] = {uq.x, uq.y};
          float dg[4], du[4], hh[4];
          float ag = 0.0f, au = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t gb = gw[e >> 1], ub = uw[e >> 1];
            const float g = __uint_as_float((e & 1) ? (gb & 0xffff0000u) : (gb << 16));
            const float u = __uint_as_float((e & 1) ? (ub & 0xffff0000u) : (ub << 16));
            const float sg = 1.0f / (1.0f + __expf(-g));
            const float sl = g * sg;
            // rounded to bf16 here, so the quantised blocks see the stored values
            dg[e] = bf16_round(dh[e] * u * sg * (1.0f + g * (1.0f - sg)));
            du[e] = bf16_round(dh[e] * sl);
            hh[e] = sl * u;
            ag = fmaxf(ag, fabsf(dg[e]));
            au = fmaxf(au, fabsf(du[e]));
          }
#pragma unroll
          for (int x = 1; x < 8; x <<= 1) {
            ag = fmaxf(ag, __shfl_xor(ag, x, 64));
            au = fmaxf(au, __shfl_xor(au, x, 64));
          }
          const int sgx = mx_scale_exp(ag), sux = mx_scale_exp(au);
          const float ig = mx_inv_scale(sgx), iu = mx_inv_scale(sux);
          uint32_t cg = 0, cu = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            cg |= e4m3_code(dg[e] * ig) << (8 * e);
            cu |= e4m3_code(du[e] * iu) << (8 * e);
          }
          if (ok) {
            bf16_t* dgp = bw.dgu + rg * 2 * F + n;
            *reinterpret_cast<uint2*>(dgp) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
            *reinterpret_cast<uint2*>(dgp + F) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
            *reinterpret_cast<uint2*>(bw.h + rg * F + n) =
                make_uint2(pack_bf16x2(hh[0], hh[1]), pack_bf16x2(hh[2], hh[3]));
            uint8_t* cp = job.C + (long long)m * job.ldc + n;
            *reinterpret_cast<uint32_t*>(cp) = cg;
            *reinterpret_cast<uint32_t*>(cp + F) = cu;
            if ((lane & 7) == 0) {
              sC[(long long)m * (job.ldc / 32) + n / 32] = (uint8_t)(sgx + 127);
              sC[(long long)m * (job.ldc / 32) + (F + n) / 32] = (uint8_t)(sux + 127);
            }
          }
        }
      });
    });
    return;
  }

  if constexpr (EPI == EPI_WGRAD) {
    // a weight gradient: 4 consecutive fp32 (or bf16) values per lane and
    // 32-column block, straight from the accumulators; the group is job.row0
    const int Mrest = job.rows - bw.wsplit;
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int m = job.m0 + wm * WTM + i * 32 + frag_row;
      if (!live || m >= job.rows) continue;
      const long long row = m < bw.wsplit
                                ? ((long long)job.row0 * bw.wsplit + m) * job.N
                                : ((long long)job.row0 * Mrest + (m - bw.wsplit)) * job.N;
      void* base = m < bw.wsplit ? bw.w0 : bw.w1;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int nblk = job.n0 + wn * WTN + j * 32;
        if (nblk >= job.N) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nblk + 8 * q + 4 * hsel;
          const f32x16_t& Cv = acc[0][i][j];
          if (bw.wbf16)
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(base) + row + n) =
                make_uint2(pack_bf16x2(Cv[4 * q], Cv[4 * q + 1]),
                           pack_bf16x2(Cv[4 * q + 2], Cv[4 * q + 3]));
          else
            *reinterpret_cast<float4*>(static_cast<float*>(base) + row + n) =
                make_float4(Cv[4 * q], Cv[4 * q + 1], Cv[4 * q + 2], Cv[4 * q + 3]);
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
    const bool row_ok = m < job.rows;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nblk = job.n0 + wn * WTN + j * 32;          // 32-column block
      if (nblk >= job.N) continue;                          // N is a multiple of 32
      if constexpr (EPI == EPI_SWIGLU) {
        // h = silu(g) * u, one MX block per (row, 32 columns): the lane pair
        // (l, l + 32) holds the block's 32 values.
        const f32x16_t& G = acc[0][i][j];
        const f32x16_t& U = acc[NB - 1][i][j];
        float hv[16];
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          hv[v] = silu_fast(G[v]) * U[v];
          amax = fmaxf(amax, fabsf(hv[v]));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const int s = mx_scale_exp(amax);
        const float inv = mx_inv_scale(s);
        uint32_t d[4];   // d[q]: columns 8 q + 4 hsel + (0..3)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t w = 0;
#pragma unroll
          for (int r = 0; r < 4; ++r) w |= e4m3_code(hv[4 * q + r] * inv) << (8 * r);
          d[q] = w;
        }
        // Lane l (hsel 0) gathers columns 0-15 of the block, lane l + 32
        // columns 16-31: each sends the two dwords the other needs.
        const uint32_t x0 = __shfl_xor(hsel ? d[0] : d[2], 32, 64);
        const uint32_t x1 = __shfl_xor(hsel ? d[1] : d[3], 32, 64);
        const uint4 out = hsel ? make_uint4(x0, d[2], x1, d[3]) : make_uint4(d[0], x0, d[1], x1);
        if (row_ok) {
          *reinterpret_cast<uint4*>(job.C + (long long)m * job.ldc + nblk + 16 * hsel) = out;
          if (hsel == 0) sC[(long long)m * (job.N / 32) + nblk / 32] = (uint8_t)(s + 127);
        }
      } else {
        if (!row_ok) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nblk + 8 * q + 4 * hsel;
          const f32x16_t& Cv = acc[0][i][j];
          const uint2 pk = make_uint2(pack_bf16x2(Cv[4 * q], Cv[4 * q + 1]),
                                      pack_bf16x2(Cv[4 * q + 2], Cv[4 * q + 3]));
          *reinterpret_cast<uint2*>(job.C + (long long)m * job.ldc + n) = pk;
        }
      }
    }
  }
}


template <int BM, int BN, int NB, int EPI, int WM, int WN, int SG, int TL>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_mx_kernel(const GemmArgs args, const MxScales sc, const MxBwd bw) {
  using S0 = MxShape<BM, BN, NB, WM, WN, SG, 0>;
  using S1 = MxShape<BM, BN, NB, WM, WN, SG, 1>;
  constexpr int RING = (TL && S1::RING > S0::RING) ? S1::RING : S0::RING;
  constexpr int SRING = (TL && S1::SRING > S0::SRING) ? S1::SRING : S0::SRING;
  static_assert(RING + SRING + 64 <= 160 * 1024, "LDS");
  using TOut = MxOut<EPI>;
  // the operand ring, and beside it the scale slices (+64 bytes: the last
  // step's unused read of a next step may touch a byte past the end)
  __shared__ __attribute__((aligned(1024))) uint8_t ring[RING];
  __shared__ __attribute__((aligned(1024))) uint8_t sring[SRING + 64];
  TileJob<uint8_t, TOut> job;
  if (!decode_tile<BM, BN>(args, job)) return;
  if (TL && __builtin_amdgcn_readfirstlane(job.cls) != 0)
    mx_tile<BM, BN, NB, EPI, WM, WN, SG, 1>(args, sc, bw, job, ring, sring);
  else
    mx_tile<BM, BN, NB, EPI, WM, WN, SG, 0>(args, sc, bw, job, ring, sring);
}

// Scale loads are grouped eight K steps at a time when every group of the
// launch has at least 16 scale bytes per row (K >= 512).
template <int BM, int BN, int NB, int EPI, int WM, int WN>
hipError_t launch_mx_gemm(const GemmArgs& a, const MxScales& sc, int R, hipStream_t st,
                          const MxBwd& bw = MxBwd{}) {
  const int grid = grid_upper_bound(a, BM, BN, R);
  if (grid == 0) return hipSuccess;
  const bool grouped = (a.E == 0 || a.K >= 512) && (a.Td == 0 || a.Kd >= 512);
  if (grouped)
    gemm_mx_kernel<BM, BN, NB, EPI, WM, WN, 8, 1><<<grid, 64 * WM * WN, 0, st>>>(a, sc, bw);
  else
    gemm_mx_kernel<BM, BN, NB, EPI, WM, WN, 1, 1><<<grid, 64 * WM * WN, 0, st>>>(a, sc, bw);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP8 weight gradients (Primus blog, low-precision section: the permuted
// tokens are padded to the quantisation block boundary).  A weight gradient
// contracts over an expert's rows, so its operands are quantised along the
// rows, in 32-row blocks from the expert's first row.  Each expert's row
// count is padded to a multiple of 128 (the GEMM's scale granularity: one
// scale dword per row covers two 64-value steps) with zero rows, which
// change no block maximum and add nothing to the sums.
//
//   pad_offsets:   poffs[e] = sum over e' < e of the padded row counts
//   quantize_tok:  src [R, C] bf16 (rows grouped by offsets) -> codes
//                  [C, ldq] and scales [C, ldq / 32]: padded row P of
//                  expert e is source row offsets[e] + P - poffs[e] when
//                  that row is the expert's, else zero
//   wgrad GEMM:    per expert, dW[e][m, n] = sum_k A_q[m, k] B_q[n, k]
//                  over its padded rows k, on the scaled MFMA
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(1024)
pad_offsets_kernel(const int32_t* __restrict__ offsets, int E, int32_t* __restrict__ poffs) {
  __shared__ int s[1024];
  const int g = threadIdx.x;
  int v = 0;
  if (g < E) {
    const int c = offsets[g + 1] - offsets[g];
    v = (c + 127) / 128 * 128;
  }
  s[g] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int a = (g >= off) ? s[g - off] : 0;
    __syncthreads();
    s[g] += a;
    __syncthreads();
  }
  for (int i = g; i <= E; i += 1024) poffs[i] = (i == 0) ? 0 : s[i - 1];
}

// A workgroup takes 128 padded rows x 64 columns (one expert's rows: the
// padded counts are multiples of 128) through LDS, 16-byte loads of whole
// 128-byte row segments; thread (block b, column c) then quantises the 32
// rows of block b of column c, so each column's 128 codes leave as one full
// 128-byte line written by four neighbouring threads.  Callers pass cols a
// multiple of 8.  Row blocks past poffs[E] exit: the GEMM reads only the
// padded rows of each expert.
__global__ void __launch_bounds__(256)
mx_quantize_tok_kernel(const bf16_t* __restrict__ src, int cols,
                       const int32_t* __restrict__ offsets, const int32_t* __restrict__ poffs,
                       int E, long long ldq, uint8_t* __restrict__ q, uint8_t* __restrict__ sq) {
  __shared__ bf16_t tile[128][64 + 8];          // rows of 144 bytes: 16-byte aligned
  const int P0 = blockIdx.y * 128, c0 = blockIdx.x * 64;
  if (P0 >= poffs[E]) return;
  // the expert of padded row P0: largest e with poffs[e] <= P0
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poffs[mid] <= P0) lo = mid; else hi = mid - 1;
  }
  const int r0 = offsets[lo] + (P0 - poffs[lo]);
  const int rend = offsets[lo + 1];
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rr = (tid >> 3) + 32 * u, ch = tid & 7;
    const int r = r0 + rr, c = c0 + 8 * ch;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);      // rows past the expert and columns past cols: 0
    if (r < rend && c < cols) v = *reinterpret_cast<const uint4*>(src + (long long)r * cols + c);
    *reinterpret_cast<uint4*>(&tile[rr][8 * ch]) = v;
  }
  __syncthreads();
  const int cc = tid & 63, b = tid >> 6;
  float v[32];
  float amax = 0.0f;
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    v[p] = to_f32<bf16_t>(tile[32 * b + p][cc]);
    amax = fmaxf(amax, fabsf(v[p]));
  }
  const int sx = mx_scale_exp(amax);
  const float inv = mx_inv_scale(sx);
  uint32_t w[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t x = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) x |= e4m3_code(v[4 * g + p] * inv) << (8 * p);
    w[g] = x;
  }
  const int c = c0 + cc;
  if (c < cols) {
    uint4* dst = reinterpret_cast<uint4*>(q + (long long)c * ldq + P0 + 32 * b);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    sq[(long long)c * (ldq / 32) + P0 / 32 + b] = (uint8_t)(sx + 127);
  }
}

// Weight-gradient tiles: per expert a fixed grid of ceil(Mw / BM) x
// ceil(N / BN) tiles, row tiles adjacent; each XCD walks a contiguous range.
// A and B are the quantised operands (rows of lda padded-row codes); a
// tile's K is its expert's padded row count, starting at poffs[e].
template <int BM, int BN>
__device__ __forceinline__ bool decode_wgrad_tile(const GemmArgs& a,
                                                  TileJob<uint8_t, bf16_t>& j) {
  const int mt = cdiv(a.Mw, BM), nt = cdiv(a.N, BN);
  const int total = a.E * mt * nt;
  const int per = (total + 7) >> 3, slot = blockIdx.x >> 3;
  if (slot >= per) return false;
  const int lid = (blockIdx.x & 7) * per + slot;
  if (lid >= total) return false;
  const int g = lid / (mt * nt), r = lid - g * (mt * nt);
  const int p0 = a.offsets[g];
  j.m0 = (r % mt) * BM;
  j.n0 = (r / mt) * BN;
  j.A = static_cast<const uint8_t*>(a.A) + p0;
  j.lda = a.lda;
  j.gather = nullptr;
  j.rows = a.Mw;
  j.B0 = static_cast<const uint8_t*>(a.B0) + p0;
  j.B1 = nullptr;
  j.N = a.N;
  j.K = a.offsets[g + 1] - p0;
  j.k0 = 0;
  j.klen = j.K;
  j.C = nullptr;
  j.ldc = a.N;
  j.GU = nullptr;
  j.ldgu = 0;
  j.P = nullptr;
  j.cls = 0;
  j.dense = 0;
  j.row0 = g;                 // EPI_WGRAD: the expert
  j.ctok = nullptr;
  j.cgate = nullptr;
  return true;
}

template <int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_mx_wgrad_kernel(const GemmArgs args, const MxScales sc, const MxBwd bw) {
  using S0 = MxShape<BM, BN, 1, WM, WN, 1, 0>;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[S0::RING];
  __shared__ __attribute__((aligned(1024))) uint8_t sring[S0::SRING + 64];
  TileJob<uint8_t, bf16_t> job;
  if (!decode_wgrad_tile<BM, BN>(args, job)) return;
  mx_tile<BM, BN, 1, EPI_WGRAD, WM, WN, 1, 0>(args, sc, bw, job, ring, sring);
}

hipError_t launch_mx_wgrad(const MxWgrad& g, hipStream_t st) {
  if (g.E == 0) return hipSuccess;
  pad_offsets_kernel<<<1, 1024, 0, st>>>(g.offsets, g.E, g.poffs);
  const unsigned yb = (unsigned)(g.wrows / 128);   // wrows: a multiple of 128
  mx_quantize_tok_kernel<<<dim3(cdiv(g.M, 64), yb), 256, 0, st>>>(
      static_cast<const bf16_t*>(g.A), g.M, g.offsets, g.poffs, g.E, g.wrows, g.qa, g.sa);
  mx_quantize_tok_kernel<<<dim3(cdiv(g.N, 64), yb), 256, 0, st>>>(
      static_cast<const bf16_t*>(g.B), g.N, g.offsets, g.poffs, g.E, g.wrows, g.qb, g.sb);
  GemmArgs a = {};
  MxScales sc = {};
  a.E = g.E;
  a.offsets = g.poffs;
  a.A = g.qa;
  a.lda = g.wrows;
  a.B0 = g.qb;
  a.N = g.N;
  a.K = 0;
  a.Mw = g.M;
  sc.A = g.sa;
  sc.B0 = g.sb;
  MxBwd bw = {};
  bw.w0 = g.w0;
  bw.w1 = g.w1;
  bw.wsplit = g.wsplit;
  bw.wbf16 = g.wbf16;
  const long long tiles = (long long)g.E * cdiv(g.M, MX_FC2_BM) * cdiv(g.N, MX_FC2_BN);
  const int grid = (int)(((tiles + 7) / 8) * 8);
  gemm_mx_wgrad_kernel<MX_FC2_BM, MX_FC2_BN, 4, 2><<<grid, 512, 0, st>>>(a, sc, bw);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn_mxfp8(const moe_shape& s, const uint8_t* xq, const uint8_t* xs,
                                    const int32_t* row_token, const int32_t* offsets,
                                    const MxWeights& w, void* y_perm, void* y_shared,
                                    const MxFfnWs& ws, hipStream_t st, const float* row_gate,
                                    float* y) {
  const int R = s.T * s.k;
  const bool shared = s.F_shared > 0 && s.T > 0;
  GemmArgs a1 = {};
  MxScales s1 = {};
  a1.E = R > 0 ? s.E : 0;
  a1.offsets = offsets;
  a1.tiles = ws.tiles1;
  a1.A = xq;
  a1.gather = row_token;
  a1.lda = s.d;
  a1.B0 = w.gate_q;
  a1.B1 = w.up_q;
  a1.strideB = (long long)s.F * s.d;
  a1.N = s.F;
  a1.K = s.d;
  a1.C = ws.hq;
  a1.ldc = s.F;
  s1.A = xs;
  s1.B0 = w.gate_s;
  s1.B1 = w.up_s;
  s1.C = ws.hs;
  if (shared) {
    a1.Td = s.T;
    a1.Ad = xq;
    a1.ldad = s.d;
    a1.Bd0 = w.sgate_q;
    a1.Bd1 = w.sup_q;
    a1.Nd = s.F_shared;
    a1.Kd = s.d;
    a1.Cd = ws.shq;
    a1.ldcd = s.F_shared;
    s1.Ad = xs;
    s1.Bd0 = w.sgate_s;
    s1.Bd1 = w.sup_s;
    s1.Cd = ws.shs;
  }
  GemmArgs a2 = {};
  MxScales s2 = {};
  a2.E = a1.E;
  a2.offsets = offsets;
  a2.tiles = ws.tiles2;
  a2.A = ws.hq;
  a2.lda = s.F;
  a2.B0 = w.down_q;
  a2.strideB = (long long)s.d * s.F;
  a2.N = s.d;
  a2.K = s.F;
  a2.C = y_perm;
  a2.ldc = s.d;
  s2.A = ws.hs;
  s2.B0 = w.down_s;
  if (shared) {
    a2.Td = s.T;
    a2.Ad = ws.shq;
    a2.ldad = s.F_shared;
    a2.Bd0 = w.sdown_q;
    a2.Nd = s.d;
    a2.Kd = s.F_shared;
    a2.Cd = y_shared;
    a2.ldcd = s.d;
    s2.Ad = ws.shs;
    s2.Bd0 = w.sdown_s;
  }
  if (y) {
    // the combine in FC2's epilogue: y = 0, then every FC2 row adds its
    // gate-scaled output into its token's row (the shared expert's with gate 1)
    const long long ny = (long long)s.T * s.d;
    if (ny == 0) return hipSuccess;
    hipError_t e = launch_zero_f32(y, ny, st);
    if (e != hipSuccess) return e;
    a2.C = nullptr;
    a2.Cd = nullptr;
    a2.comb_token = row_token;
    a2.comb_gate = row_gate;
    a2.Y = y;
    a2.ldy = s.d;
  }
  if (a1.E == 0 && !shared) return hipSuccess;
  // routed groups use tail tiles (BM/2 x 2BN) for their last rows
  a1.tail = a2.tail = 1;
  if (a1.E > 0) {
    schedule_tiles_kernel<<<1, 1024, 0, st>>>(offsets, s.E, MX_FC1_BM, cdiv(s.F, MX_FC1_BN),
                                              ws.tiles1, MX_FC2_BM, cdiv(s.d, MX_FC2_BN),
                                              ws.tiles2, 1);
  }
  hipError_t e = launch_mx_gemm<MX_FC1_BM, MX_FC1_BN, 2, EPI_SWIGLU, 4, 2>(a1, s1, R, st);
  if (e != hipSuccess) return e;
  if (y) return launch_mx_gemm<MX_FC2_BM, MX_FC2_BN, 1, EPI_COMBINE, 4, 2>(a2, s2, R, st);
  return launch_mx_gemm<MX_FC2_BM, MX_FC2_BN, 1, EPI_STORE, 4, 2>(a2, s2, R, st);
}

// The backward's two data-gradient GEMMs over the routed groups (or one
// group of all tokens for the shared expert): dh with the SwiGLU-backward
// epilogue, then dX_perm.  F and d are multiples of 128.
hipError_t launch_mx_dgrad(const moe_shape& s, const MxDgrad& g, hipStream_t st) {
  const int R = g.rows;
  GemmArgs a1 = {};
  MxScales s1 = {};
  a1.E = R > 0 ? s.E : 0;
  a1.offsets = g.offsets;
  a1.tiles = g.tiles1;
  a1.A = g.dyq;
  a1.lda = s.d;
  a1.B0 = g.wd_tq;
  a1.strideB = (long long)s.F * s.d;
  a1.N = s.F;
  a1.K = s.d;
  a1.C = g.dguq;
  a1.ldc = 2 * s.F;
  s1.A = g.dys;
  s1.B0 = g.wd_ts;
  s1.C = g.dgus;
  MxBwd bw;
  bw.gu = static_cast<const bf16_t*>(g.gu);
  bw.dgu = static_cast<bf16_t*>(g.dgu);
  bw.h = static_cast<bf16_t*>(g.h);
  bw.F = s.F;
  GemmArgs a2 = {};
  MxScales s2 = {};
  a2.E = a1.E;
  a2.offsets = g.offsets;
  a2.tiles = g.tiles2;
  a2.A = g.dguq;
  a2.lda = 2 * s.F;
  a2.B0 = g.wgu_tq;
  a2.strideB = (long long)s.d * 2 * s.F;
  a2.N = s.d;
  a2.K = 2 * s.F;
  a2.C = g.dX;
  a2.ldc = s.d;
  s2.A = g.dgus;
  s2.B0 = g.wgu_ts;
  if (a1.E == 0) return hipSuccess;
  schedule_tiles_kernel<<<1, 1024, 0, st>>>(g.offsets, s.E, MX_FC2_BM, cdiv(s.F, MX_FC2_BN),
                                            g.tiles1, MX_FC2_BM, cdiv(s.d, MX_FC2_BN), g.tiles2, 1);
  a1.tail = a2.tail = 1;
  hipError_t e = launch_mx_gemm<MX_FC2_BM, MX_FC2_BN, 1, EPI_DSWIGLU, 4, 2>(a1, s1, R, st, bw);
  if (e != hipSuccess) return e;
  return launch_mx_gemm<MX_FC2_BM, MX_FC2_BN, 1, EPI_STORE, 4, 2>(a2, s2, R, st);
}

}  // namespace moe
