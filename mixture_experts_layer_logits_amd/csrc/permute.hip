// Padding-free permutation into expert-contiguous order: expert histogram,
// exclusive prefix scan, stable scatter (Primus blog, MegaMoE section: the
// tokens are reordered so that each expert's rows sit together; the buffer
// holds only routed rows, as in the padding-free token buffer of the X-MoE
// verdict page).
//
// Row order is (expert, token) ascending, so every index is fixed by the
// routing alone and no atomic decides a position:
//   pos[t, j] = offsets[e] + #{t' < t : e in topk_idx[t']},  e = topk_idx[t, j].
//
// Tokens are cut into blocks of 256 (one workgroup, four 64-token waves).  A
// wave marks, per expert, which of its 64 tokens picked that expert in a
// 64-bit mask in LDS (bitwise OR is order-free); the rank of a token among
// the wave's tokens that picked e is then popcount(mask & lanes-below).
//   1. count:  per (expert, block) counts, stored expert-major;
//   2. scan:   one exclusive scan over that expert-major array gives each
//              (expert, block) its first row and, at block 0, the offsets;
//   3. maps:   token_row, row_token and row_gate from the masks again.
//              When the count table is small (at most 64 blocks and 16384
//              entries) each maps block does step 2 itself from the whole
//              table, which saves the scan launch;
//   4. rows:   one workgroup per token copies x[t] once from HBM into its k
//              destination rows (full-row, 16-byte coalesced stores).  Without
//              an x_perm buffer this step is skipped: the grouped FFN can read
//              each row from x through row_token instead.
#include <mutex>

#include "gemm_tiles.h"

namespace moe {

constexpr int PB = 256;  // tokens per block

int permute_nblk(const moe_shape& s) { return cdiv(s.T, PB); }

// Fills masks[4][E] (one per wave) for the block's tokens.
__device__ __forceinline__ void build_masks(unsigned long long* masks, const int32_t* idx,
                                            int T, int E, int k, int blk) {
  for (int e = threadIdx.x; e < 4 * E; e += PB) masks[e] = 0ull;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blk * PB + threadIdx.x;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(long long)t * k + j];
      if (e >= 0 && e < E) atomicOr(&masks[wave * E + e], 1ull << lane);
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(PB)
permute_count_kernel(const int32_t* __restrict__ idx, int T, int E, int k, int nblk,
                     int32_t* __restrict__ blk_cnt) {
  extern __shared__ unsigned long long masks[];
  build_masks(masks, idx, T, E, k, blockIdx.x);
  for (int e = threadIdx.x; e < E; e += PB) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) c += __popcll(masks[w * E + e]);
    blk_cnt[(long long)e * nblk + blockIdx.x] = c;
  }
}

// Exclusive scan of n = E * nblk counts (expert-major) by one workgroup of
// 1024 threads, each owning a contiguous run.
__global__ void __launch_bounds__(1024)
permute_scan_kernel(const int32_t* __restrict__ blk_cnt, int E, int nblk,
                    int32_t* __restrict__ blk_base, int32_t* __restrict__ offsets) {
  __shared__ int s[1024];
  const int n = E * nblk;
  const int per = cdiv(n, 1024);
  const int tid = threadIdx.x;
  const int lo = min(n, tid * per), hi = min(n, lo + per);
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += blk_cnt[i];
  s[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += v;
    __syncthreads();
  }
  int run = tid > 0 ? s[tid - 1] : 0;
  for (int i = lo; i < hi; ++i) {
    blk_base[i] = run;
    run += blk_cnt[i];
  }
  __syncthreads();
  // offsets[e] = first row of expert e = base of (e, block 0); offsets[E] = R
  for (int e = tid; e <= E; e += 1024)
    offsets[e] = (e < E) ? (nblk > 0 ? blk_base[(long long)e * nblk] : 0) : s[1023];
}

constexpr int FUSE_MAX_BLK = 64, FUSE_MAX_ENTRIES = 16384;

bool permute_fused_scan(const moe_shape& s) {
  const int nblk = permute_nblk(s);
  return nblk > 0 && nblk <= FUSE_MAX_BLK && (long long)nblk * s.E <= FUSE_MAX_ENTRIES;
}

// First row of (expert, this block) for every expert, from the whole
// expert-major count table: base[e] = sum of all blocks' counts of experts
// below e, plus the counts of expert e in blocks below this one.  Block 0
// also writes offsets.  E <= 1024.
__device__ void block_bases(const int32_t* __restrict__ blk_cnt, int E, int nblk, int blk,
                            int* __restrict__ base, int32_t* __restrict__ offsets) {
  __shared__ int s_tot[1024];
  __shared__ int s_part[PB];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += PB) {
    const int32_t* row = blk_cnt + (long long)e * nblk;
    int tot = 0, pre = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = row[b];
      pre += (b < blk) ? c : 0;
      tot += c;
    }
    s_tot[e] = tot;
    base[e] = pre;
  }
  __syncthreads();
  // exclusive scan of s_tot: thread tid owns experts [4 tid, 4 tid + 4)
  const int e0 = 4 * tid;
  int run = 0;
  for (int e = e0; e < e0 + 4 && e < E; ++e) run += s_tot[e];
  s_part[tid] = run;
  __syncthreads();
  for (int off = 1; off < PB; off <<= 1) {
    const int v = tid >= off ? s_part[tid - off] : 0;
    __syncthreads();
    s_part[tid] += v;
    __syncthreads();
  }
  int excl = tid > 0 ? s_part[tid - 1] : 0;
  for (int e = e0; e < e0 + 4 && e < E; ++e) {
    if (blk == 0) offsets[e] = excl;
    base[e] += excl;
    excl += s_tot[e];
  }
  if (blk == 0 && tid == PB - 1) offsets[E] = s_part[PB - 1];
  __syncthreads();
}

__global__ void __launch_bounds__(PB)
permute_maps_kernel(const int32_t* __restrict__ idx, const float* __restrict__ w, int T,
                    int E, int k, int nblk, const int32_t* __restrict__ blk_base,
                    const int32_t* __restrict__ blk_cnt, int32_t* __restrict__ offsets,
                    int32_t* __restrict__ row_token, int32_t* __restrict__ token_row,
                    float* __restrict__ row_gate) {
  extern __shared__ unsigned long long masks[];
  __shared__ int s_base[1024];
  if (blk_cnt) block_bases(blk_cnt, E, nblk, blockIdx.x, s_base, offsets);
  build_masks(masks, idx, T, E, k, blockIdx.x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * PB + threadIdx.x;
  if (t >= T) return;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int j = 0; j < k; ++j) {
    const long long tj = (long long)t * k + j;
    const int e = idx[tj];
    if (e < 0 || e >= E) {
      token_row[tj] = -1;
      continue;
    }
    int pos = blk_cnt ? s_base[e] : blk_base[(long long)e * nblk + blockIdx.x];
    for (int v = 0; v < wave; ++v) pos += __popcll(masks[v * E + e]);
    pos += __popcll(masks[wave * E + e] & below);
    token_row[tj] = pos;
    row_token[pos] = t;
    row_gate[pos] = w[tj];
  }
}

// One workgroup per token: read x[t] once, write it to its k rows.
template <bool VEC>
__global__ void __launch_bounds__(256)
permute_rows_kernel(const uint8_t* __restrict__ x, const int32_t* __restrict__ token_row,
                    int k, long long row_bytes, uint8_t* __restrict__ x_perm) {
  const int t = blockIdx.x;
  const int32_t* rows = token_row + (long long)t * k;  // uniform loads
  const uint8_t* src = x + (long long)t * row_bytes;
  if (VEC) {
    const long long nseg = row_bytes / 16;
    for (long long sgi = threadIdx.x; sgi < nseg; sgi += 256) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[sgi];
      for (int j = 0; j < k; ++j) {
        const int r = rows[j];
        if (r >= 0) reinterpret_cast<uint4*>(x_perm + (long long)r * row_bytes)[sgi] = v;
      }
    }
  } else {
    for (long long b = threadIdx.x; b < row_bytes; b += 256) {
      const uint8_t v = src[b];
      for (int j = 0; j < k; ++j) {
        const int r = rows[j];
        if (r >= 0) x_perm[(long long)r * row_bytes + b] = v;
      }
    }
  }
}

hipError_t launch_permute(const moe_shape& s, const void* x, const int32_t* topk_idx,
                          const float* topk_w, int32_t* offsets, int32_t* row_token,
                          int32_t* token_row, float* row_gate, void* x_perm,
                          const PermuteWs& ws, hipStream_t st) {
  const int nblk = permute_nblk(s);
  const size_t lds = sizeof(unsigned long long) * 4 * s.E;
  if (nblk > 0) {
    permute_count_kernel<<<nblk, PB, lds, st>>>(topk_idx, s.T, s.E, s.k, nblk, ws.blk_cnt);
  }
  const bool fused = permute_fused_scan(s);
  if (!fused)
    permute_scan_kernel<<<1, 1024, 0, st>>>(ws.blk_cnt, s.E, nblk, ws.blk_base, offsets);
  if (nblk > 0) {
    permute_maps_kernel<<<nblk, PB, lds, st>>>(topk_idx, topk_w, s.T, s.E, s.k, nblk,
                                               ws.blk_base, fused ? ws.blk_cnt : nullptr,
                                               offsets, row_token, token_row, row_gate);
    const long long row_bytes = (long long)s.d * (s.dtype == MOE_DTYPE_BF16 ? 2 : 4);
    if (!x_perm) return hipGetLastError();   // maps only (FC1 gathers the rows)
    if (row_bytes % 16 == 0)
      permute_rows_kernel<true><<<s.T, 256, 0, st>>>(static_cast<const uint8_t*>(x), token_row,
                                                     s.k, row_bytes,
                                                     static_cast<uint8_t*>(x_perm));
    else
      permute_rows_kernel<false><<<s.T, 256, 0, st>>>(static_cast<const uint8_t*>(x), token_row,
                                                      s.k, row_bytes,
                                                      static_cast<uint8_t*>(x_perm));
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// A fixed scratch area for callers that cannot allocate (moe_permute_noalloc):
// the per-(expert, block) counts and first rows, 2 x 2^18 int32 (2 MiB).
// Each GPU holds its own copy for the life of the process; its device
// address is looked up once per device with that device current, and only
// that address is ever handed to kernels.  Every entry the kernels read is
// written earlier in the same call (counts by the count kernel, bases by the
// scan), so nothing needs clearing; calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) int32_t scratch[2 * PERMUTE_NOALLOC_MAX_ENTRIES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t permute_noalloc_ws(PermuteWs& ws) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  ws.blk_cnt = g_scratch_ptr[dev];
  ws.blk_base = g_scratch_ptr[dev] + PERMUTE_NOALLOC_MAX_ENTRIES;
  return hipSuccess;
}

}  // namespace moe
