// C ABI of the MoE layer: argument validation, workspace layout and launch
// sequencing.  Every check happens before anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "../../include/moe.h"
#include "moe_common.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t esize(const moe_shape& s) { return s.dtype == MOE_DTYPE_BF16 ? 2 : 4; }

int check_shape(const moe_shape* sp) {
  if (!sp) return MOE_ERR_INVALID_ARG;
  const moe_shape& s = *sp;
  if (s.T < 0 || s.d < 1 || s.E < 1 || s.E > 1024 || s.k < 1 || s.k > 64 || s.k > s.E ||
      s.F < 1 || s.F_shared < 0)
    return MOE_ERR_INVALID_ARG;
  if (s.n_groups < 1 || s.n_groups > 64 || s.E % s.n_groups != 0) return MOE_ERR_INVALID_ARG;
  if (s.topk_groups < 1 || s.topk_groups > s.n_groups) return MOE_ERR_INVALID_ARG;
  if ((long long)s.topk_groups * (s.E / s.n_groups) < s.k) return MOE_ERR_INVALID_ARG;
  if (s.score != MOE_SCORE_SOFTMAX && s.score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (s.n_groups > 1 && s.score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (s.renorm != 0 && s.renorm != 1) return MOE_ERR_INVALID_ARG;
  if (s.dtype != MOE_DTYPE_F32 && s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.wgrad_dtype != MOE_DTYPE_F32 && s.wgrad_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.wgrad_mx != 0 && s.wgrad_mx != 1) return MOE_ERR_INVALID_ARG;
  // Row indices are int32.  Arrays of R routed rows are addressed with
  // 64-bit row offsets (the tile kernels fold each load block's first row
  // into a 64-bit base), so only arrays indexed by absolute token row in
  // 32 bits (x gathered by the fused permutation, logits) and one expert's
  // weight matrix bound the products.
  const long long R = (long long)s.T * s.k;
  const long long wide = std::max<long long>({s.d, s.F, s.F_shared, s.E, 2LL * s.F});
  if (R >= (1LL << 31) || (long long)s.T * wide >= (1LL << 31)) return MOE_ERR_INVALID_ARG;
  if ((long long)s.F * s.d >= (1LL << 31)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// A buffer of `bytes` bytes: may be null only when empty; 16-byte aligned.
bool ok_buf(const void* p, long long bytes) {
  if (bytes <= 0) return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
}

// Rows of the MXFP8 weight gradients' token-axis operands: every expert's
// row count padded to a multiple of 128 (at most R + 127 E), and the shared
// expert's T rows padded the same way.
size_t mx_wgrad_rows(const moe_shape& s) {
  const size_t R = (size_t)s.T * s.k;
  const size_t routed = (R + 127 * (size_t)s.E + 127) / 128 * 128;
  const size_t shared = ((size_t)s.T + 127) / 128 * 128;
  return std::max(routed, shared);
}

size_t ws_bytes_for(const moe_shape& s, int op) {
  const size_t R = (size_t)s.T * s.k;
  const size_t es = esize(s);
  switch (op) {
    case MOE_OP_ROUTE: {   // the split router GEMM's partial sums
      const int ks = moe::router_ksplit(s);
      return ks > 1 ? align_up((size_t)ks * s.T * s.E * 4) : 0;
    }
    case MOE_OP_COMBINE:
      return 0;
    case MOE_OP_PERMUTE: {
      const size_t n = (size_t)s.E * moe::permute_nblk(s);
      return 2 * align_up(n * 4);
    }
    case MOE_OP_FFN: {
      const int ks = moe::ffn_fc2_ksplit(s);
      return 2 * align_up((s.E + 1) * 4) + align_up(R * s.F * es) +
             align_up((size_t)s.T * s.F_shared * es) +
             (ks > 1 ? align_up((size_t)ks * R * s.d * 4) : 0);
    }
    case MOE_OP_BACKWARD:
    case MOE_OP_BACKWARD_RECOMPUTE: {
      size_t b = 2 * align_up((s.E + 1) * 4) + 2 * align_up(R * s.d * es) +
                 align_up(R * 2 * s.F * es) + align_up(R * s.F * es);
      if (s.F_shared > 0) {
        const size_t T = (size_t)s.T, Fs = (size_t)s.F_shared;
        b += 3 * align_up(2 * 4) + align_up(T * 2 * Fs * es) + align_up(T * Fs * es) +
             align_up(T * s.d * es);
      }
      if (op == MOE_OP_BACKWARD_RECOMPUTE)   // the recomputed g | u
        b += align_up((R * 2 * s.F + (size_t)s.T * 2 * s.F_shared) * es);
      return b;
    }
    case MOE_OP_BACKWARD_MXFP8: {   // the bf16 backward's, plus the quantised GEMM inputs
      size_t b = ws_bytes_for(s, MOE_OP_BACKWARD);
      b += align_up(R * s.d) + align_up(R * s.d / 32) + align_up(R * 2 * s.F) +
           align_up(R * 2 * s.F / 32);
      if (s.F_shared > 0) {
        const size_t T = (size_t)s.T, Fs = (size_t)s.F_shared;
        b += align_up(T * s.d) + align_up(T * s.d / 32) + align_up(T * 2 * Fs) +
             align_up(T * 2 * Fs / 32);
      }
      if (s.wgrad_mx) {
        // padded row offsets, and the two operands of one weight-gradient
        // GEMM quantised along the padded rows (reused by the next GEMM)
        const size_t rp = mx_wgrad_rows(s);
        const size_t ma = std::max<size_t>({(size_t)s.d, 2 * (size_t)s.F, 2 * (size_t)s.F_shared});
        const size_t mb = std::max<size_t>({(size_t)s.d, (size_t)s.F, (size_t)s.F_shared});
        b += 2 * align_up((s.E + 1) * 4) + align_up(ma * rp) + align_up(ma * rp / 32) +
             align_up(mb * rp) + align_up(mb * rp / 32);
      }
      return b;
    }
    case MOE_OP_FFN_COMBINE:   // no split-K partials: slices add into y
      return 2 * align_up((s.E + 1) * 4) + align_up(R * s.F * es) +
             align_up((size_t)s.T * s.F_shared * es);
    case MOE_OP_FFN_MXFP8:
      return 2 * align_up((s.E + 1) * 4) + align_up(R * s.F) + align_up(R * s.F / 32) +
             align_up((size_t)s.T * s.F_shared) + align_up((size_t)s.T * s.F_shared / 32);
    default:
      return 0;
  }
}

int check_ws(const moe_shape& s, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(s, op);
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 15) != 0) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

struct Carver {
  char* p;
  template <typename T>
  T* take(size_t bytes) {
    T* r = reinterpret_cast<T*>(p);
    p += align_up(bytes);
    return r;
  }
};

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The backward's workspace pieces, in MOE_OP_BACKWARD's order.
void carve_backward(const moe_shape& s, Carver& c, moe::BwdWs& bw) {
  const size_t R = (size_t)s.T * s.k, es = esize(s);
  bw = moe::BwdWs{};
  bw.tiles = c.take<int32_t>((s.E + 1) * 4);
  bw.tiles2 = c.take<int32_t>((s.E + 1) * 4);
  bw.dY = c.take<char>(R * s.d * es);
  bw.dX = c.take<char>(R * s.d * es);
  bw.dgu = c.take<char>(R * 2 * s.F * es);
  bw.h = c.take<char>(R * s.F * es);
  if (s.F_shared > 0) {
    bw.s_offsets = c.take<int32_t>(2 * 4);
    bw.s_tiles = c.take<int32_t>(2 * 4);
    bw.s_tiles2 = c.take<int32_t>(2 * 4);
    bw.s_dgu = c.take<char>((size_t)s.T * 2 * s.F_shared * es);
    bw.s_h = c.take<char>((size_t)s.T * s.F_shared * es);
    bw.s_dX = c.take<char>((size_t)s.T * s.d * es);
  }
}

}  // namespace

thread_local moe::PhaseEvents moe::g_phase_events = {nullptr, 0};

extern "C" {

int moe_set_phase_events(void* const* events, int n_events) {
  if (n_events < 0 || (n_events > 0 && !events)) return MOE_ERR_INVALID_ARG;
  moe::g_phase_events = {n_events > 0 ? events : nullptr, n_events};
  return MOE_OK;
}

int moe_workspace_size(const moe_shape* shape, int op, size_t* bytes) {
  const int st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!bytes || op < MOE_OP_ROUTE || op > MOE_OP_BACKWARD_MXFP8) return MOE_ERR_INVALID_ARG;
  *bytes = ws_bytes_for(*shape, op);
  return MOE_OK;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null, misaligned or out-of-range argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid shape not supported by this build";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
    default: return "unknown moe_status";
  }
}

int moe_route_topk(const moe_shape* shape, const void* x, const void* w_router,
                   const float* router_bias, float* logits, const float* score_bias,
                   int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                   void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long long es = (long long)esize(s);
  const bool compute_logits = !(x == nullptr && w_router == nullptr);
  if (compute_logits) {
    if (!ok_buf(x, (long long)s.T * s.d * es) || !ok_buf(w_router, (long long)s.E * s.d * es))
      return MOE_ERR_INVALID_ARG;
    if (!ok_buf(router_bias, 0)) return MOE_ERR_INVALID_ARG;
  } else if (router_bias) {
    return MOE_ERR_INVALID_ARG;  // a bias only applies to computed logits
  }
  if (!ok_buf(logits, (long long)s.T * s.E * 4) || !ok_buf(topk_idx, (long long)s.T * s.k * 4) ||
      !ok_buf(topk_w, (long long)s.T * s.k * 4) || !ok_buf(score_bias, 0))
    return MOE_ERR_INVALID_ARG;
  // the partial sums are only needed (and the workspace only required)
  // when the logits are computed here
  if (compute_logits && (st = check_ws(s, MOE_OP_ROUTE, ws, ws_bytes)) != MOE_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (compute_logits) {
    if ((st = hip_status(moe::launch_router_logits(s, x, w_router, router_bias, logits,
                                                   static_cast<float*>(ws), hs))) != MOE_OK)
      return st;
  }
  return hip_status(moe::launch_topk(s, logits, score_bias, topk_idx, topk_w, hs));
}

// moe_permute's argument checks (the workspace aside).
static int check_permute_args(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                              const float* topk_w, int32_t* expert_offsets,
                              int32_t* row_token, int32_t* token_row, float* row_gate,
                              void* x_perm) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long long es = (long long)esize(s);
  const long long R = (long long)s.T * s.k;
  // x_perm NULL: only the maps (then x is not read and may be NULL too)
  const bool rows = x_perm != nullptr;
  if ((rows && !ok_buf(x, (long long)s.T * s.d * es)) || !ok_buf(topk_idx, R * 4) ||
      !ok_buf(topk_w, R * 4) || !ok_buf(expert_offsets, (long long)(s.E + 1) * 4) ||
      !ok_buf(row_token, R * 4) || !ok_buf(token_row, R * 4) || !ok_buf(row_gate, R * 4) ||
      (rows && !ok_buf(x_perm, R * s.d * es)))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int moe_permute_noalloc(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                        const float* topk_w, int32_t* expert_offsets, int32_t* row_token,
                        int32_t* token_row, float* row_gate, void* x_perm, void* stream) {
  int st = check_permute_args(shape, x, topk_idx, topk_w, expert_offsets, row_token,
                              token_row, row_gate, x_perm);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if ((long long)s.E * moe::permute_nblk(s) > moe::PERMUTE_NOALLOC_MAX_ENTRIES)
    return MOE_ERR_WORKSPACE;
  moe::PermuteWs pw;
  if ((st = hip_status(moe::permute_noalloc_ws(pw))) != MOE_OK) return st;
  return hip_status(moe::launch_permute(s, x, topk_idx, topk_w, expert_offsets, row_token,
                                        token_row, row_gate, x_perm, pw,
                                        static_cast<hipStream_t>(stream)));
}

int moe_permute(const moe_shape* shape, const void* x, const int32_t* topk_idx,
                const float* topk_w, int32_t* expert_offsets, int32_t* row_token,
                int32_t* token_row, float* row_gate, void* x_perm, void* ws, size_t ws_bytes,
                void* stream) {
  int st = check_permute_args(shape, x, topk_idx, topk_w, expert_offsets, row_token,
                              token_row, row_gate, x_perm);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if ((st = check_ws(s, MOE_OP_PERMUTE, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  const size_t n = (size_t)s.E * moe::permute_nblk(s);
  moe::PermuteWs pw;
  pw.blk_cnt = c.take<int32_t>(n * 4);
  pw.blk_base = c.take<int32_t>(n * 4);
  return hip_status(moe::launch_permute(s, x, topk_idx, topk_w, expert_offsets, row_token,
                                        token_row, row_gate, x_perm, pw,
                                        static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn(const moe_shape* shape, const void* x_perm, const int32_t* row_token,
                    const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                    const void* w_down, const void* x, const void* ws_gate, const void* ws_up,
                    const void* ws_down, void* y_perm, void* y_shared, void* gu_save, void* ws,
                    size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long long es = (long long)esize(s);
  const long long R = (long long)s.T * s.k;
  const long long wsz = (long long)s.E * s.F * s.d * es;
  const bool gather = x_perm == nullptr && R > 0;
  if (gather) {
    // rows come from x[row_token[r]]; byte offsets into x are 32-bit
    if (!ok_buf(x, (long long)s.T * s.d * es) || !ok_buf(row_token, R * 4))
      return MOE_ERR_INVALID_ARG;
    if ((long long)s.T * s.d * es >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  } else if (!ok_buf(x_perm, R * s.d * es)) {
    return MOE_ERR_INVALID_ARG;
  }
  if (!ok_buf(expert_offsets, (long long)(s.E + 1) * 4) ||
      !ok_buf(w_gate, wsz) || !ok_buf(w_up, wsz) || !ok_buf(w_down, wsz) ||
      !ok_buf(y_perm, R * s.d * es) || !ok_buf(gu_save, 0))
    return MOE_ERR_INVALID_ARG;
  if (s.F_shared > 0) {
    const long long sz = (long long)s.F_shared * s.d * es;
    if (!ok_buf(x, (long long)s.T * s.d * es) || !ok_buf(ws_gate, sz) || !ok_buf(ws_up, sz) ||
        !ok_buf(ws_down, sz) || !ok_buf(y_shared, (long long)s.T * s.d * es))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(s, MOE_OP_FFN, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  moe::FfnWs fw;
  fw.tiles1 = c.take<int32_t>((s.E + 1) * 4);
  fw.tiles2 = c.take<int32_t>((s.E + 1) * 4);
  fw.h = c.take<char>((size_t)R * s.F * es);
  fw.h_shared = c.take<char>((size_t)s.T * s.F_shared * es);
  const int ks = moe::ffn_fc2_ksplit(s);
  fw.part = ks > 1 ? c.take<float>((size_t)ks * R * s.d * 4) : nullptr;
  return hip_status(moe::launch_grouped_ffn(s, x_perm, gather ? row_token : nullptr,
                                            expert_offsets, w_gate, w_up, w_down, x,
                                            ws_gate, ws_up, ws_down, y_perm, y_shared, gu_save,
                                            fw, static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn_combine(const moe_shape* shape, const void* x_perm,
                            const int32_t* row_token, const float* row_gate,
                            const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                            const void* w_down, const void* x, const void* ws_gate,
                            const void* ws_up, const void* ws_down, float* y, void* ws,
                            size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long long es = (long long)esize(s);
  const long long R = (long long)s.T * s.k;
  const long long wsz = (long long)s.E * s.F * s.d * es;
  const bool gather = x_perm == nullptr && R > 0;
  if (gather) {
    if (!ok_buf(x, (long long)s.T * s.d * es)) return MOE_ERR_INVALID_ARG;
    if ((long long)s.T * s.d * es >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  } else if (!ok_buf(x_perm, R * s.d * es)) {
    return MOE_ERR_INVALID_ARG;
  }
  if (!ok_buf(row_token, R * 4) || !ok_buf(row_gate, R * 4) ||
      !ok_buf(expert_offsets, (long long)(s.E + 1) * 4) || !ok_buf(w_gate, wsz) ||
      !ok_buf(w_up, wsz) || !ok_buf(w_down, wsz) || !ok_buf(y, (long long)s.T * s.d * 4))
    return MOE_ERR_INVALID_ARG;
  if (s.F_shared > 0) {
    const long long sz = (long long)s.F_shared * s.d * es;
    if (!ok_buf(x, (long long)s.T * s.d * es) || !ok_buf(ws_gate, sz) || !ok_buf(ws_up, sz) ||
        !ok_buf(ws_down, sz))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(s, MOE_OP_FFN_COMBINE, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  moe::FfnWs fw;
  fw.tiles1 = c.take<int32_t>((s.E + 1) * 4);
  fw.tiles2 = c.take<int32_t>((s.E + 1) * 4);
  fw.h = c.take<char>((size_t)R * s.F * es);
  fw.h_shared = c.take<char>((size_t)s.T * s.F_shared * es);
  fw.part = nullptr;
  return hip_status(moe::launch_grouped_ffn_combine(s, x_perm, row_token, row_gate,
                                                    expert_offsets, w_gate, w_up, w_down, x,
                                                    ws_gate, ws_up, ws_down, y, fw,
                                                    static_cast<hipStream_t>(stream)));
}

int moe_unpermute_combine(const moe_shape* shape, const void* y_perm, const int32_t* token_row,
                          const float* topk_w, const void* y_shared, float* y, void* ws,
                          size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  const long long es = (long long)esize(s);
  const long long R = (long long)s.T * s.k;
  if (!ok_buf(y_perm, R * s.d * es) || !ok_buf(token_row, R * 4) || !ok_buf(topk_w, R * 4) ||
      !ok_buf(y, (long long)s.T * s.d * 4))
    return MOE_ERR_INVALID_ARG;
  if (s.F_shared > 0 && !ok_buf(y_shared, (long long)s.T * s.d * es)) return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_COMBINE, ws, ws_bytes)) != MOE_OK) return st;
  return hip_status(moe::launch_combine(s, y_perm, token_row, topk_w, y_shared, y,
                                        static_cast<hipStream_t>(stream)));
}

int moe_ffn_backward(const moe_shape* shape, const void* dy, const void* x_perm,
                     const void* gu_save, const void* y_perm, const int32_t* expert_offsets,
                     const int32_t* row_token, const int32_t* token_row,
                     const int32_t* topk_idx, const float* topk_w, const float* logits,
                     const void* w_gate, const void* w_up, const void* w_down, const void* x,
                     const void* ws_gate, const void* ws_up, const void* ws_down, float* dx,
                     void* dw_gate, void* dw_up, void* dw_down, void* dws_gate, void* dws_up,
                     void* dws_down, float* d_gate, float* d_logits, void* ws, size_t ws_bytes,
                     void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (!moe::backward_supported(s)) return MOE_ERR_UNSUPPORTED;
  const long long es = (long long)esize(s);
  const long long R = (long long)s.T * s.k;
  const long long wsz = (long long)s.E * s.F * s.d;
  const long long wes = s.wgrad_dtype == MOE_DTYPE_BF16 ? 2 : 4;   // weight-gradient bytes
  const long long gu_elems = R * 2 * s.F + (long long)s.T * 2 * s.F_shared;
  if (s.F_shared > 0) {
    const long long sz = (long long)s.F_shared * s.d;
    if (!ok_buf(x, (long long)s.T * s.d * es) || !ok_buf(ws_gate, sz * es) ||
        !ok_buf(ws_up, sz * es) || !ok_buf(ws_down, sz * es) || !ok_buf(dws_gate, sz * wes) ||
        !ok_buf(dws_up, sz * wes) || !ok_buf(dws_down, sz * wes))
      return MOE_ERR_INVALID_ARG;
  }
  // gu_save NULL: g | u are recomputed by FC1 into the workspace
  const bool recompute = gu_save == nullptr;
  const int op = recompute ? MOE_OP_BACKWARD_RECOMPUTE : MOE_OP_BACKWARD;
  if (!ok_buf(dy, (long long)s.T * s.d * es) || !ok_buf(x_perm, R * s.d * es) ||
      (!recompute && !ok_buf(gu_save, gu_elems * es)) || !ok_buf(y_perm, R * s.d * es) ||
      !ok_buf(expert_offsets, (long long)(s.E + 1) * 4) || !ok_buf(row_token, R * 4) ||
      !ok_buf(token_row, R * 4) || !ok_buf(topk_idx, R * 4) || !ok_buf(topk_w, R * 4) ||
      !ok_buf(logits, (long long)s.T * s.E * 4) || !ok_buf(w_gate, wsz * es) ||
      !ok_buf(w_up, wsz * es) || !ok_buf(w_down, wsz * es) ||
      !ok_buf(dx, (long long)s.T * s.d * 4) || !ok_buf(dw_gate, wsz * wes) ||
      !ok_buf(dw_up, wsz * wes) || !ok_buf(dw_down, wsz * wes) || !ok_buf(d_gate, R * 4) ||
      !ok_buf(d_logits, (long long)s.T * s.E * 4))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, op, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  moe::BwdWs bw;
  carve_backward(s, c, bw);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (recompute) {
    void* gu = c.take<char>((size_t)gu_elems * es);
    if ((st = hip_status(moe::launch_fc1_recompute(s, x_perm, expert_offsets, w_gate, w_up, x,
                                                   ws_gate, ws_up, gu, bw.h, bw.s_h, bw.tiles,
                                                   hs))) != MOE_OK)
      return st;
    gu_save = gu;
  }
  return hip_status(moe::launch_backward(s, dy, x_perm, gu_save, y_perm, expert_offsets,
                                         row_token, token_row, topk_idx, topk_w, logits,
                                         w_gate, w_up, w_down, x, ws_gate, ws_up, ws_down, dx,
                                         dw_gate, dw_up, dw_down, dws_gate, dws_up, dws_down,
                                         d_gate, d_logits, bw, hs));
}

int moe_mx_quantize(const void* src, int64_t rows, int32_t cols, uint8_t* q, uint8_t* scales,
                    void* stream) {
  if (rows < 0 || cols < 32 || cols % 32 != 0) return MOE_ERR_INVALID_ARG;
  if ((long long)rows * cols >= (1LL << 40)) return MOE_ERR_INVALID_ARG;
  const long long n = (long long)rows * cols;
  if (!ok_buf(src, n * 2) || !ok_buf(q, n) || !ok_buf(scales, n / 32)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_mx_quantize(src, rows, cols, q, scales,
                                            static_cast<hipStream_t>(stream)));
}

int moe_mx_quantize_t(const void* src, int64_t batches, int32_t rows, int32_t cols, int32_t ldq,
                      uint8_t* q, uint8_t* scales, void* stream) {
  if (batches < 0 || batches > 65535 || rows < 0 || rows % 32 != 0 || cols < 0 ||
      ldq < rows || ldq % 32 != 0)
    return MOE_ERR_INVALID_ARG;
  const long long n = batches * (long long)rows * cols;
  const long long nq = batches * (long long)cols * ldq;
  if (n >= (1LL << 40) || nq >= (1LL << 40)) return MOE_ERR_INVALID_ARG;
  if (n == 0) return MOE_OK;
  // codes are written 8 bytes at a time; scale bytes one at a time
  if (!ok_buf(src, n * 2) || !q || (reinterpret_cast<uintptr_t>(q) & 7) != 0 || !scales)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_mx_quantize_t(src, batches, rows, cols, ldq, q, scales,
                                              static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn_mxfp8(const moe_shape* shape, const uint8_t* xq, const uint8_t* xs,
                          const int32_t* row_token, const int32_t* expert_offsets,
                          const uint8_t* w_gate_q, const uint8_t* w_gate_s,
                          const uint8_t* w_up_q, const uint8_t* w_up_s,
                          const uint8_t* w_down_q, const uint8_t* w_down_s,
                          const uint8_t* ws_gate_q, const uint8_t* ws_gate_s,
                          const uint8_t* ws_up_q, const uint8_t* ws_up_s,
                          const uint8_t* ws_down_q, const uint8_t* ws_down_s, void* y_perm,
                          void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;   // y is bf16
  if (s.d % 128 != 0 || s.F % 128 != 0 || s.F_shared % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)s.T * s.k;
  const long long xn = (long long)s.T * s.d;
  const long long wn = (long long)s.E * s.F * s.d;
  if (!ok_buf(xq, xn) || !ok_buf(xs, xn / 32) || !ok_buf(row_token, R * 4) ||
      !ok_buf(expert_offsets, (long long)(s.E + 1) * 4) || !ok_buf(w_gate_q, wn) ||
      !ok_buf(w_gate_s, wn / 32) || !ok_buf(w_up_q, wn) || !ok_buf(w_up_s, wn / 32) ||
      !ok_buf(w_down_q, wn) || !ok_buf(w_down_s, wn / 32) || !ok_buf(y_perm, R * s.d * 2))
    return MOE_ERR_INVALID_ARG;
  if (s.F_shared > 0) {
    const long long sn = (long long)s.F_shared * s.d;
    if (!ok_buf(ws_gate_q, sn) || !ok_buf(ws_gate_s, sn / 32) || !ok_buf(ws_up_q, sn) ||
        !ok_buf(ws_up_s, sn / 32) || !ok_buf(ws_down_q, sn) || !ok_buf(ws_down_s, sn / 32) ||
        !ok_buf(y_shared, xn * 2))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(s, MOE_OP_FFN_MXFP8, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  moe::MxFfnWs fw;
  fw.tiles1 = c.take<int32_t>((s.E + 1) * 4);
  fw.tiles2 = c.take<int32_t>((s.E + 1) * 4);
  fw.hq = c.take<uint8_t>((size_t)R * s.F);
  fw.hs = c.take<uint8_t>((size_t)R * s.F / 32);
  fw.shq = c.take<uint8_t>((size_t)s.T * s.F_shared);
  fw.shs = c.take<uint8_t>((size_t)s.T * s.F_shared / 32);
  const moe::MxWeights w = {w_gate_q, w_gate_s, w_up_q, w_up_s, w_down_q, w_down_s,
                            ws_gate_q, ws_gate_s, ws_up_q, ws_up_s, ws_down_q, ws_down_s};
  return hip_status(moe::launch_grouped_ffn_mxfp8(s, xq, xs, row_token, expert_offsets, w,
                                                  y_perm, y_shared, fw,
                                                  static_cast<hipStream_t>(stream)));
}

int moe_grouped_ffn_mxfp8_combine(const moe_shape* shape, const uint8_t* xq, const uint8_t* xs,
                                  const int32_t* row_token, const float* row_gate,
                                  const int32_t* expert_offsets,
                                  const uint8_t* w_gate_q, const uint8_t* w_gate_s,
                                  const uint8_t* w_up_q, const uint8_t* w_up_s,
                                  const uint8_t* w_down_q, const uint8_t* w_down_s,
                                  const uint8_t* ws_gate_q, const uint8_t* ws_gate_s,
                                  const uint8_t* ws_up_q, const uint8_t* ws_up_s,
                                  const uint8_t* ws_down_q, const uint8_t* ws_down_s, float* y,
                                  void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.d % 128 != 0 || s.F % 128 != 0 || s.F_shared % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)s.T * s.k;
  const long long xn = (long long)s.T * s.d;
  const long long wn = (long long)s.E * s.F * s.d;
  if (!ok_buf(xq, xn) || !ok_buf(xs, xn / 32) || !ok_buf(row_token, R * 4) ||
      !ok_buf(row_gate, R * 4) || !ok_buf(expert_offsets, (long long)(s.E + 1) * 4) ||
      !ok_buf(w_gate_q, wn) || !ok_buf(w_gate_s, wn / 32) || !ok_buf(w_up_q, wn) ||
      !ok_buf(w_up_s, wn / 32) || !ok_buf(w_down_q, wn) || !ok_buf(w_down_s, wn / 32) ||
      !ok_buf(y, xn * 4))
    return MOE_ERR_INVALID_ARG;
  if (s.F_shared > 0) {
    const long long sn = (long long)s.F_shared * s.d;
    if (!ok_buf(ws_gate_q, sn) || !ok_buf(ws_gate_s, sn / 32) || !ok_buf(ws_up_q, sn) ||
        !ok_buf(ws_up_s, sn / 32) || !ok_buf(ws_down_q, sn) || !ok_buf(ws_down_s, sn / 32))
      return MOE_ERR_INVALID_ARG;
  }
  if ((st = check_ws(s, MOE_OP_FFN_MXFP8, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  moe::MxFfnWs fw;
  fw.tiles1 = c.take<int32_t>((s.E + 1) * 4);
  fw.tiles2 = c.take<int32_t>((s.E + 1) * 4);
  fw.hq = c.take<uint8_t>((size_t)R * s.F);
  fw.hs = c.take<uint8_t>((size_t)R * s.F / 32);
  fw.shq = c.take<uint8_t>((size_t)s.T * s.F_shared);
  fw.shs = c.take<uint8_t>((size_t)s.T * s.F_shared / 32);
  const moe::MxWeights w = {w_gate_q, w_gate_s, w_up_q, w_up_s, w_down_q, w_down_s,
                            ws_gate_q, ws_gate_s, ws_up_q, ws_up_s, ws_down_q, ws_down_s};
  return hip_status(moe::launch_grouped_ffn_mxfp8(s, xq, xs, row_token, expert_offsets, w,
                                                  nullptr, nullptr, fw,
                                                  static_cast<hipStream_t>(stream), row_gate, y));
}

int moe_ffn_backward_mxfp8(const moe_shape* shape, const void* dy, const void* x_perm,
                           const void* gu_save, const void* y_perm,
                           const int32_t* expert_offsets, const int32_t* row_token,
                           const int32_t* token_row, const int32_t* topk_idx,
                           const float* topk_w, const float* logits,
                           const uint8_t* w_down_tq, const uint8_t* w_down_ts,
                           const uint8_t* w_gu_tq, const uint8_t* w_gu_ts, const void* x,
                           const uint8_t* ws_down_tq, const uint8_t* ws_down_ts,
                           const uint8_t* ws_gu_tq, const uint8_t* ws_gu_ts, float* dx,
                           void* dw_gate, void* dw_up, void* dw_down, void* dws_gate,
                           void* dws_up, void* dws_down, float* d_gate, float* d_logits,
                           void* ws, size_t ws_bytes, void* stream) {
  int st = check_shape(shape);
  if (st != MOE_OK) return st;
  const moe_shape& s = *shape;
  if (s.dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID_ARG;
  if (s.d % 128 != 0 || s.F % 128 != 0 || s.F_shared % 128 != 0) return MOE_ERR_UNSUPPORTED;
  // the MXFP8 weight gradients' padded row count is an int32
  if (s.wgrad_mx && (long long)mx_wgrad_rows(s) >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)s.T * s.k;
  const long long wsz = (long long)s.E * s.F * s.d;
  const long long wes = s.wgrad_dtype == MOE_DTYPE_BF16 ? 2 : 4;
  const long long gu_elems = R * 2 * s.F + (long long)s.T * 2 * s.F_shared;
  // every quantised weight: codes one byte per value, scales one per 32
  auto ok_q = [](const uint8_t* q, const uint8_t* sc, long long n) {
    return ok_buf(q, n) && ok_buf(sc, n / 32);
  };
  if (s.F_shared > 0) {
    const long long sz = (long long)s.F_shared * s.d;
    if (!ok_buf(x, (long long)s.T * s.d * 2) || !ok_q(ws_down_tq, ws_down_ts, sz) ||
        !ok_q(ws_gu_tq, ws_gu_ts, 2 * sz) || !ok_buf(dws_gate, sz * wes) ||
        !ok_buf(dws_up, sz * wes) || !ok_buf(dws_down, sz * wes))
      return MOE_ERR_INVALID_ARG;
  }
  if (!ok_buf(dy, (long long)s.T * s.d * 2) || !ok_buf(x_perm, R * s.d * 2) ||
      (gu_elems > 0 && gu_save == nullptr) || !ok_buf(gu_save, gu_elems * 2) ||
      !ok_buf(y_perm, R * s.d * 2) ||
      !ok_buf(expert_offsets, (long long)(s.E + 1) * 4) || !ok_buf(row_token, R * 4) ||
      !ok_buf(token_row, R * 4) || !ok_buf(topk_idx, R * 4) || !ok_buf(topk_w, R * 4) ||
      !ok_buf(logits, (long long)s.T * s.E * 4) || !ok_q(w_down_tq, w_down_ts, wsz) ||
      !ok_q(w_gu_tq, w_gu_ts, 2 * wsz) || !ok_buf(dx, (long long)s.T * s.d * 4) ||
      !ok_buf(dw_gate, wsz * wes) || !ok_buf(dw_up, wsz * wes) ||
      !ok_buf(dw_down, wsz * wes) || !ok_buf(d_gate, R * 4) ||
      !ok_buf(d_logits, (long long)s.T * s.E * 4))
    return MOE_ERR_INVALID_ARG;
  if ((st = check_ws(s, MOE_OP_BACKWARD_MXFP8, ws, ws_bytes)) != MOE_OK) return st;
  Carver c{static_cast<char*>(ws)};
  moe::BwdWs bw;
  carve_backward(s, c, bw);
  bw.dyq = c.take<uint8_t>((size_t)R * s.d);
  bw.dys = c.take<uint8_t>((size_t)R * s.d / 32);
  bw.dguq = c.take<uint8_t>((size_t)R * 2 * s.F);
  bw.dgus = c.take<uint8_t>((size_t)R * 2 * s.F / 32);
  bw.s_dyq = bw.s_dys = bw.s_dguq = bw.s_dgus = nullptr;
  if (s.F_shared > 0) {
    const size_t T = (size_t)s.T, Fs = (size_t)s.F_shared;
    bw.s_dyq = c.take<uint8_t>(T * s.d);
    bw.s_dys = c.take<uint8_t>(T * s.d / 32);
    bw.s_dguq = c.take<uint8_t>(T * 2 * Fs);
    bw.s_dgus = c.take<uint8_t>(T * 2 * Fs / 32);
  }
  bw.poffs = bw.s_poffs = nullptr;
  bw.wqa = bw.wsa = bw.wqb = bw.wsb = nullptr;
  bw.wrows = 0;
  if (s.wgrad_mx) {
    const size_t rp = mx_wgrad_rows(s);
    const size_t ma = std::max<size_t>({(size_t)s.d, 2 * (size_t)s.F, 2 * (size_t)s.F_shared});
    const size_t mb = std::max<size_t>({(size_t)s.d, (size_t)s.F, (size_t)s.F_shared});
    bw.poffs = c.take<int32_t>((s.E + 1) * 4);
    bw.s_poffs = c.take<int32_t>((s.E + 1) * 4);
    bw.wqa = c.take<uint8_t>(ma * rp);
    bw.wsa = c.take<uint8_t>(ma * rp / 32);
    bw.wqb = c.take<uint8_t>(mb * rp);
    bw.wsb = c.take<uint8_t>(mb * rp / 32);
    bw.wrows = (long long)rp;
  }
  moe::MxBwdWeights mw = {w_down_tq, w_down_ts, w_gu_tq, w_gu_ts,
                          ws_down_tq, ws_down_ts, ws_gu_tq, ws_gu_ts};
  return hip_status(moe::launch_backward(s, dy, x_perm, gu_save, y_perm, expert_offsets,
                                         row_token, token_row, topk_idx, topk_w, logits,
                                         nullptr, nullptr, nullptr, x, nullptr, nullptr,
                                         nullptr, dx, dw_gate, dw_up, dw_down, dws_gate,
                                         dws_up, dws_down, d_gate, d_logits, bw,
                                         static_cast<hipStream_t>(stream), &mw));
}

}  // extern "C"
