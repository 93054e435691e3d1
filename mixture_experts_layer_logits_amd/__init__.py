"""One GPU's Mixture-of-Experts layer on AMD Instinct MI355X (gfx950).

Route (router GEMM + top-k) -> padding-free permutation -> grouped SwiGLU
expert FFN (+ shared expert) -> unpermute-and-scale combine, and the backward
pass, all in hand-written HIP kernels behind the C ABI of include/moe.h.
"""
from ._lib import (MoeError, MoeShape, load, make_shape, moe_ffn_backward,  # noqa: F401
                   moe_grouped_ffn, moe_grouped_ffn_combine, moe_grouped_ffn_mxfp8,
                   moe_grouped_ffn_mxfp8_combine,
                   moe_ffn_backward_mxfp8, moe_mx_quantize, moe_mx_quantize_t,
                   moe_permute, moe_permute_noalloc, moe_route_topk, moe_set_phase_events,
                   moe_unpermute_combine,
                   moe_workspace_size, status_string)
from .layer import MoELayer  # noqa: F401
