"""The layer at a size the routed rows take past 2^31 elements.

A DeepSeek-V3-width step of 40000 tokens at k = 8 over 32 experts has
R d = 320000 x 7168 = 2.29e9 elements in x_perm, y_perm, dY_perm and
dX_perm (4.6 GB each in bf16).  The tile kernels address routed rows with
64-bit bases, so only token-indexed arrays (T d) and one expert's weights
(F d) are bounded by 2^31.  Forward and backward run in full on the GPU;
the oracle routes from its own scores, and y, dx, d_gate and d_logits are
compared on sampled tokens, the weight gradients on whole experts, each
expert evaluated by the oracle on just the rows needed.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import MoEConfig, make_inputs
from parity_util import (assert_close, assert_equal_int, check_maps_valid,
                         oracle_sampled_backward, oracle_sampled_forward, prec_of,
                         route_and_check, sample_tokens)

pytestmark = pytest.mark.gpu


def test_training_step_with_routed_rows_beyond_2_31_elements():
    from mixture_experts_layer_logits_amd import MoELayer
    cfg = MoEConfig("large_t40000_d7168", T=40000, d=7168, E=32, k=8, F=256, backward=True)
    R = cfg.T * cfg.k
    assert R * cfg.d >= 1 << 31 and cfg.T * cfg.d < 1 << 31
    print(f"[large] {cfg.name}: R d = {R * cfg.d:.3e}", flush=True)
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    out = layer.forward(inp)
    g = layer.backward(inp, inp["dy"])
    torch.cuda.synchronize()
    prec = prec_of(cfg)
    idx, w, amb, same = route_and_check(cfg, inp, out, max_ambiguous_frac=0.01)
    check_maps_valid(out, out["topk_idx"].cpu().numpy(), out["topk_w"].cpu().numpy(), cfg.E)
    p = O.permute(None, idx, w, cfg.E)
    if same:
        for key in ("expert_offsets", "row_token", "token_row"):
            assert_equal_int(key, out[key], p["offsets" if key == "expert_offsets" else key])
    # sampled tokens, including the last ones (whose rows sit past 2^31
    # elements in the routed buffers of the last experts)
    toks = np.array([t for t in sample_tokens(cfg.T, 24) if not amb[t]] + [cfg.T - 1])
    toks = np.unique(toks[~amb[toks]])
    tt = torch.as_tensor(toks, device="cuda")
    ref = oracle_sampled_forward(cfg, inp, toks, idx, w)
    assert_close("y[sample]", out["y"][tt], ref["y"], prec)
    if same:
        rows = out["token_row"][tt].reshape(-1).long()
        assert_close("y_perm[sample]", out["y_perm"][rows], ref["y_rows"].reshape(-1, cfg.d), prec)
        # whole experts: the first, and the last, whose rows all lie past
        # element 2^31 of the routed buffers
        experts = [0, cfg.E - 1]
        assert int(p["offsets"][cfg.E - 1]) * cfg.d >= 1 << 31
        logits = O.router_logits(inp["x"], inp["w_router"], inp.get("router_bias"), "f32")
        rb = oracle_sampled_backward(cfg, inp, p, idx, w, logits, toks, experts)
        assert_close("dx[sample]", g["dx"][tt], rb["dx"], prec)
        assert_close("d_gate[sample]", g["d_gate"][tt], rb["d_gate"], prec)
        assert_close("d_logits[sample]", g["d_logits"][tt], rb["d_logits"], prec)
        for e in experts:
            for key in ("dw_gate", "dw_up", "dw_down"):
                assert_close(f"{key}[{e}]", g[key][e], rb["dw"][e][key], prec)
    del layer, out, g, inp
    torch.cuda.empty_cache()
