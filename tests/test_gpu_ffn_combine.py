"""GPU parity of the FFN with the combine folded into FC2's epilogue
(moe_grouped_ffn_combine: y straight from the expert GEMMs, no y_perm)
against the oracle's grouped_ffn_combine, in which the expert outputs are
never rounded.

Routing comes from the GPU's own route and maps-only permute and is checked
against the oracle's as in the layer tests; y is compared on every token
whose routing is unambiguous.  The additions into y are fp32 atomics whose
order varies, so two runs are compared within fp32 rounding, not bitwise.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import CONFIGS, MoEConfig, SCORE_SIGMOID, make_inputs
from parity_util import (assert_close, np64, oracle_sampled_forward, prec_of,
                         route_and_check, sample_tokens)

pytestmark = pytest.mark.gpu

CASES = {
    # MFMA path, FC2 with its contraction split (slices add into y)
    "bf16_softmax_t300": MoEConfig("bf16_softmax_t300", T=300, d=256, E=8, k=2, F=384),
    # MFMA path with the shared expert in the same launches, k = 8
    "bf16_sigmoid_groups_shared_t200": MoEConfig(
        "bf16_sigmoid_groups_shared_t200", T=200, d=128, E=64, k=8, F=128,
        F_shared=192, n_groups=8, topk_groups=4, score=SCORE_SIGMOID, score_bias_std=0.1),
    # several row tiles per expert, ragged tails, d not a multiple of 256
    "bf16_t1500_d320": MoEConfig("bf16_t1500_d320", T=1500, d=320, E=6, k=2, F=256),
    # skewed loads with empty experts
    "bf16_skewed_t520": MoEConfig("bf16_skewed_t520", T=520, d=192, E=32, k=4, F=256,
                                  zipf_s=1.2),
    # generic tile kernel (odd widths) with a shared expert, and the fp32 layer
    "bf16_generic_shapes_t77": MoEConfig("bf16_generic_shapes_t77", T=77, d=200, E=6, k=2,
                                         F=96, F_shared=40),
    "f32_odd_t37": MoEConfig("f32_odd_t37", T=37, d=20, E=5, k=3, F=12, dtype=0),
    "bf16_one_token": MoEConfig("bf16_one_token", T=1, d=128, E=16, k=4, F=128),
    "bf16_single_expert_t65": MoEConfig("bf16_single_expert_t65", T=65, d=64, E=1, k=1, F=64),
}


def _combined(cfg, inp):
    from mixture_experts_layer_logits_amd import MoELayer
    layer = MoELayer(cfg)
    out = layer.forward_combined(inp)
    torch.cuda.synchronize()
    return layer, out


@pytest.mark.parametrize("name", list(CASES))
def test_ffn_combine_small(name):
    cfg = CASES[name]
    print(f"[ffn combine] {name}", flush=True)
    inp = make_inputs(cfg, device="cuda")
    layer, out = _combined(cfg, inp)
    prec = prec_of(cfg)
    idx, w, amb, same = route_and_check(cfg, inp, out)
    p = O.permute(np64(inp["x"]), idx, w, cfg.E)
    sh = None
    if cfg.F_shared > 0:
        sh = (np64(inp["x"]), np64(inp["ws_gate"]), np64(inp["ws_up"]), np64(inp["ws_down"]))
    ref = O.grouped_ffn_combine(p["x_perm"], p["offsets"], p["token_row"], w,
                                np64(inp["w_gate"]), np64(inp["w_up"]), np64(inp["w_down"]),
                                sh, prec)
    ok = ~amb
    assert_close("y", out["y"][torch.as_tensor(ok).cuda()], ref[ok], prec)
    # two runs agree to fp32 rounding of the few additions per element
    y1 = out["y"].clone()
    layer.ffn_combine(inp)
    torch.cuda.synchronize()
    assert_close("y (second run)", out["y"], y1, "f32")


def test_ffn_combine_matches_unfused_forward():
    """Against the layer's unfused forward (y_perm rounded to bf16, then the
    per-token combine): equal up to that rounding."""
    cfg = CASES["bf16_sigmoid_groups_shared_t200"]
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    y_unfused = layer.forward(inp)["y"].clone()
    y = layer.forward_combined(inp)["y"]
    torch.cuda.synchronize()
    assert_close("y vs unfused", y, y_unfused, "bf16")
    assert not torch.equal(y, y_unfused)


def test_ffn_combine_with_x_perm_matches_gather():
    """With x_perm given (rows not gathered) the result is the same up to
    the order of the atomic additions."""
    cfg = CASES["bf16_t1500_d320"]
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    layer.forward(inp)
    layer.ffn_combine(inp, gather=False)
    torch.cuda.synchronize()
    y = layer.buf["y"].clone()
    layer.ffn_combine(inp, gather=True)
    torch.cuda.synchronize()
    assert_close("y gather vs x_perm", layer.buf["y"], y, "f32")


def test_ffn_combine_overwrites_y():
    """y is overwritten, not accumulated into: garbage beforehand changes
    nothing."""
    cfg = CASES["bf16_skewed_t520"]
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    layer.forward_combined(inp)
    torch.cuda.synchronize()
    y = layer.buf["y"].clone()
    layer.buf["y"].fill_(float("nan"))
    layer.ffn_combine(inp)
    torch.cuda.synchronize()
    assert torch.isfinite(layer.buf["y"]).all()
    assert_close("y after nan fill", layer.buf["y"], y, "f32")


@pytest.mark.parametrize("name", ["mixtral_t4096", "deepseek_v3_t8192",
                                  "qwen3_30b_skewed_t16384"])
def test_ffn_combine_full_size_sampled(name):
    cfg = CONFIGS[name]
    print(f"[ffn combine full] {name}", flush=True)
    inp = make_inputs(cfg, device="cuda")
    layer, out = _combined(cfg, inp)
    prec = prec_of(cfg)
    idx, w, amb, same = route_and_check(cfg, inp, out)
    n = 16 if cfg.E >= 256 else 48
    toks = np.array([t for t in sample_tokens(cfg.T, n) if not amb[t]])
    ref = oracle_sampled_forward(cfg, inp, toks, idx, w, combined=True)
    assert_close("y[sample]", out["y"][torch.as_tensor(toks, device="cuda")], ref["y"], prec)
    del layer, out, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("k", [1, 2])
def test_ffn_combine_two_addends_is_bitwise_reproducible(k):
    """With at most two additions into each y element the result does not
    depend on their order (0 + a + b = 0 + b + a exactly).  T = 8192, d =
    4096, E = 8, F = 512 and no shared expert: at k = 2, FC2 has
    (64 + 8) x 16 = 1152 tiles, enough to run unsplit; at k = 1 it has
    (32 + 8) x 16 = 640 and runs in two slices.  Either way each element
    gets two addends, and three runs agree bit for bit."""
    cfg = MoEConfig(f"bf16_k{k}_t8192", T=8192, d=4096, E=8, k=k, F=512)
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    layer.forward_combined(inp)
    torch.cuda.synchronize()
    y0 = layer.buf["y"].clone()
    for _ in range(2):
        layer.ffn_combine(inp)
        torch.cuda.synchronize()
        assert torch.equal(layer.buf["y"], y0)
    del layer, inp
    torch.cuda.empty_cache()
