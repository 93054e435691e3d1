"""End-to-end GPU parity of the layer (route -> permute -> grouped FFN ->
combine) against the oracle run entirely on its own inputs.

The oracle computes its own router scores in fp64 and routes from them.
Routing must match bit for bit on every token whose selection is
unambiguous at fp32 resolution (decided by the oracle: see
parity_util.ambiguous_tokens); where the oracle finds a near-tie, any
selection valid within that bound is accepted.  When routing matches
everywhere (the expected case), every map is compared bit for bit.
Full-size workloads compare sampled token rows computed one expert at a
time.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import CONFIGS, MoEConfig, SCORE_SIGMOID, child_seed, make_inputs, normal
from parity_util import (assert_close, assert_equal_int, check_maps_valid, np64,
                         oracle_sampled_forward, prec_of, route_and_check, sample_tokens)

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_fp32": CONFIGS["tiny_fp32"],
    "bf16_softmax_t300": MoEConfig("bf16_softmax_t300", T=300, d=256, E=8, k=2, F=384),
    "bf16_sigmoid_groups_shared_t200": MoEConfig(
        "bf16_sigmoid_groups_shared_t200", T=200, d=128, E=64, k=8, F=128,
        F_shared=192, n_groups=8, topk_groups=4, score=SCORE_SIGMOID, score_bias_std=0.1),
    "bf16_skewed_t520": MoEConfig("bf16_skewed_t520", T=520, d=192, E=32, k=4, F=256,
                                  zipf_s=1.2),
    "bf16_generic_shapes_t77": MoEConfig("bf16_generic_shapes_t77", T=77, d=200, E=6, k=2,
                                         F=96, F_shared=40),
    "f32_odd_t37": MoEConfig("f32_odd_t37", T=37, d=20, E=5, k=3, F=12, dtype=0),
    "bf16_single_expert_t65": MoEConfig("bf16_single_expert_t65", T=65, d=64, E=1, k=1, F=64),
    "bf16_one_token": MoEConfig("bf16_one_token", T=1, d=128, E=16, k=4, F=128),
    "bf16_full_probs_t129": MoEConfig("bf16_full_probs_t129", T=129, d=128, E=12, k=3,
                                      F=192, renorm=0),
}


def _run(cfg, inp=None):
    from mixture_experts_layer_logits_amd import MoELayer
    if inp is None:
        inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    out = layer.forward(inp)
    torch.cuda.synchronize()
    return inp, layer, out


_route_and_check = route_and_check


def _maps(out, inp, cfg):
    """Validity of the GPU's maps for the GPU's own routing (always)."""
    check_maps_valid(out, out["topk_idx"].cpu().numpy(), out["topk_w"].cpu().numpy(), cfg.E,
                     x=inp["x"])


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    cfg = SMALL[name]
    print(f"[layer] {name}", flush=True)
    inp, layer, out = _run(cfg)
    prec = prec_of(cfg)
    idx, w, amb, same = _route_and_check(cfg, inp, out)
    _maps(out, inp, cfg)
    ref = O.forward(inp, cfg, prec=prec)
    if same:
        assert_equal_int("expert_offsets", out["expert_offsets"], ref["offsets"])
        assert_equal_int("row_token", out["row_token"], ref["row_token"])
        assert_equal_int("token_row", out["token_row"], ref["token_row"])
        rt = torch.as_tensor(ref["row_token"], device="cuda").long()
        assert torch.equal(out["x_perm"], inp["x"][rt])
        assert_close("y_perm", out["y_perm"], ref["y_perm"], prec)
    if cfg.F_shared > 0:
        assert_close("y_shared", out["y_shared"], ref["y_shared"], prec)
    ok = torch.as_tensor(~amb | same)
    assert_close("y", out["y"][ok.cuda()], ref["y"][ok.numpy()], prec)


@pytest.mark.parametrize("name", ["bf16_sigmoid_groups_shared_t200", "bf16_skewed_t520",
                                  "f32_odd_t37"])
def test_layer_fused_forward_matches_unfused(name):
    """The fused forward (maps-only permute, FC1 gathering rows from x) gives
    bitwise the same y_perm and y as the path through x_perm."""
    cfg = SMALL[name]
    print(f"[layer fused] {name}", flush=True)
    inp, layer, out = _run(cfg)
    y_perm, y = out["y_perm"].clone(), out["y"].clone()
    layer.forward(inp, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(out["y_perm"], y_perm)
    assert torch.equal(out["y"], y)


def test_layer_is_bitwise_deterministic():
    cfg = SMALL["bf16_sigmoid_groups_shared_t200"].replace(T=1000)
    inp, layer, out = _run(cfg)
    first = {k: v.clone() for k, v in out.items() if v is not None}
    layer.forward(inp)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(v, out[k]), k


@pytest.mark.parametrize("wgrad", [0, 1], ids=["wgrad_fp32", "wgrad_bf16"])
def test_layer_no_tokens(wgrad):
    """T = 0 through every call of the layer (forward through x_perm, fused,
    with the combine in FC2, and the bf16 and MXFP8 backward).  Nothing of
    size T exists; the weight gradients, sums over no tokens, are exactly
    zero for the routed and the shared experts alike."""
    from mixture_experts_layer_logits_amd import MoELayer
    cfg = MoEConfig(f"no_tokens_wgrad{wgrad}", T=0, d=256, E=16, k=4, F=256,
                    F_shared=256, n_groups=4, topk_groups=2, score=SCORE_SIGMOID,
                    backward=True, wgrad_dtype=wgrad)
    print(f"[layer no tokens] {cfg.name}", flush=True)
    inp = make_inputs(cfg, device="cuda")
    infer = MoELayer(cfg.replace(backward=False))
    keys = ("dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up", "dws_down")
    for run in ("forward", "fused", "combined"):
        if run == "forward":
            out = infer.forward(inp)
        elif run == "fused":
            out = infer.forward(inp, fused=True)
        else:
            out = infer.forward_combined(inp)
        torch.cuda.synchronize()
        assert out["y"].shape == (0, cfg.d)
        assert out["expert_offsets"].cpu().tolist() == [0] * (cfg.E + 1)
    layer = MoELayer(cfg)
    layer.forward(inp)
    layer.quantize_weights_t(inp)
    for bwd in (layer.backward, layer.backward_mxfp8):
        if layer.grad is None:
            layer._alloc_grad()
        for key in keys:
            layer.grad[key].fill_(float("nan"))
        g = bwd(inp, inp["dy"])
        torch.cuda.synchronize()
        for key in keys:
            assert torch.all(g[key] == 0), (bwd.__name__, key)
        assert g["dx"].shape == (0, cfg.d) and g["d_logits"].shape == (0, cfg.E)


def test_layer_training_with_shared_expert():
    """Forward (saving g|u of routed and shared rows) then backward of a layer
    with sigmoid group-limited routing and a shared expert, against the
    oracle's own forward and backward.  The shared expert's gradients do not
    depend on the routing; dx[t] depends only on token t's own routing and
    is compared where that is unambiguous; the routed weight gradients sum
    over all tokens of an expert and are compared when the routing matches
    the oracle's everywhere."""
    cfg = SMALL["bf16_sigmoid_groups_shared_t200"].replace(backward=True)
    print(f"[layer train] {cfg.name}", flush=True)
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    out = layer.forward(inp)
    g = layer.backward(inp, inp["dy"])
    torch.cuda.synchronize()
    prec = prec_of(cfg)
    idx, w, amb, same = _route_and_check(cfg, inp, out)
    ref = O.forward(inp, cfg, prec=prec, save_gu=True)
    gu_r, gu_s = layer.gu_views()
    assert_close("gu_shared", gu_s, ref["gu_shared"], prec)
    host = lambda t: np64(t)
    bw = O.ffn_backward(host(inp["dy"]), ref["x_perm"], ref["gu_save"], ref["y_perm"],
                        ref["offsets"], ref["token_row"], ref["topk_idx"], ref["topk_w"],
                        ref["route_logits"], host(inp["w_gate"]), host(inp["w_up"]),
                        host(inp["w_down"]), cfg.score, cfg.renorm, prec,
                        shared=dict(x=host(inp["x"]), gu=ref["gu_shared"],
                                    ws_gate=host(inp["ws_gate"]), ws_up=host(inp["ws_up"]),
                                    ws_down=host(inp["ws_down"])))
    for key in ("dws_gate", "dws_up", "dws_down"):
        assert_close(key, g[key], bw[key], prec)
    ok = torch.as_tensor(~amb)
    assert_close("dx[unambiguous]", g["dx"][ok.cuda()], bw["dx"][ok.numpy()], prec)
    if same:
        for key in ("dw_gate", "dw_up", "dw_down", "d_gate"):
            assert_close(key, g[key], bw[key], prec)


FULL = ["mixtral_t4096", "deepseek_v3_t8192", "qwen3_30b_skewed_t16384",
        "qwen3_235b_train_t8192", "deepseek_v3_ep8_rank_t8192"]


@pytest.mark.parametrize("name", FULL)
def test_layer_full_size_sampled(name):
    cfg = CONFIGS[name]
    print(f"[layer full] {name}", flush=True)
    inp, layer, out = _run(cfg)
    prec = prec_of(cfg)
    idx, w, amb, same = _route_and_check(cfg, inp, out, max_ambiguous_frac=0.01)
    _maps(out, inp, cfg)
    p = O.permute(None, idx, w, cfg.E)
    counts = np.diff(p["offsets"])
    print(f"  rows/expert min {counts.min()} max {counts.max()} zero {int((counts == 0).sum())}",
          flush=True)
    if cfg.zipf_s > 0:
        assert (counts == 0).any(), "the skewed workload must leave an expert empty"
    if same:
        assert_equal_int("expert_offsets", out["expert_offsets"], p["offsets"])
        assert_equal_int("row_token", out["row_token"], p["row_token"])
        assert_equal_int("token_row", out["token_row"], p["token_row"])
        rt = torch.as_tensor(p["row_token"], device="cuda").long()
        assert torch.equal(out["x_perm"], inp["x"][rt])
    n = 16 if cfg.E >= 256 else 48
    toks = np.array([t for t in sample_tokens(cfg.T, n) if not amb[t]])
    tt = torch.as_tensor(toks, device="cuda")
    ref = oracle_sampled_forward(cfg, inp, toks, idx, w)
    rows = out["token_row"][tt].reshape(-1).long()
    assert_close("y_perm[sample]", out["y_perm"][rows], ref["y_rows"].reshape(-1, cfg.d), prec)
    if out["gu_save"] is not None:
        assert_close("gu_save[sample]", layer.gu_views()[0][rows],
                     ref["gu_rows"].reshape(-1, 2 * cfg.F), prec)
    if cfg.F_shared > 0:
        assert_close("y_shared[sample]", out["y_shared"][tt], ref["ys"], prec)
    assert_close("y[sample]", out["y"][tt], ref["y"], prec)
    del layer, out, inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["bf16_sigmoid_groups_shared_t200", "bf16_generic_shapes_t77",
                                  "f32_odd_t37", "qwen3_235b_train_t8192"])
def test_backward_recompute_matches_saved_bitwise(name):
    """Selective rematerialisation: a forward that keeps no g | u and a
    backward that reruns FC1 give bitwise the gradients of the saved path
    (the same FC1 kernels and schedule recompute the same values)."""
    from mixture_experts_layer_logits_amd import MoELayer
    cfg = SMALL.get(name) or CONFIGS[name]
    print(f"[backward recompute] {name}", flush=True)
    inp = make_inputs(cfg, device="cuda")
    dy = inp.get("dy")
    if dy is None:
        dy = normal((cfg.T, cfg.d), 1.0, cfg.torch_dtype, "cuda", child_seed(9, "dy"))
    saved = MoELayer(cfg, save_gu=True)
    saved.forward(inp)
    g1 = {k: (v.clone() if v is not None else None) for k, v in saved.backward(inp, dy).items()}
    remat = MoELayer(cfg, recompute=True)
    out = remat.forward(inp)
    assert out["gu_save"] is None
    g2 = remat.backward(inp, dy)
    torch.cuda.synchronize()
    for k, v in g1.items():
        if v is None:
            assert g2[k] is None, k
        else:
            assert torch.equal(v, g2[k]), k
    del saved, remat
    torch.cuda.empty_cache()
