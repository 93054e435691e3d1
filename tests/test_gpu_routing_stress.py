"""The layer under extreme and deliberately imbalanced routing, end to end on
the GPU against the oracle.

* Every token routed to one expert: a router bias of 100 on one expert of 8
  (top-1), so one group holds all T rows and seven are empty; forward and
  backward compared in full.
* Round-robin routing at the Qwen3-235B training shape: token t takes
  experts (t k + j) mod E, so every expert gets exactly T k / E rows.
* Imbalanced round-robin routing at the same shape (the Primus blog's
  MegaMoE section repeats its measurement under a deliberately imbalanced
  round-robin routing): expert e appears (e mod 5) times per cycle of the
  schedule, so loads range from 0 to about 1000 rows.

The round-robin routings enter as router scores with the picks planted on
top (moe_route_topk from given scores); the oracle routes from the same
scores.  Indices and every map must match the oracle bit for bit; y, and in
the training runs dx, d_gate, d_logits and whole experts' weight gradients,
are compared on sampled tokens and experts, each evaluated by the oracle one
expert at a time.
"""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import (CONFIGS, MoEConfig, make_inputs, planted_logits, round_robin_topk,
                        weighted_round_robin_topk)
from parity_util import (assert_close, assert_equal_int, check_maps_valid, np64,
                         oracle_sampled_backward, oracle_sampled_forward, prec_of,
                         route_and_check, sample_tokens)

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _grads_equal_ref(g, ref, keys, prec):
    for key in keys:
        assert_close(key, g[key], ref[key], prec)


@pytest.mark.parametrize("k", [1, 2])
def test_all_tokens_to_one_expert(k):
    """A router bias of 100 on expert 5 (and 90 on expert 2 for k = 2) sends
    every token there; the other experts get no rows, so their weight
    gradients are exactly zero."""
    from mixture_experts_layer_logits_amd import MoELayer
    cfg = MoEConfig(f"all_to_one_k{k}", T=2048, d=256, E=8, k=k, F=512, backward=True)
    _log(f"[routing stress] {cfg.name}")
    inp = make_inputs(cfg, device="cuda")
    bias = torch.zeros(cfg.E, dtype=torch.float32)
    bias[5] = 100.0
    if k == 2:
        bias[2] = 90.0
    inp["router_bias"] = bias.cuda()
    layer = MoELayer(cfg)
    out = layer.forward(inp)
    g = layer.backward(inp, inp["dy"])
    torch.cuda.synchronize()
    prec = prec_of(cfg)
    idx, w, amb, same = route_and_check(cfg, inp, out, max_ambiguous_frac=0.0)
    assert same and not amb.any()
    hot = [5] if k == 1 else [5, 2]
    assert np.all(idx == np.asarray(hot)[None, :])
    check_maps_valid(out, idx, out["topk_w"].cpu().numpy(), cfg.E, x=inp["x"])
    ref = O.forward(inp, cfg, prec=prec, save_gu=True)
    counts = np.diff(ref["offsets"])
    assert sorted(np.nonzero(counts)[0].tolist()) == sorted(hot)
    assert np.all(counts[hot] == cfg.T)
    for key in ("expert_offsets", "row_token", "token_row"):
        assert_equal_int(key, out[key], ref["offsets" if key == "expert_offsets" else key])
    assert_close("y_perm", out["y_perm"], ref["y_perm"], prec)
    assert_close("gu_save", layer.gu_views()[0], ref["gu_save"], prec)
    assert_close("y", out["y"], ref["y"], prec)
    bw = O.ffn_backward(np64(inp["dy"]), ref["x_perm"], ref["gu_save"], ref["y_perm"],
                        ref["offsets"], ref["token_row"], ref["topk_idx"], ref["topk_w"],
                        ref["route_logits"], np64(inp["w_gate"]), np64(inp["w_up"]),
                        np64(inp["w_down"]), cfg.score, cfg.renorm, prec)
    _grads_equal_ref(g, bw, ("dx", "d_gate", "d_logits"), prec)
    for e in hot:
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert_close(f"{key}[{e}]", g[key][e], bw[key][e], prec)
    for e in range(cfg.E):
        if e not in hot:
            for key in ("dw_gate", "dw_up", "dw_down"):
                assert torch.all(g[key][e] == 0), (key, e)


@pytest.mark.parametrize("routing", ["round_robin", "imbalanced_round_robin"])
def test_round_robin_routing_training_shape(routing):
    from mixture_experts_layer_logits_amd import MoELayer
    cfg = CONFIGS["qwen3_235b_train_t8192"]
    _log(f"[routing stress] {routing} at {cfg.name}")
    if routing == "round_robin":
        planned = round_robin_topk(cfg.T, cfg.E, cfg.k)
    else:
        planned = weighted_round_robin_topk(cfg.T, cfg.E, cfg.k, [e % 5 for e in range(cfg.E)])
    logits = planted_logits(planned, cfg.E, seed=21)
    inp = make_inputs(cfg, device="cuda")
    inp["logits"] = logits.cuda()
    layer = MoELayer(cfg)
    out = layer.forward(inp)
    g = layer.backward(inp, inp["dy"])
    torch.cuda.synchronize()
    prec = prec_of(cfg)
    l64 = np64(logits)
    idx, w = O.route(l64, cfg.k, cfg.score, cfg.renorm, prec="f32")
    assert np.array_equal(idx, planned.numpy())        # the oracle sees the planted picks
    assert_equal_int("topk_idx", out["topk_idx"], idx)
    assert_close("topk_w", out["topk_w"], w, "f32")
    check_maps_valid(out, idx, out["topk_w"].cpu().numpy(), cfg.E, x=inp["x"])
    p = O.permute(None, idx, w, cfg.E)
    counts = np.diff(p["offsets"])
    if routing == "round_robin":
        assert np.all(counts == cfg.T * cfg.k // cfg.E)
    else:
        assert (counts == 0).sum() > 0 and counts.max() > 3 * counts[counts > 0].min()
    _log(f"  rows/expert min {counts.min()} max {counts.max()} zero {int((counts == 0).sum())}")
    for key in ("expert_offsets", "row_token", "token_row"):
        assert_equal_int(key, out[key], p["offsets" if key == "expert_offsets" else key])
    toks = sample_tokens(cfg.T, 48)
    tt = torch.as_tensor(toks, device="cuda")
    ref = oracle_sampled_forward(cfg, inp, toks, idx, w)
    rows = out["token_row"][tt].reshape(-1).long()
    assert_close("y_perm[sample]", out["y_perm"][rows], ref["y_rows"].reshape(-1, cfg.d), prec)
    assert_close("gu_save[sample]", layer.gu_views()[0][rows],
                 ref["gu_rows"].reshape(-1, 2 * cfg.F), prec)
    assert_close("y[sample]", out["y"][tt], ref["y"], prec)
    heavy = int(np.argmax(counts))
    empty = [int(e) for e in np.nonzero(counts == 0)[0][:1]]
    experts = sorted({1, cfg.E // 2 + 2, heavy, *empty})
    rb = oracle_sampled_backward(cfg, inp, p, idx, w, l64, toks, experts)
    assert_close("dx[sample]", g["dx"][tt], rb["dx"], prec)
    assert_close("d_gate[sample]", g["d_gate"][tt], rb["d_gate"], prec)
    assert_close("d_logits[sample]", g["d_logits"][tt], rb["d_logits"], prec)
    for e in experts:
        for key in ("dw_gate", "dw_up", "dw_down"):
            if rb["dw"][e] is None:
                assert torch.all(g[key][e] == 0), (key, e)
            else:
                assert_close(f"{key}[{e}]", g[key][e], rb["dw"][e][key], prec)
    del layer, out, g, inp
    torch.cuda.empty_cache()
