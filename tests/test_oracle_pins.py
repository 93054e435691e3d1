"""Pins of the CPU oracle against facts other than itself.

Each test checks an oracle function against something independent of its
code: a library routine that computes the same thing another way (a stable
sort, torch's bf16 conversion, scipy's softmax), a closed form, brute force on
tiny inputs with plain Python loops, an invariant of the method, a number the
pages print, or central finite differences of the oracle's own forward in fp64.
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import softmax as sp_softmax

import oracle as O
from moe_inputs import CONFIGS, MoEConfig, expert_weight, make_inputs, \
    round_robin_topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def test_round_bf16_matches_torch_conversion_of_fp32_values():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(200000).astype(np.float32)
    a[:1000] *= 1e-38          # subnormal range
    a[1000:2000] *= 1e30
    # exact halfway points between neighbouring bf16 values
    base = torch.from_numpy(rng.standard_normal(1000).astype(np.float32))
    base = base.to(torch.bfloat16).float().numpy()
    half = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    a = np.concatenate([a, half, np.float32([0.0, -0.0])])
    ref = torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    got = O.round_bf16(a.astype(np.float64))
    assert np.array_equal(got, ref.astype(np.float64))


def test_round_bf16_ties_to_even_and_fixed_points():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.
    assert O.round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: even is 1 + 2^-6.
    assert O.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    vals = np.array([1.5, -3.25, 2.0 ** -130, 65280.0])
    assert np.array_equal(O.round_bf16(vals), vals)


def test_round_f32_hand_worked_ties_and_subnormals():
    """fp32 keeps 24 significant bits: the spacing above 1 is 2^-23 and the
    smallest subnormal is 2^-149.  Values worked by hand, not by a cast."""
    # halfway between 1 and 1 + 2^-23: the even neighbour is 1
    assert O.round_f32(1.0 + 2.0 ** -24) == 1.0
    # halfway between 1 + 2^-23 (odd) and 1 + 2^-22 (even)
    assert O.round_f32(1.0 + 3 * 2.0 ** -24) == 1.0 + 2.0 ** -22
    # just above halfway rounds up
    assert O.round_f32(1.0 + 2.0 ** -24 + 2.0 ** -40) == 1.0 + 2.0 ** -23
    # just below halfway rounds down, also for negative values
    assert O.round_f32(-(1.0 + 2.0 ** -24 - 2.0 ** -40)) == -1.0
    # between 2 and 4 the spacing doubles: 3 + 2^-23 is halfway, even is 3
    assert O.round_f32(3.0 + 2.0 ** -23) == 3.0
    # subnormals: 1.5 * 2^-149 is halfway between 2^-149 (odd) and 2^-148
    assert O.round_f32(1.5 * 2.0 ** -149) == 2.0 ** -148
    # 2^-150 is halfway between 0 and 2^-149: the even neighbour is 0
    assert O.round_f32(2.0 ** -150) == 0.0
    # 1/3 in fp32 is 11184811 * 2^-25 (0x3eaaaaab)
    assert O.round_f32(1.0 / 3.0) == 11184811 * 2.0 ** -25
    # exactly representable values stay
    vals = np.array([0.5, -1024.75, 2.0 ** -126, 16777215.0])
    assert np.array_equal(O.round_f32(vals), vals)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def _sort_select(keys, k, allowed=None):
    """Independent top-k: a full stable sort by (-key, index) per row."""
    out = []
    for t in range(keys.shape[0]):
        cand = [e for e in range(keys.shape[1])
                if allowed is None or allowed[t, e]]
        cand.sort(key=lambda e: (-keys[t, e], e))
        out.append(cand[:k])
    return np.array(out, dtype=np.int64)


def test_select_topk_matches_stable_sort_with_ties():
    rng = np.random.default_rng(3)
    keys = np.round(rng.standard_normal((300, 16)), 1)   # many exact ties
    for k in (1, 2, 5, 16):
        assert np.array_equal(O.select_topk(keys, k), _sort_select(keys, k))
    allowed = rng.random((300, 16)) < 0.6
    allowed[:, :5] = True
    assert np.array_equal(O.select_topk(keys, 4, allowed),
                          _sort_select(keys, 4, allowed))


def test_constructed_ties_go_to_lowest_index():
    l = np.zeros((3, 8), dtype=np.float32)
    l[1, [2, 5, 7]] = 1.0
    l[2, :] = -2.0
    l[2, 6] = 3.0
    idx, w = O.route_softmax(l, 2)
    assert idx.tolist() == [[0, 1], [2, 5], [6, 0]]
    assert np.allclose(w[0], [0.5, 0.5])


def test_softmax_top2_gates_closed_form():
    rng = np.random.default_rng(4)
    l = rng.standard_normal((200, 8)).astype(np.float32)
    idx, w = O.route_softmax(l, 2)
    for t in range(200):
        l0, l1 = float(l[t, idx[t, 0]]), float(l[t, idx[t, 1]])
        w0 = 1.0 / (1.0 + math.exp(l1 - l0))
        assert abs(w[t, 0] - w0) <= 1e-7 and abs(w[t, 1] - (1 - w0)) <= 1e-7


def test_softmax_gates_renormalise_and_full_softmax_matches_scipy():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((100, 32)).astype(np.float32)
    idx, w = O.route_softmax(l, 6, renorm=1)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 6 * 2.0 ** -23)
    # renormalised gates equal the full softmax renormalised over the picks
    p = sp_softmax(l.astype(np.float64), axis=1)
    ps = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    assert np.allclose(w, ps / ps.sum(axis=1, keepdims=True), rtol=1e-6)
    idx2, w2 = O.route_softmax(l, 6, renorm=0)
    assert np.array_equal(idx, idx2)
    assert np.allclose(w2, ps, rtol=1e-6)
    # selected keys dominate unselected ones
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    mask = np.ones_like(l, dtype=bool)
    np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
    assert np.all(sel.min(axis=1) >= np.where(mask, l, -np.inf).max(axis=1))


def test_sigmoid_single_group_without_bias_is_plain_topk():
    rng = np.random.default_rng(6)
    l = (rng.standard_normal((400, 64)) * 1.5).astype(np.float32)
    idx, w = O.route_sigmoid_grouped(l, 8, 1, 1, None)
    assert np.array_equal(idx, O.select_topk(l, 8).astype(np.int32))
    s = 1.0 / (1.0 + np.exp(-l.astype(np.float64)))
    ss = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    assert np.allclose(w, ss / ss.sum(axis=1, keepdims=True), rtol=1e-6)
    assert np.all(np.abs(w.sum(axis=1) - 1.0) <= 8 * 2.0 ** -23)


def test_sigmoid_group_limited_routing_brute_force():
    rng = np.random.default_rng(7)
    T, E, n_groups, topk_groups, k = 60, 32, 8, 4, 8
    l = (rng.standard_normal((T, E)) * 1.7).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.1).astype(np.float32)
    idx, w = O.route_sigmoid_grouped(l, k, n_groups, topk_groups, bias)
    G = E // n_groups
    for t in range(T):
        s = [np.float32(1.0 / (1.0 + math.exp(-float(v)))) for v in l[t]]
        key = [np.float32(s[e] + bias[e]) for e in range(E)]
        gs = []
        for g in range(n_groups):
            top = sorted(key[g * G:(g + 1) * G], reverse=True)
            gs.append(np.float32(top[0] + top[1]))
        kept = sorted(range(n_groups), key=lambda g: (-gs[g], g))[:topk_groups]
        cand = [e for e in range(E) if e // G in kept]
        cand.sort(key=lambda e: (-key[e], e))
        assert idx[t].tolist() == cand[:k]
        tot = sum(float(s[e]) for e in cand[:k])
        assert np.allclose(w[t], [float(s[e]) / tot for e in cand[:k]],
                           rtol=1e-6)
        assert len({e // G for e in idx[t]}) <= topk_groups


# --------------------------------------------------------------------------
# permutation
# --------------------------------------------------------------------------
def _rand_routing(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def test_permutation_matches_stable_sort_and_invariants():
    rng = np.random.default_rng(8)
    T, E, k, d = 97, 11, 3, 5
    idx = _rand_routing(rng, T, E, k)
    idx[:10] = [0, 1, 2]            # a popular expert set
    w = rng.random((T, k))
    x = rng.standard_normal((T, d))
    p = O.permute(x, idx, w, E)
    # independent: a stable sort of the (t, j) entries by expert id
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(p["row_token"], order // k)
    assert np.array_equal(p["row_gate"], w.reshape(-1)[order])
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(p["counts"], counts)
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    assert p["offsets"][-1] == T * k
    tr = p["token_row"]
    for t in range(T):
        for j in range(k):
            assert p["row_token"][tr[t, j]] == t
            assert np.array_equal(p["x_perm"][tr[t, j]], x[t])
    for e in range(E):
        seg = p["row_token"][p["offsets"][e]:p["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)
    assert sorted(tr.reshape(-1).tolist()) == list(range(T * k))


def test_round_robin_routing_is_balanced():
    # The deliberately balanced routing of the Primus blog's imbalance study
    # gives each expert exactly T*k/E rows, the balanced-routing count
    # bs*N_r/N of the DeepSeek-V3 memory-model page.
    for T, E, k in ((256, 8, 2), (8192, 256, 8), (4096, 128, 8)):
        idx = round_robin_topk(T, E, k).numpy()
        p = O.permute(None, idx, np.ones((T, k)), E)
        assert np.all(p["counts"] == T * k // E)


def test_permute_then_unpermute_with_unit_gates_is_identity():
    rng = np.random.default_rng(9)
    T, E, k, d = 50, 7, 3, 6
    idx = _rand_routing(rng, T, E, k)
    x = O.round_bf16(rng.standard_normal((T, d)))
    p = O.permute(x, idx, np.ones((T, k)), E)
    # one slot at a time with gate 1 gives back x exactly
    for j in range(k):
        onehot = np.zeros((T, k))
        onehot[:, j] = 1.0
        y = O.combine(p["x_perm"], p["token_row"], onehot, None, "f64")
        assert np.array_equal(y, x)
    # renormalised gates over k copies give x up to fp32 rounding
    _, w = O.route_softmax(rng.standard_normal((T, E)).astype(np.float32), k)
    p = O.permute(x, idx, w, E)
    y = O.combine(p["x_perm"], p["token_row"], w, None, "f32")
    assert np.allclose(y, x, rtol=1e-6, atol=1e-6)


# --------------------------------------------------------------------------
# FFN + combine: dense brute force (never permutes)
# --------------------------------------------------------------------------
def _small_inputs(rng, T, d, E, F, Fs=0, prec="f64"):
    rnd = O.rounder(prec)
    inp = dict(
        x=rnd(rng.standard_normal((T, d))),
        w_router=rnd(rng.standard_normal((E, d)) * 0.5),
        w_gate=rnd(rng.standard_normal((E, F, d)) * 0.3),
        w_up=rnd(rng.standard_normal((E, F, d)) * 0.3),
        w_down=rnd(rng.standard_normal((E, d, F)) * 0.3),
        router_bias=None, score_bias=None)
    if Fs:
        inp.update(ws_gate=rnd(rng.standard_normal((Fs, d)) * 0.3),
                   ws_up=rnd(rng.standard_normal((Fs, d)) * 0.3),
                   ws_down=rnd(rng.standard_normal((d, Fs)) * 0.3))
    return inp


def _loop_ffn(xt, wg, wu, wd, rnd, rnd_out=None):
    """Plain-Python SwiGLU FFN of one token vector (h rounded by rnd, the
    output by rnd_out, default rnd)."""
    rnd_out = rnd if rnd_out is None else rnd_out
    F, d = len(wg), len(xt)
    h = []
    for f in range(F):
        g = sum(xt[i] * wg[f][i] for i in range(d))
        u = sum(xt[i] * wu[f][i] for i in range(d))
        h.append(float(rnd(g / (1.0 + math.exp(-g)) * u)))
    return [float(rnd_out(sum(h[f] * wd[i][f] for f in range(F))))
            for i in range(d)]


@pytest.mark.parametrize("prec", ["f64", "bf16"])
@pytest.mark.parametrize("shared", [0, 3])
def test_forward_matches_dense_bruteforce(prec, shared):
    rng = np.random.default_rng(10 + shared)
    T, d, E, k, F = 9, 4, 5, 2, 3
    inp = _small_inputs(rng, T, d, E, F, shared, prec)
    cfg = MoEConfig("t", T=T, d=d, E=E, k=k, F=F, F_shared=shared)
    out = O.forward(inp, cfg, prec=prec)
    rnd = O.rounder(prec)
    # dense gate matrix G[t, e] from the routing output
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            G[t, out["topk_idx"][t, j]] = out["topk_w"][t, j]
    x = inp["x"].tolist()
    for t in range(T):
        acc = [0.0] * d
        if shared:
            ys = _loop_ffn(x[t], inp["ws_gate"].tolist(), inp["ws_up"].tolist(),
                           inp["ws_down"].tolist(), rnd)
            acc = [a + b for a, b in zip(acc, ys)]
        for e in range(E):
            if G[t, e] == 0.0:
                continue
            ye = _loop_ffn(x[t], inp["w_gate"][e].tolist(),
                           inp["w_up"][e].tolist(), inp["w_down"][e].tolist(),
                           rnd)
            acc = [a + G[t, e] * b for a, b in zip(acc, ye)]
        tol = 1e-12 if prec == "f64" else 1e-6
        assert np.allclose(out["y"][t], acc, rtol=tol, atol=tol)


@pytest.mark.parametrize("shared", [0, 3])
def test_ffn_combine_matches_dense_bruteforce(shared):
    """The FFN with the combine folded into FC2: per token, a plain loop over
    the experts its dense gate row selects, h rounded to bf16 and the expert
    outputs kept exact; y rounded to fp32 once."""
    rng = np.random.default_rng(30 + shared)
    T, d, E, k, F = 11, 4, 5, 3, 3
    inp = _small_inputs(rng, T, d, E, F, shared, "bf16")
    cfg = MoEConfig("t", T=T, d=d, E=E, k=k, F=F, F_shared=shared)
    out = O.forward(inp, cfg, prec="bf16")
    sh = (inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"]) if shared else None
    y = O.grouped_ffn_combine(out["x_perm"], out["offsets"], out["token_row"],
                              out["topk_w"], inp["w_gate"], inp["w_up"],
                              inp["w_down"], sh, "bf16")
    rnd = O.rounder("bf16")
    exact = lambda v: v
    G = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            G[t, out["topk_idx"][t, j]] = out["topk_w"][t, j]
    x = inp["x"].tolist()
    for t in range(T):
        acc = [0.0] * d
        if shared:
            ys = _loop_ffn(x[t], inp["ws_gate"].tolist(), inp["ws_up"].tolist(),
                           inp["ws_down"].tolist(), rnd, exact)
            acc = [a + b for a, b in zip(acc, ys)]
        for e in range(E):
            if G[t, e] != 0.0:
                ye = _loop_ffn(x[t], inp["w_gate"][e].tolist(), inp["w_up"][e].tolist(),
                               inp["w_down"][e].tolist(), rnd, exact)
                acc = [a + G[t, e] * b for a, b in zip(acc, ye)]
        want = np.array(acc, dtype=np.float32).astype(np.float64)
        assert np.allclose(y[t], want, rtol=1e-7, atol=1e-12)
    # the unfused layer rounds each expert output to bf16 first
    assert not np.array_equal(y, out["y"])
    assert np.allclose(y, out["y"], rtol=2e-2, atol=1e-3)


def test_ffn_combine_hand_worked():
    """One token, one expert (gate 1), d = 2, F = 1: g = 1, u = 2, so
    h = bf16(2 silu(1)) = bf16(1.46212) = 1.4609375 (1.0111011 in binary;
    the next bf16 value up is 1.46875), and with w_down = (1/3, 1/7) the
    combined output is fp32(h / 3), fp32(h / 7); the unfused layer's expert
    output is bf16(h / 3) = 0.486328125 instead."""
    x = np.array([[1.0, 2.0]])
    h = 1.4609375
    y = O.grouped_ffn_combine(x, np.array([0, 1]), np.array([[0]]), np.array([[1.0]]),
                              np.array([[[1.0, 0.0]]]), np.array([[[0.0, 1.0]]]),
                              np.array([[[1 / 3], [1 / 7]]]), None, "bf16")
    assert y.tolist() == [[float(np.float32(h / 3)), float(np.float32(h / 7))]]
    yp, _ = O.grouped_ffn(x, np.array([0, 1]), np.array([[[1.0, 0.0]]]),
                          np.array([[[0.0, 1.0]]]), np.array([[[1 / 3], [1 / 7]]]), "bf16")
    assert yp[0, 0] == 0.486328125


def test_hand_worked_two_expert_example():
    """Closed form: x = (1, 2), logits (1, 0), each expert picks one input
    coordinate for g and the other for u, F = 1.  Then
    y = (2 sigmoid(1) silu(1), (1 - sigmoid(1)) silu(2))."""
    inp = dict(x=np.array([[1.0, 2.0]]), w_router=np.eye(2),
               router_bias=np.array([0.0, -2.0]), score_bias=None,
               w_gate=np.array([[[1.0, 0.0]], [[0.0, 1.0]]]),
               w_up=np.array([[[0.0, 1.0]], [[1.0, 0.0]]]),
               w_down=np.array([[[1.0], [0.0]], [[0.0], [1.0]]]))
    cfg = MoEConfig("hand", T=1, d=2, E=2, k=2, F=1)
    logits = np.array([[1.0, 0.0]])
    out = O.forward(inp, cfg, prec="f64", logits=logits)
    sig = lambda z: 1.0 / (1.0 + math.exp(-z))
    assert out["topk_idx"].tolist() == [[0, 1]]
    assert np.allclose(out["topk_w"], [[sig(1), 1 - sig(1)]], rtol=1e-15)
    assert np.allclose(out["y"], [[2 * sig(1) * 1 * sig(1),
                                   (1 - sig(1)) * 2 * sig(2)]], rtol=1e-14)
    # the oracle's own router reproduces those logits: x . I + (0, -2)
    assert np.allclose(out["logits"], logits)


def test_single_expert_top1_is_a_plain_swiglu_mlp():
    rng = np.random.default_rng(11)
    T, d, F = 13, 6, 5
    inp = _small_inputs(rng, T, d, 1, F)
    cfg = MoEConfig("mlp", T=T, d=d, E=1, k=1, F=F)
    out = O.forward(inp, cfg, prec="f64")
    x = inp["x"]
    g = np.einsum("td,fd->tf", x, inp["w_gate"][0])
    u = np.einsum("td,fd->tf", x, inp["w_up"][0])
    h = g * sp_expit(g) * u
    y = np.einsum("tf,df->td", h, inp["w_down"][0])
    assert np.allclose(out["y"], y, rtol=1e-12, atol=1e-14)
    assert np.all(out["topk_w"] == 1.0)


def sp_expit(z):
    from scipy.special import expit
    return expit(z)


def test_deepseek_v3_expert_parameter_count():
    vals = {}
    with open(os.path.join(GOLDEN, "deepseek_v3_expert_params.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, v = line.split()
                vals[key] = int(v)
    cfg = CONFIGS["deepseek_v3_t8192"]
    assert (cfg.d, cfg.F) == (vals["hidden"], vals["expert_width"])
    n = sum(expert_weight(cfg, name, 0).numel()
            for name in ("w_gate", "w_up", "w_down"))
    assert n == vals["params_per_expert"] == cfg.expert_params()
    assert n * vals["expert_stacks_per_device"] == \
        vals["expert_params_per_device"]


# --------------------------------------------------------------------------
# backward: finite differences of the fp64 forward
# --------------------------------------------------------------------------
def _fwd_loss(x, logits, wg, wu, wd, dy, cfg, bias, shared=None):
    inp = dict(x=x, w_router=np.zeros((cfg.E, cfg.d)), router_bias=None,
               score_bias=bias, w_gate=wg, w_up=wu, w_down=wd)
    if shared is not None:
        inp.update(ws_gate=shared[0], ws_up=shared[1], ws_down=shared[2])
    out = O.forward(inp, cfg, prec="f64", logits=logits, save_gu=True)
    return float((out["y"] * dy).sum()), out


@pytest.mark.parametrize("score,renorm,groups,Fs", [
    (O.SCORE_SOFTMAX, 1, (1, 1), 0), (O.SCORE_SOFTMAX, 0, (1, 1), 0),
    (O.SCORE_SIGMOID, 1, (2, 1), 0), (O.SCORE_SIGMOID, 0, (1, 1), 0),
    (O.SCORE_SIGMOID, 1, (2, 1), 2)])
def test_backward_matches_central_differences(score, renorm, groups, Fs):
    rng = np.random.default_rng(12 + score * 2 + renorm + Fs)
    T, d, E, k, F = 5, 4, 4, 2, 3
    cfg = MoEConfig("fd", T=T, d=d, E=E, k=k, F=F, F_shared=Fs, score=score,
                    renorm=renorm, n_groups=groups[0], topk_groups=groups[1])
    x = rng.standard_normal((T, d))
    # well separated logits so that no selection flips under the step
    logits = np.stack([rng.permutation(E) * 0.7 + rng.random(E) * 0.1
                       for _ in range(T)]) - 1.2
    bias = (rng.standard_normal(E) * 0.05) if score == O.SCORE_SIGMOID else None
    wg = rng.standard_normal((E, F, d)) * 0.5
    wu = rng.standard_normal((E, F, d)) * 0.5
    wd = rng.standard_normal((E, d, F)) * 0.5
    dy = rng.standard_normal((T, d))
    sh = None
    if Fs:
        sh = (rng.standard_normal((Fs, d)) * 0.5, rng.standard_normal((Fs, d)) * 0.5,
              rng.standard_normal((d, Fs)) * 0.5)
    _, out = _fwd_loss(x, logits, wg, wu, wd, dy, cfg, bias, sh)
    shared = None
    if Fs:
        shared = dict(x=x, gu=out["gu_shared"], ws_gate=sh[0], ws_up=sh[1], ws_down=sh[2])
    bw = O.ffn_backward(dy, out["x_perm"], out["gu_save"], out["y_perm"],
                        out["offsets"], out["token_row"], out["topk_idx"],
                        out["topk_w"], logits, wg, wu, wd, score, renorm,
                        prec="f64", shared=shared)
    eps = 1e-6

    def fd(arr, fn):
        g = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            old = arr[i]
            arr[i] = old + eps
            lp = fn()
            arr[i] = old - eps
            lm = fn()
            arr[i] = old
            g[i] = (lp - lm) / (2 * eps)
        return g

    loss = lambda: _fwd_loss(x, logits, wg, wu, wd, dy, cfg, bias, sh)[0]
    checks = [("dx", x), ("dw_gate", wg), ("dw_up", wu), ("dw_down", wd),
              ("d_logits", logits)]
    if Fs:
        checks += [("dws_gate", sh[0]), ("dws_up", sh[1]), ("dws_down", sh[2])]
    for name, arr in checks:
        num = fd(arr, loss)
        assert np.allclose(bw[name], num, rtol=1e-6, atol=1e-8), name
    # the gate gradient: perturb the gates inside the combine only
    w = out["topk_w"].copy()
    comb = lambda: float((O.combine(out["y_perm"], out["token_row"], w, None,
                                    "f64") * dy).sum())
    assert np.allclose(bw["d_gate"], fd(w, comb), rtol=1e-6, atol=1e-8)
    if score == O.SCORE_SOFTMAX:
        # the softmax Jacobian's rows sum to zero
        assert np.allclose(bw["d_logits"].sum(axis=1), 0.0, atol=1e-12)


def test_zero_row_experts_have_exactly_zero_weight_gradients():
    rng = np.random.default_rng(13)
    T, d, E, k, F = 20, 6, 6, 2, 4
    idx = np.stack([rng.permutation(4)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    x = O.round_bf16(rng.standard_normal((T, d)))
    p = O.permute(x, idx, w, E)
    wg = O.round_bf16(rng.standard_normal((E, F, d)) * 0.1)
    wu = O.round_bf16(rng.standard_normal((E, F, d)) * 0.1)
    wd = O.round_bf16(rng.standard_normal((E, d, F)) * 0.1)
    y_perm, gu = O.grouped_ffn(p["x_perm"], p["offsets"], wg, wu, wd, "bf16",
                               save_gu=True)
    dy = O.round_bf16(rng.standard_normal((T, d)))
    bw = O.ffn_backward(dy, p["x_perm"], gu, y_perm, p["offsets"],
                        p["token_row"], idx, w, rng.standard_normal((T, E)),
                        wg, wu, wd, prec="bf16")
    for e in (4, 5):
        assert p["counts"][e] == 0
        for name in ("dw_gate", "dw_up", "dw_down"):
            assert np.all(bw[name][e] == 0.0)
    for e in range(4):
        assert np.any(bw["dw_gate"][e] != 0.0)


# --------------------------------------------------------------------------
# the workloads' input recipe
# --------------------------------------------------------------------------
def test_dispatch_grad_rounds_each_scaled_row_to_bf16_once():
    """dY_perm[token_row[t, j]] = bf16(w[t, j] dy[t]), worked by hand: the
    product is formed exactly and rounded once, to nearest, ties to even.
    bf16 keeps 8 significant bits: the spacing is 2^-7 in [1, 2), 2^-6 in
    [2, 4), 2^-8 in [0.5, 1) and 2^-9 in [0.25, 0.5)."""
    w13 = 11184811 * 2.0 ** -25                   # fp32(1/3) = 0.3333333432...
    dy = np.array([[1.0, 3.0, 1.5, -3.0, 2.0, -1.0]])
    w = np.array([[1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, w13]])
    tr = np.array([[2, 0, 1]])                    # slot j goes to row tr[j]
    dY = O.dispatch_grad(dy, tr, w, 3, "bf16")
    # w = 1 + 2^-8: 1 + 2^-8 and 2 + 2^-7 (and their negatives) are ties that
    # go to the even neighbour; 3 + 0.75 * 2^-6 and 1.5 + 0.75 * 2^-7 round up
    assert dY[2].tolist() == [1.0, 3.015625, 1.5078125, -3.015625, 2.0, -1.0]
    # w = 1 + 3 * 2^-8: 1 + 1.5 * 2^-7 and 2 + 1.5 * 2^-6 are ties whose even
    # neighbour lies above; 3 + 2.25 * 2^-6 and 1.5 + 2.25 * 2^-7 round down
    assert dY[0].tolist() == [1.015625, 3.03125, 1.515625, -3.03125, 2.03125, -1.015625]
    # w = fp32(1/3): 0.3333333433 -> 171 * 2^-9; 1.0000000298 -> 1;
    # 0.5000000149 -> 0.5; 0.6666666865 -> 171 * 2^-8
    assert dY[1].tolist() == [0.333984375, 1.0, 0.5, -1.0, 0.66796875, -0.333984375]
    # unrounded (the fp64 variant) the products differ from these
    assert O.dispatch_grad(dy, tr, w, 3, "f64")[1][2] != 0.5


def test_inputs_are_seeded_and_shaped():
    cfg = CONFIGS["tiny_fp32"]
    a = make_inputs(cfg)
    b = make_inputs(cfg)
    for key in ("x", "w_router", "w_gate", "w_up", "w_down"):
        assert torch.equal(a[key], b[key])
    assert a["x"].shape == (256, 128) and a["w_gate"].shape == (8, 256, 128)
    assert a["w_down"].shape == (8, 128, 256)
    assert abs(float(a["w_gate"].std()) - 0.02) < 1e-3
    # every expert can be regenerated on its own
    assert torch.equal(a["w_up"][5], expert_weight(cfg, "w_up", 5))
    small = CONFIGS["qwen3_30b_skewed_t16384"].replace(T=64, d=64, F=64)
    inp = make_inputs(small)
    rb = inp["router_bias"].numpy()
    # Zipf offsets: -1.2 ln(rank) over a permutation of the ranks 1..E
    ranks = np.exp(-rb / 1.2)
    assert np.allclose(np.sort(ranks), np.arange(1, 129), rtol=1e-5)


# --------------------------------------------------------------------------
# MXFP8: E4M3 rounding and the block scale
# --------------------------------------------------------------------------
def test_e4m3_round_matches_torch_float8_e4m3fn():
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even) is
    an independent implementation of the same rounding for |v| <= 448."""
    rng = np.random.default_rng(21)
    mag = np.exp2(rng.uniform(-12, np.log2(448.0), 20000))
    v = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    # exact halfway points between neighbouring E4M3 values
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    finite = np.unique(codes[np.isfinite(codes)])
    mids = ((finite[:-1] + finite[1:]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).float().numpy()
    ok = np.isfinite(ref)
    assert ok.all()
    assert np.array_equal(O.e4m3_round(v), ref.astype(np.float64))


def test_e4m3_round_is_identity_on_every_code_and_saturates():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    finite = codes[np.isfinite(codes)].astype(np.float64)
    assert finite.size == 254                       # two NaN codes, no infinities
    assert np.array_equal(O.e4m3_round(finite), finite)
    assert finite.max() == 448.0 and np.min(finite[finite > 0]) == 2.0 ** -9
    assert np.array_equal(O.e4m3_round(np.array([449.0, 1e6, -1e6])), [448.0, 448.0, -448.0])


def test_mx_block_scale_rule():
    # amax 1 -> scale 2^(0 - 8); the element 1 becomes 256 exactly
    q, s = O.mx_quantize(np.r_[1.0, np.zeros(31)])
    assert s.tolist() == [-8.0] and q[0] == 256.0
    # amax 448 * 2^10 -> scale 2^(18 - 8) = 2^10, element 448 exactly; 3 / 2^10
    # is 1.5 subnormal quanta (2^-9) and rounds to the even neighbour, 2^-8
    q, s = O.mx_quantize(np.r_[448.0 * 2 ** 10, 3.0, np.zeros(30)])
    assert s.tolist() == [10.0] and q[0] == 448.0 and q[1] == 2.0 ** -8
    # a value just below the next power of two keeps the lower exponent
    q, s = O.mx_quantize(np.r_[1.99, np.zeros(31)])
    assert s.tolist() == [-8.0] and q[0] == 448.0   # 1.99 * 256 = 509 saturates
    # an all-zero block: smallest E8M0 scale, zero elements
    q, s = O.mx_quantize(np.zeros(32))
    assert s.tolist() == [-127.0] and not q.any()
    # blocks are independent and run along the last axis
    a = np.stack([np.r_[np.ones(32), 4 * np.ones(32)], np.r_[0.5 * np.ones(32), np.ones(32)]])
    _, s = O.mx_quantize(a)
    assert s.tolist() == [[-8.0, -6.0], [-9.0, -8.0]]


def test_mx_round_is_idempotent_and_bounded():
    rng = np.random.default_rng(22)
    a = rng.standard_normal((8, 256)) * np.exp2(rng.integers(-10, 10, (8, 1)))
    r = O.mx_round(a)
    assert np.array_equal(O.mx_round(r), r)
    # With the scale 2^(floor(log2 amax) - 8) a block's largest elements land
    # in [256, 512) * 2^s; those at or above 448 * 2^s saturate to exactly
    # +-448 * 2^s, every other element not below the smallest normal is
    # within half an E4M3 quantum (relative 2^-4).
    _, s = O.mx_quantize(a)
    scale = np.repeat(np.exp2(s), 32, axis=1)
    sat = np.abs(a) >= 448.0 * scale
    assert np.array_equal(np.abs(r[sat]), 448.0 * scale[sat])
    normal = ~sat & (np.abs(a) >= 2.0 ** -6 * scale)
    assert np.all(np.abs(r - a)[normal] <= np.abs(a)[normal] * 2.0 ** -4)


def _e4m3_nearest_brute(v, table):
    """Nearest E4M3 value by search over the decoded code table, ties to the
    value whose code is even (the last mantissa bit 0); beyond 448 the
    largest finite value (saturation)."""
    best = None
    for code, val in table:
        d = abs(v - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, val, code)
    return best[1]


def _mx_round_brute(a, table):
    """MX rounding of a 1-D array in blocks of 32, with the block exponent
    taken from math.frexp (amax = m * 2^e, 0.5 <= m < 1, so floor(log2 amax)
    is e - 1)."""
    import math
    out = []
    for b in range(0, len(a), 32):
        blk = [float(x) for x in a[b:b + 32]]
        amax = max(abs(x) for x in blk)
        s = -127 if amax == 0.0 else max(-127, math.frexp(amax)[1] - 1 - 8)
        out += [_e4m3_nearest_brute(x / 2.0 ** s, table) * 2.0 ** s for x in blk]
    return out


def test_swiglu_ffn_mxfp8_by_brute_force():
    """The MXFP8 expert on a tiny case with Python loops: x, w_gate, w_up
    quantised along d, w_down along F, h = silu(g) u quantised along F, y
    rounded to bf16.  Independent of the oracle's rounding code (table search
    over torch's E4M3 decoding, frexp exponents)."""
    import math
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    table = [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] >= 0]
    table += [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] < 0]
    rng = np.random.default_rng(23)
    n, d, F = 3, 64, 64
    x = rng.standard_normal((n, d)) * np.exp2(rng.integers(-3, 3, (n, 1)))
    wg, wu = rng.standard_normal((F, d)) * 0.1, rng.standard_normal((F, d)) * 0.1
    wd = rng.standard_normal((d, F)) * 0.1
    xq = [_mx_round_brute(x[i], table) for i in range(n)]
    wgq = [_mx_round_brute(wg[f], table) for f in range(F)]
    wuq = [_mx_round_brute(wu[f], table) for f in range(F)]
    wdq = [_mx_round_brute(wd[j], table) for j in range(d)]
    y = np.zeros((n, d))
    hq_all = []
    for i in range(n):
        h = []
        for f in range(F):
            g = sum(xq[i][c] * wgq[f][c] for c in range(d))
            u = sum(xq[i][c] * wuq[f][c] for c in range(d))
            h.append(g / (1.0 + math.exp(-g)) * u)
        hq = _mx_round_brute(np.array(h), table)
        hq_all.append(hq)
        for j in range(d):
            y[i, j] = sum(hq[f] * wdq[j][f] for f in range(F))
    ref = O.swiglu_ffn_mxfp8(x, wg, wu, wd)
    # the loops sum in another order than the library matmul, so an h value
    # on a rounding boundary may land one E4M3 step away; nearly all match
    hq_all = np.array(hq_all)
    assert np.mean(ref["h"] == hq_all) >= 0.99
    assert np.allclose(ref["h"], hq_all, rtol=2.0 ** -3, atol=0)
    y_bf16 = torch.from_numpy(y).float().to(torch.bfloat16).double().numpy()
    assert np.allclose(O.as64(ref["y"]), y_bf16, rtol=2.0 ** -7, atol=1e-12)


def test_expert_backward_mxfp8_by_brute_force():
    """The MXFP8 data-gradient GEMMs on a tiny case with Python loops: dY and
    the columns of W_d quantised along d give dh; [dg | du] and the columns
    of [W_g; W_u] quantised along F give dX (rounded to bf16).  The MX
    rounding is the brute-force one (table search over torch's E4M3
    decoding, frexp exponents), independent of the oracle's."""
    import math
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    table = [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] >= 0]
    table += [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] < 0]
    rng = np.random.default_rng(29)
    n, d, F = 3, 64, 64
    rb = O.round_bf16
    dY = rb(rng.standard_normal((n, d)) * np.exp2(rng.integers(-3, 3, (n, 1))))
    x = rb(rng.standard_normal((n, d)))
    gu = rb(rng.standard_normal((n, 2 * F)))
    wg, wu = rb(rng.standard_normal((F, d)) * 0.1), rb(rng.standard_normal((F, d)) * 0.1)
    wd = rb(rng.standard_normal((d, F)) * 0.1)
    ref = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16", mxfp8=True)
    dYq = [_mx_round_brute(dY[i], table) for i in range(n)]
    wd_cols = [_mx_round_brute(wd[:, f], table) for f in range(F)]
    dgu = np.zeros((n, 2 * F))
    for i in range(n):
        for f in range(F):
            dh = sum(dYq[i][c] * wd_cols[f][c] for c in range(d))
            g, u = gu[i, f], gu[i, F + f]
            s = 1.0 / (1.0 + math.exp(-g))
            dgu[i, f] = float(rb(np.array(dh * u * s * (1.0 + g * (1.0 - s)))))
            dgu[i, F + f] = float(rb(np.array(dh * g * s)))
    # dh is summed in another order here, so a bf16 rounding may differ
    assert np.mean(ref["dg"] == dgu[:, :F]) >= 0.97 and np.mean(ref["du"] == dgu[:, F:]) >= 0.97
    assert np.allclose(ref["dg"], dgu[:, :F], rtol=2.0 ** -7, atol=1e-12)
    wcat = np.concatenate([wg, wu], axis=0)
    w_cols = [_mx_round_brute(wcat[:, c], table) for c in range(d)]
    dguq = [_mx_round_brute(np.concatenate([ref["dg"][i], ref["du"][i]]), table) for i in range(n)]
    dX = np.array([[sum(dguq[i][k] * w_cols[c][k] for k in range(2 * F)) for c in range(d)]
                   for i in range(n)])
    assert np.allclose(O.as64(ref["dX"]), rb(dX), rtol=2.0 ** -7, atol=1e-12)
    # the weight gradients use the unquantised operands
    plain = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16")
    assert np.array_equal(plain["dw_down"], ref["dw_down"])   # dY^T h: nothing quantised
    assert np.allclose(ref["dw_gate"], ref["dg"].T @ x, rtol=1e-12, atol=1e-12)


def test_expert_backward_mxfp8_is_exact_on_mx_representable_operands():
    """When dY and W_d hold values that MXFP8 represents exactly (block
    maxima 2, elements in {0, +-1/2, +-1, +-2}: codes 64, 128, 256 times
    2^-7), dh is unchanged by quantisation, so dg, du, h and every weight
    gradient equal the bf16 backward's bit for bit."""
    rng = np.random.default_rng(31)
    n, d, F = 5, 64, 32
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0])
    dY = rng.choice(vals, (n, d))
    dY[:, ::32] = 2.0                                   # every block's amax is 2
    wd = rng.choice(vals, (d, F))
    wd[::32, :] = -2.0
    x = O.round_bf16(rng.standard_normal((n, d)))
    gu = O.round_bf16(rng.standard_normal((n, 2 * F)))
    wg, wu = (O.round_bf16(rng.standard_normal((F, d)) * 0.1) for _ in range(2))
    assert np.array_equal(O.mx_round(dY), dY) and np.array_equal(O.mx_round(wd.T).T, wd)
    a = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16", mxfp8=True)
    b = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16")
    for key in ("dg", "du", "dw_down", "dw_gate", "dw_up"):
        assert np.array_equal(a[key], b[key]), key
    assert not np.array_equal(a["dX"], b["dX"])          # dg | du are not MX-exact
    assert np.allclose(a["dX"], b["dX"], rtol=0.15, atol=0.05 * np.abs(b["dX"]).max())


def test_grouped_ffn_mxfp8_combine_by_brute_force():
    """The MXFP8 FFN with the combine in FC2 on a tiny two-expert case:
    brute-force MX rounding (table search, frexp exponents) of x, the
    weights and h, the expert outputs summed exactly with their gates
    (Python loops), one fp32 rounding; the unfused path differs by the bf16
    rounding of each expert output."""
    import math
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    table = [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] >= 0]
    table += [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] < 0]
    rng = np.random.default_rng(37)
    T, d, F, E = 3, 32, 32, 2
    x = rng.standard_normal((T, d))
    wg = rng.standard_normal((E, F, d)) * 0.2
    wu = rng.standard_normal((E, F, d)) * 0.2
    wd = rng.standard_normal((E, d, F)) * 0.2
    # every token goes to both experts with gates (w, 1 - w)
    idx = np.array([[0, 1]] * T)
    w = np.array([[0.25, 0.75], [0.5, 0.5], [0.875, 0.125]])
    p = O.permute(x, idx, w, E)
    y = O.grouped_ffn_mxfp8_combine(p["x_perm"], p["offsets"], p["token_row"], w, wg, wu, wd)
    q = lambda v: np.array(_mx_round_brute(np.asarray(v, dtype=np.float64), table))
    for t in range(T):
        xq = q(x[t])
        acc = [0.0] * d
        for e in range(E):
            wgq = [q(wg[e][f]) for f in range(F)]
            wuq = [q(wu[e][f]) for f in range(F)]
            wdq = [q(wd[e][i]) for i in range(d)]
            h = []
            for f in range(F):
                g = sum(xq[c] * wgq[f][c] for c in range(d))
                u = sum(xq[c] * wuq[f][c] for c in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            hq = q(h)
            for i in range(d):
                acc[i] += w[t, e] * sum(hq[f] * wdq[i][f] for f in range(F))
        want = np.array(acc, dtype=np.float32).astype(np.float64)
        # an h on an E4M3 rounding boundary could land one step away (another
        # summation order); on this case every element agrees exactly
        assert np.mean(y[t] == want) >= 0.95
        assert np.allclose(y[t], want, rtol=1e-3, atol=1e-6 * np.abs(want).max())
    unfused = O.combine(O.grouped_ffn_mxfp8(p["x_perm"], p["offsets"], wg, wu, wd),
                        p["token_row"], w)
    assert not np.array_equal(y, unfused)
    assert np.allclose(y, unfused, rtol=2e-2, atol=1e-3)


def test_expert_backward_mx_weight_gradients_by_brute_force():
    """The MXFP8 weight-gradient GEMMs on a tiny expert with Python loops:
    every operand column quantised along the expert's 37 rows in blocks of
    32 consecutive rows from the first one (the last block holds 5 rows: its
    zero padding changes no block maximum), then summed over rows exactly.
    dY and h for dW_down, dg | du and x for dW_gate | dW_up.  The MX rounding
    is the brute-force one (table search over torch's E4M3 decoding, frexp
    exponents); h is recomputed here from the saved g, u."""
    import math
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    table = [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] >= 0]
    table += [(c, float(codes[c])) for c in range(256) if np.isfinite(codes[c]) and codes[c] < 0]
    rng = np.random.default_rng(41)
    n, d, F = 37, 32, 32
    rb = O.round_bf16
    dY = rb(rng.standard_normal((n, d)) * np.exp2(rng.integers(-4, 4, (n, 1))))
    x = rb(rng.standard_normal((n, d)))
    gu = rb(rng.standard_normal((n, 2 * F)))
    wg, wu = rb(rng.standard_normal((F, d)) * 0.1), rb(rng.standard_normal((F, d)) * 0.1)
    wd = rb(rng.standard_normal((d, F)) * 0.1)
    r = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16", mx_wgrad=True)
    h = np.array([[float(rb(np.array(gu[t, f] / (1.0 + math.exp(-gu[t, f])) * gu[t, F + f])))
                   for f in range(F)] for t in range(n)])
    col = lambda a, j: _mx_round_brute(a[:, j], table)      # one column along the rows
    qdY = [col(dY, i) for i in range(d)]
    qh = [col(h, f) for f in range(F)]
    qx = [col(x, i) for i in range(d)]
    qdg = [col(r["dg"], f) for f in range(F)]
    qdu = [col(r["du"], f) for f in range(F)]
    dw_down = np.array([[sum(qdY[i][t] * qh[f][t] for t in range(n)) for f in range(F)]
                        for i in range(d)])
    dw_gate = np.array([[sum(qdg[f][t] * qx[i][t] for t in range(n)) for i in range(d)]
                        for f in range(F)])
    dw_up = np.array([[sum(qdu[f][t] * qx[i][t] for t in range(n)) for i in range(d)]
                      for f in range(F)])
    for key, want in (("dw_down", dw_down), ("dw_gate", dw_gate), ("dw_up", dw_up)):
        assert np.allclose(r[key], want, rtol=1e-12, atol=1e-12 * np.abs(want).max()), key
    # and they differ from the unquantised weight gradients
    plain = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16")
    assert not np.allclose(plain["dw_down"], r["dw_down"], rtol=1e-6, atol=0)


def test_mx_weight_gradient_blocks_start_at_each_experts_first_row():
    """ffn_backward with MXFP8 weight gradients quantises each expert's rows
    on their own (blocks restart at the expert's first row, the last one
    padded): expert 1's gradients equal expert_backward on its rows alone,
    and differ from a quantisation whose blocks run on across the previous
    expert's rows."""
    rng = np.random.default_rng(43)
    T, d, E, F = 40, 32, 2, 32
    rb = O.round_bf16
    idx = np.array([[0, 1] if t < 24 else [1, 0] for t in range(T)])
    w = np.full((T, 2), 0.5)
    idx[30:, :] = [[0, 1]] * 10
    p = O.permute(None, idx, w, E)
    counts = np.diff(p["offsets"])
    assert counts[0] % 32 != 0
    R = T * 2
    x_perm = rb(rng.standard_normal((R, d)))
    gu = rb(rng.standard_normal((R, 2 * F)))
    y_perm = rb(rng.standard_normal((R, d)))
    dy = rb(rng.standard_normal((T, d)) * np.exp2(rng.integers(-4, 4, (T, 1))))
    wg, wu = rb(rng.standard_normal((E, F, d)) * 0.1), rb(rng.standard_normal((E, F, d)) * 0.1)
    wd = rb(rng.standard_normal((E, d, F)) * 0.1)
    logits = rng.standard_normal((T, E))
    out = O.ffn_backward(dy, x_perm, gu, y_perm, p["offsets"], p["token_row"], idx, w, logits,
                         wg, wu, wd, prec="bf16", mx_wgrad=True)
    dY = O.dispatch_grad(dy, p["token_row"], w, R, "bf16")
    a, b = int(p["offsets"][1]), int(p["offsets"][2])
    alone = O.expert_backward(dY[a:b], x_perm[a:b], gu[a:b], wg[1], wu[1], wd[1], "bf16",
                              mx_wgrad=True)
    assert np.array_equal(out["dw_gate"][1], O.round_f32(alone["dw_gate"]))
    # blocks aligned to the start of all rows instead of expert 1's first row
    shift = O.mx_round_rows(x_perm)[a:b]
    assert not np.array_equal(shift, O.mx_round_rows(x_perm[a:b]))


def test_mx_weight_gradients_exact_on_mx_representable_operands():
    """When dY and h are exactly representable in MXFP8 along the rows
    (block maxima 2, elements in {0, +-1/2, +-1, +-2}) dW_down is unchanged
    by quantisation, bit for bit; dW_gate, whose dg is not, changes (with
    g = 0, du = dh silu(0) = 0, so dW_up is zero either way)."""
    rng = np.random.default_rng(47)
    n, d, F = 64, 32, 32
    vals = np.array([0.0, 0.5, -0.5, 1.0, -1.0, 2.0, -2.0])
    dY = rng.choice(vals, (n, d))
    dY[::32, :] = 2.0
    x = O.round_bf16(rng.standard_normal((n, d)))
    # g = 0 gives h = silu(0) u = 0: h exactly representable for any u
    gu = np.concatenate([np.zeros((n, F)), O.round_bf16(rng.standard_normal((n, F)))], axis=1)
    wg, wu = (O.round_bf16(rng.standard_normal((F, d)) * 0.1) for _ in range(2))
    wd = O.round_bf16(rng.standard_normal((d, F)) * 0.1)
    assert np.array_equal(O.mx_round_rows(dY), dY)
    a = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16", mx_wgrad=True)
    b = O.expert_backward(dY, x, gu, wg, wu, wd, "bf16")
    assert np.array_equal(a["dw_down"], b["dw_down"])
    assert not np.array_equal(a["dw_gate"], b["dw_gate"])
    assert not np.any(a["dw_up"]) and not np.any(b["dw_up"])
