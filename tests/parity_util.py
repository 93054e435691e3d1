"""Helpers shared by the GPU parity tests: tolerances and the sampled oracle.

Tolerances (the layer's stated bar): bf16 storage with fp32 accumulation:
relative Frobenius error <= 5e-3 and max-abs error <= 2e-2 * max|ref|; fp32
storage: relative error <= 1e-5, read as relative Frobenius error <= 1e-5
and max-abs error <= 1e-5 * max|ref|.  Integer outputs must match exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O

TOL = {"bf16": (5e-3, 2e-2), "f32": (1e-5, 1e-5)}


def np64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def errors(got, ref):
    got, ref = np64(got), np64(ref)
    diff = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / nref if nref > 0 else np.linalg.norm(diff)
    mref = np.abs(ref).max() if ref.size else 0.0
    mabs = np.abs(diff).max() if diff.size else 0.0
    return float(rel), float(mabs), float(mref)


def assert_close(name, got, ref, prec):
    rel_tol, abs_tol = TOL[prec]
    rel, mabs, mref = errors(got, ref)
    assert rel <= rel_tol, f"{name}: relative Frobenius error {rel:.3e} > {rel_tol}"
    assert mabs <= abs_tol * mref + 1e-30, \
        f"{name}: max-abs error {mabs:.3e} > {abs_tol} * {mref:.3e}"
    return rel, mabs


def assert_equal_int(name, got, ref):
    g = got.detach().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    r = np.asarray(ref)
    assert g.shape == r.shape, f"{name}: shape {g.shape} vs {r.shape}"
    bad = np.nonzero(g.reshape(-1) != r.reshape(-1))[0]
    assert bad.size == 0, f"{name}: {bad.size} mismatches, first at {bad[:5]}: " \
        f"{g.reshape(-1)[bad[:5]]} vs {r.reshape(-1)[bad[:5]]}"


def prec_of(cfg):
    return "f32" if cfg.dtype == 0 else "bf16"


def sample_tokens(T, n):
    if T <= n:
        return np.arange(T)
    s = np.unique(np.linspace(0, T - 1, n).round().astype(np.int64))
    return s


def oracle_sampled_forward(cfg, inp, tokens, idx, w, combined=False):
    """Oracle rows for sampled tokens: per (t, j) the expert output
    y_e(x[t]) (rounded as the layer materialises it), the shared expert's
    output and the combined y[t].  Experts are evaluated one at a time, each
    on just the sampled rows routed to it.  combined: the expert outputs are
    those of the FFN with the combine in FC2's epilogue, never materialised
    and so not rounded (the oracle's grouped_ffn_combine, row by row)."""
    prec = prec_of(cfg)
    x = np64(inp["x"][torch.as_tensor(tokens, device=inp["x"].device)])
    idx_s = np.asarray(idx)[tokens]
    w_s = np.asarray(w)[tokens]
    y_rows = np.zeros((len(tokens), cfg.k, cfg.d))
    gu_rows = np.zeros((len(tokens), cfg.k, 2 * cfg.F))
    for e in np.unique(idx_s):
        sel = np.argwhere(idx_s == e)
        r = O.swiglu_ffn(x[sel[:, 0]], np64(inp["w_gate"][int(e)]),
                         np64(inp["w_up"][int(e)]), np64(inp["w_down"][int(e)]), prec)
        y_rows[sel[:, 0], sel[:, 1]] = (r["h"] @ np64(inp["w_down"][int(e)]).T
                                        if combined else r["y"])
        rnd = O.rounder(prec)
        gu_rows[sel[:, 0], sel[:, 1], :cfg.F] = rnd(r["g"])
        gu_rows[sel[:, 0], sel[:, 1], cfg.F:] = rnd(r["u"])
    ys = None
    if cfg.F_shared > 0:
        if combined:
            hs = O.swiglu_ffn(x, np64(inp["ws_gate"]), np64(inp["ws_up"]),
                              np64(inp["ws_down"]), prec)["h"]
            ys = hs @ np64(inp["ws_down"]).T
        else:
            ys = O.shared_ffn(x, np64(inp["ws_gate"]), np64(inp["ws_up"]),
                              np64(inp["ws_down"]), prec)
    acc = np.zeros((len(tokens), cfg.d)) if ys is None else ys.copy()
    for j in range(cfg.k):
        acc += w_s[:, j:j + 1] * y_rows[:, j]
    y = O.out_f32(prec)(acc)
    return dict(y_rows=y_rows, gu_rows=gu_rows, ys=ys, y=y)


def logit_tolerance(d, logits):
    """A bound on |fp32-accumulated - exact| router scores: 100 * u * sqrt(d)
    * rms(l), u = 2^-24 (a random-walk estimate of fp32 summation error with
    a wide margin), plus one fp32 rounding of the largest score."""
    l = np64(logits)
    rms = float(np.sqrt((l ** 2).mean())) if l.size else 0.0
    return 100 * 2.0 ** -24 * np.sqrt(d) * rms + 2.0 ** -23 * float(np.abs(l).max(initial=0.0))


def routing_keys(cfg, logits, score_bias):
    """The oracle's selection keys and group scores (for ambiguity checks)."""
    l = np64(logits)
    if cfg.score == O.SCORE_SOFTMAX:
        return l, None
    s = O.sigmoid_scores(l)
    key = s if score_bias is None else O.round_f32(s + np64(score_bias)[None, :])
    G = cfg.E // cfg.n_groups
    srt = -np.sort(-key.reshape(key.shape[0], cfg.n_groups, G), axis=2)
    gs = srt[:, :, 0] + (srt[:, :, 1] if G >= 2 else 0.0)
    return key, gs


def key_tolerance(cfg, tol):
    """How far a selection key can move when the router scores move by tol:
    softmax keys are the scores themselves; a sigmoid score moves by at most
    tol / 4 (the slope of the sigmoid) plus its fp32 rounding (half an ulp
    below 1, on each side), and the biased key s + bias by one more fp32
    rounding (an ulp below 2)."""
    if cfg.score == O.SCORE_SOFTMAX:
        return tol
    return tol / 4 + 2.0 ** -24 + 2.0 ** -23


def ambiguous_tokens(cfg, logits, score_bias, tol, idx):
    """Tokens whose routing could change if the scores moved by tol, judged
    on the oracle's own selection idx: two consecutive picks, or the last
    pick and the best unpicked candidate of the kept groups, are closer than
    the bound (or, with a group limit, the kept and dropped groups are).
    Decided by the oracle alone."""
    key, gs = routing_keys(cfg, logits, score_bias)
    ktol = key_tolerance(cfg, tol)
    T, E = key.shape
    idx = np.asarray(idx, dtype=np.int64)
    sel = np.take_along_axis(key, idx, axis=1)
    amb = (sel[:, :-1] - sel[:, 1:] < 2 * ktol).any(axis=1) if cfg.k > 1 else np.zeros(T, bool)
    allowed = np.ones((T, E), dtype=bool)
    if gs is not None and cfg.topk_groups < cfg.n_groups:
        g = -np.sort(-gs, axis=1)
        amb |= g[:, cfg.topk_groups - 1] - g[:, cfg.topk_groups] < 4 * ktol
        G = E // cfg.n_groups
        kept = np.zeros((T, cfg.n_groups), dtype=bool)
        np.put_along_axis(kept, idx // G, True, axis=1)
        allowed = np.repeat(kept, G, axis=1)
    rest = np.where(allowed, key, -np.inf)
    np.put_along_axis(rest, idx, -np.inf, axis=1)
    best_rest = rest.max(axis=1)
    amb |= sel[:, -1] - best_rest < 2 * ktol
    return amb


def check_maps_valid(out, idx, w, E, x=None):
    """Properties every correct permutation of the routing (idx, w) has,
    checked on GPU outputs whether or not that routing equals the oracle's:
    offsets are the prefix sums of the expert counts; row_token and
    token_row are inverse maps; slot (t, j) lands inside the segment of
    expert idx[t, j]; rows of a segment are in ascending token order; the
    row's gate is the slot's gate bit for bit; x_perm rows are x's rows."""
    idx = np.asarray(idx, dtype=np.int64)
    w = np.asarray(w, dtype=np.float32)
    T, k = idx.shape
    offs = out["expert_offsets"].cpu().numpy().astype(np.int64)
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert np.array_equal(offs, np.concatenate([[0], np.cumsum(counts)])), "offsets"
    rt = out["row_token"].cpu().numpy().astype(np.int64)
    tr = out["token_row"].cpu().numpy().astype(np.int64)
    rg = out["row_gate"].cpu().numpy()
    R = T * k
    assert np.all((tr >= 0) & (tr < R)), "token_row out of range"
    assert np.array_equal(rt[tr.reshape(-1)], np.repeat(np.arange(T), k)), "row_token o token_row"
    assert np.array_equal(np.sort(tr.reshape(-1)), np.arange(R)), "token_row is not a bijection"
    assert np.all((offs[idx] <= tr) & (tr < offs[idx + 1])), "slot outside its expert's segment"
    assert np.array_equal(rg[tr].view(np.uint32), w.view(np.uint32)), "row_gate != topk_w"
    for e in range(E):
        seg = rt[offs[e]:offs[e + 1]]
        assert np.all(np.diff(seg) > 0), f"expert {e}: rows not in ascending token order"
    if x is not None and out.get("x_perm") is not None and R > 0:
        import torch as _t
        rows = _t.as_tensor(rt, device=out["x_perm"].device)
        assert _t.equal(out["x_perm"], x[rows]), "x_perm rows are not x's rows"


def check_routing_valid(cfg, key, gs, ktol, ref_idx, gidx, gw):
    """Validity of a GPU selection gidx [T, k] (gates gw) on every token,
    judged by the oracle's own keys (key [T, E], group scores gs or None)
    within the score bound ktol: k distinct experts; with a group limit, at
    most topk_groups groups, each scoring within the bound of the oracle's
    last kept group; inside the groups of its picks, no unpicked expert
    beats the weakest pick by more than the bound, and (without a group
    limit) no pick falls below the oracle's k-th key by more than the bound;
    picks listed in descending key order up to the bound; renormalised gates
    positive and summing to 1 within fp32 rounding."""
    T, E = key.shape
    k = cfg.k
    gidx = np.asarray(gidx, dtype=np.int64)
    assert gidx.shape == (T, k)
    assert np.all((gidx >= 0) & (gidx < E)), "expert index out of range"
    srt = np.sort(gidx, axis=1)
    assert np.all(np.diff(srt, axis=1) > 0) if k > 1 else True, "repeated expert in a token"
    sel = np.take_along_axis(key, gidx, axis=1)
    if k > 1:
        assert np.all(sel[:, :-1] >= sel[:, 1:] - 2 * ktol), "picks not in descending key order"
    allowed = np.ones((T, E), dtype=bool)
    limited = gs is not None and cfg.topk_groups < cfg.n_groups
    if limited:
        G = E // cfg.n_groups
        grp = gidx // G
        kept = np.zeros((T, cfg.n_groups), dtype=bool)
        np.put_along_axis(kept, grp, True, axis=1)
        assert np.all(kept.sum(axis=1) <= cfg.topk_groups), "picks span too many groups"
        g_sorted = -np.sort(-gs, axis=1)
        last_kept = g_sorted[:, cfg.topk_groups - 1]
        gsel = np.take_along_axis(gs, grp, axis=1)
        assert np.all(gsel >= last_kept[:, None] - 4 * ktol), "a pick's group is not among the best"
        allowed = np.repeat(kept, G, axis=1)
    else:
        ref_kth = np.take_along_axis(key, np.asarray(ref_idx, dtype=np.int64)[:, -1:], axis=1)[:, 0]
        assert np.all(sel.min(axis=1) >= ref_kth - 2 * ktol), "a pick lies below the k-th key"
    rest = np.where(allowed, key, -np.inf)
    np.put_along_axis(rest, gidx, -np.inf, axis=1)
    assert np.all(rest.max(axis=1) <= sel.min(axis=1) + 2 * ktol), "an unpicked expert beats a pick"
    gw = np.asarray(gw, dtype=np.float64)
    assert np.all(gw > 0), "non-positive gate"
    if cfg.renorm:
        assert np.all(np.abs(gw.sum(axis=1) - 1.0) <= 2.0 ** -22 * k), "gates do not sum to 1"


def route_and_check(cfg, inp, out, max_ambiguous_frac=0.05):
    """The oracle routes from its own fp64 router scores; the GPU's routing
    is then checked against it.

    The GPU's fp32 scores differ from the exact ones by at most
    err = max |l_gpu - l_oracle|, which must lie within the a-priori bound
    logit_tolerance.  A token is ambiguous when the oracle's own keys leave a
    gap of less than 2 err (plus an fp32 rounding) somewhere in its
    selection: only there may a correct fp32 selection differ.  Unambiguous
    tokens must match the oracle bit for bit (indices) and to fp32 rounding
    (gates); every token, ambiguous or not, must hold a valid selection
    (check_routing_valid).  Returns (idx, w, ambiguous, same)."""
    ref_l = O.router_logits(inp["x"], inp["w_router"], inp.get("router_bias"), "f32")
    assert_close("logits", out["logits"], ref_l, "f32")
    gl = np64(out["logits"])
    err = float(np.abs(gl - ref_l).max()) if ref_l.size else 0.0
    bound = logit_tolerance(cfg.d, ref_l)
    assert err <= bound, f"router scores off by {err:.3e} > bound {bound:.3e}"
    tol = err + 2.0 ** -24 * float(np.abs(ref_l).max(initial=0.0))
    sb = inp.get("score_bias")
    sb = None if sb is None else np64(sb)
    idx, w = O.route(ref_l, cfg.k, cfg.score, cfg.renorm, cfg.n_groups, cfg.topk_groups,
                     sb, prec_of(cfg))
    amb = ambiguous_tokens(cfg, ref_l, sb, tol, idx)
    gidx = out["topk_idx"].cpu().numpy()
    gw = out["topk_w"].cpu().numpy()
    ok = ~amb
    assert_equal_int("topk_idx[unambiguous]", gidx[ok], idx[ok])
    assert_close("topk_w[unambiguous]", gw[ok], w[ok], "f32")
    key, gs = routing_keys(cfg, ref_l, sb)
    ktol = key_tolerance(cfg, tol)
    check_routing_valid(cfg, key, gs, ktol, idx, gidx, gw)
    same = bool(np.array_equal(gidx, idx))
    n_amb = int(amb.sum())
    print(f"  router score error {err:.2e} (bound {bound:.2e}); ambiguous tokens {n_amb} of "
          f"{cfg.T}; GPU routing differs on {int((gidx != idx).any(axis=1).sum())}; "
          f"identical: {same}", flush=True)
    assert n_amb <= max_ambiguous_frac * max(cfg.T, 1) + 2, \
        f"{n_amb} ambiguous tokens: the check would cover too little"
    return idx, w, amb, same


def oracle_sampled_backward(cfg, inp, p, idx, w, logits, toks, experts):
    """Oracle gradients for sampled tokens (dx, d_gate, d_logits) and whole
    experts (dW), each expert evaluated on just the rows needed.  Every
    routed row r of token t, slot j: x_perm[r] = x[t], g | u from the
    oracle's FC1 on x[t], dY_perm[r] = w[t, j] dy[t] (dispatch_grad)."""
    prec = prec_of(cfg)
    rnd = O.rounder(prec)
    wg, wu, wd = inp["w_gate"], inp["w_up"], inp["w_down"]
    tr, rt = p["token_row"], p["row_token"]

    def rows_of(tokens, slots, e):
        """x, saved g | u, y_perm and dY_perm of the routed rows (t, j)."""
        x = np64(inp["x"][torch.as_tensor(tokens, device="cuda")])
        f = O.swiglu_ffn(x, np64(wg[e]), np64(wu[e]), np64(wd[e]), prec)
        gu = np.concatenate([rnd(f["g"]), rnd(f["u"])], axis=1)
        dy = np64(inp["dy"][torch.as_tensor(tokens, device="cuda")])
        n = len(tokens)
        dY = O.dispatch_grad(dy, np.arange(n)[:, None], w[tokens, slots][:, None], n, prec)
        return x, gu, f["y"], dY, dy

    T, k = len(toks), cfg.k
    dX = np.zeros((T, k, cfg.d))
    yp = np.zeros((T, k, cfg.d))
    for e in np.unique(idx[toks]):
        ti, sj = np.nonzero(idx[toks] == e)
        x, gu, y, dY, _ = rows_of(toks[ti], sj, int(e))
        r = O.expert_backward(dY, x, gu, np64(wg[int(e)]), np64(wu[int(e)]),
                              np64(wd[int(e)]), prec)
        dX[ti, sj] = r["dX"]
        yp[ti, sj] = y
    dy_s = np64(inp["dy"][torch.as_tensor(toks, device="cuda")])
    d_gate = O.gate_grad(dy_s, yp.reshape(T * k, cfg.d), np.arange(T * k).reshape(T, k))
    d_logits = O.router_backward(d_gate, idx[toks], w[toks], logits[toks], cfg.E,
                                 cfg.score, cfg.renorm, prec)
    of32 = O.out_f32(prec)
    out = dict(dx=of32(dX.sum(axis=1)), d_gate=of32(d_gate), d_logits=d_logits, dw={})
    for e in experts:
        a, b = int(p["offsets"][e]), int(p["offsets"][e + 1])
        tokens = rt[a:b].astype(np.int64)
        slots = np.argmax(tr[tokens] == np.arange(a, b)[:, None], axis=1)
        if b == a:
            out["dw"][e] = None
            continue
        x, gu, _, dY, _ = rows_of(tokens, slots, e)
        r = O.expert_backward(dY, x, gu, np64(wg[e]), np64(wu[e]), np64(wd[e]), prec)
        out["dw"][e] = {key: of32(r[key]) for key in ("dw_gate", "dw_up", "dw_down")}
    return out
