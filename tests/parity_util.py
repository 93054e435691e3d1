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


def oracle_route_from(cfg, inp, logits_gpu):
    """The oracle's routing from the GPU's fp32 router scores."""
    return O.route(np64(logits_gpu), cfg.k, cfg.score, cfg.renorm,
                   cfg.n_groups, cfg.topk_groups,
                   None if inp.get("score_bias") is None else np64(inp["score_bias"]),
                   prec_of(cfg))


def sample_tokens(T, n):
    if T <= n:
        return np.arange(T)
    s = np.unique(np.linspace(0, T - 1, n).round().astype(np.int64))
    return s


def oracle_sampled_forward(cfg, inp, tokens, idx, w):
    """Oracle rows for sampled tokens: per (t, j) the expert output
    y_e(x[t]) (rounded as the layer materialises it), the shared expert's
    output and the combined y[t].  Experts are evaluated one at a time, each
    on just the sampled rows routed to it."""
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
        y_rows[sel[:, 0], sel[:, 1]] = r["y"]
        rnd = O.rounder(prec)
        gu_rows[sel[:, 0], sel[:, 1], :cfg.F] = rnd(r["g"])
        gu_rows[sel[:, 0], sel[:, 1], cfg.F:] = rnd(r["u"])
    ys = None
    if cfg.F_shared > 0:
        ys = O.shared_ffn(x, np64(inp["ws_gate"]), np64(inp["ws_up"]),
                          np64(inp["ws_down"]), prec)
    acc = np.zeros((len(tokens), cfg.d)) if ys is None else ys.copy()
    for j in range(cfg.k):
        acc += w_s[:, j:j + 1] * y_rows[:, j]
    y = O.out_f32(prec)(acc)
    return dict(y_rows=y_rows, gu_rows=gu_rows, ys=ys, y=y)
