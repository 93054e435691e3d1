"""CPU oracle for one GPU's MoE layer: plain, slow, fp64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it; the only thing both sides share is the seeded input
module ``moe_inputs``, which holds none of the layer's arithmetic.

What it computes (the layer as described on the AMD blog "MoE Training
Optimization with Primus", MegaMoE section, layer dataflow of Figure 7): the
router gives every token a score per expert and keeps the k best; the tokens are
reordered so that each expert's rows sit together; per expert, FC1 (gate and up) feeds a SwiGLU and FC2
(down); a final unpermute-and-scale sums the k gate-weighted expert outputs back
onto each token.  The permuted buffer is padding-free (the padding-free token
buffer of the X-MoE verdict page on pith.science, key_machinery field): it
holds only routed rows plus token ids, expert ids, counts and combine weights.

Every floating-point step is evaluated in fp64.  A tensor that the layer
materialises at a stated precision is rounded there, once, with
round-to-nearest-even: ``prec`` is "bf16" (x_perm, h, y_perm, the saved g/u,
dY_perm, dg/du and dX_perm are bf16), "f32" (they are fp32) or "f64" (nothing
is rounded; used by the finite-difference pins).  Outputs that the layer
defines as fp32 (router logits, gates, y, dx, dW, d_gate, d_logits) are rounded
to fp32 in every mode but "f64".

Readings of the pages that these functions take (the pages leave them open):
  * softmax gates are renormalised over the k selected experts unless
    ``renorm`` is 0; the selection key is the raw fp32 logit (softmax is
    monotone, so the set is the same) and ties go to the lower expert index;
    the k entries are listed in descending key order;
  * sigmoid scoring: s = fp32(1/(1+exp(-l))) evaluated in fp64; the selection
    key is the single fp32 sum s + bias; groups are contiguous blocks of
    E/n_groups experts scored by the fp32 sum of their two largest keys; the
    topk_groups best groups are kept (ties to the lower group); gates are the
    unbiased s renormalised over the k picks (scaling factor 1);
  * rows inside an expert segment are in ascending token order;
  * the shared expert has gate 1 and its output is added first;
  * the backward recomputes h from the saved bf16 g and u;
  * with the combine folded into FC2 (grouped_ffn_combine) the expert
    outputs are never materialised, so they carry no rounding; h still does.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1


# --------------------------------------------------------------------------
# rounding
# --------------------------------------------------------------------------
def round_bf16(a):
    """Round fp64 values to the nearest bf16 value, ties to even.

    bf16 keeps 8 significant bits and fp32's exponent range: for
    2^(e-1) <= |a| < 2^e the spacing is 2^(e-8); below 2^-126 the spacing
    stays 2^-133 (subnormals).  Values are assumed finite and in range.
    """
    a = np.asarray(a, dtype=F64)
    _, e = np.frexp(a)
    e = np.maximum(e, -125)
    ulp = np.ldexp(1.0, e - 8)
    return np.rint(a / ulp) * ulp


def round_f32(a):
    """Round fp64 values to fp32 (round-to-nearest-even), kept as fp64."""
    return np.asarray(a, dtype=F64).astype(np.float32).astype(F64)


def rounder(prec):
    if prec == "bf16":
        return round_bf16
    if prec == "f32":
        return round_f32
    if prec == "f64":
        return lambda a: np.asarray(a, dtype=F64)
    raise ValueError(prec)


def out_f32(prec):
    """fp32 outputs are rounded to fp32 except in the fp64 variant."""
    return rounder("f64" if prec == "f64" else "f32")


def as64(a):
    if hasattr(a, "detach"):          # a torch tensor handed in by a test
        a = a.detach().cpu().float().numpy()
    return np.asarray(a, dtype=F64)


# --------------------------------------------------------------------------
# router
# --------------------------------------------------------------------------
def router_logits(x, w_router, router_bias=None, prec="f32"):
    """Router scores l[t,e] = x[t] . w_router[e] (+ bias[e]), fp64 sums.

    The router scores every token against every expert (Primus blog, MegaMoE
    section, first stage of Figure 7); the DeepSeek-V3 memory-model verdict
    page counts these logits as 4bsN bytes, i.e. fp32 [T, E].
    """
    l = as64(x) @ as64(w_router).T
    if router_bias is not None:
        l = l + as64(router_bias)[None, :]
    return out_f32(prec)(l)


def select_topk(keys, k, allowed=None):
    """k passes of 'take the largest remaining key, lower index on ties'.

    keys [T, N]; allowed [T, N] bool or None.  Returns [T, k] int64 in
    descending key order.  np.argmax returns the first maximum, which is the
    lowest index among equal keys.
    """
    keys = as64(keys)
    taken = np.zeros(keys.shape, dtype=bool)
    if allowed is not None:
        taken |= ~allowed
    out = np.empty((keys.shape[0], k), dtype=np.int64)
    rows = np.arange(keys.shape[0])
    for j in range(k):
        masked = np.where(taken, -np.inf, keys)
        best = np.argmax(masked, axis=1)
        out[:, j] = best
        taken[rows, best] = True
    return out


def route_softmax(logits, k, renorm=1, prec="f32"):
    """Top-k softmax gating.

    Selection on the raw logits; gates are the softmax over the k selected
    logits (renorm=1), else the full softmax probability of each pick.
    """
    l = as64(logits)
    idx = select_topk(l, k)
    sel = np.take_along_axis(l, idx, axis=1)
    if renorm:
        z = np.exp(sel - sel[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    else:
        m = l.max(axis=1, keepdims=True)
        den = np.exp(l - m).sum(axis=1, keepdims=True)
        w = np.exp(sel - m) / den
    return idx.astype(np.int32), out_f32(prec)(w)


def sigmoid_scores(logits, prec="f32"):
    """s = fp32(1 / (1 + exp(-l))), evaluated in fp64 and rounded once."""
    with np.errstate(over="ignore"):
        return out_f32(prec)(1.0 / (1.0 + np.exp(-as64(logits))))


def route_sigmoid_grouped(logits, k, n_groups, topk_groups, score_bias=None,
                          renorm=1, prec="f32"):
    """DeepSeek-V3-style routing: sigmoid scores, selection-only per-expert
    bias (the bias adjustment for load balancing that the Piper podcast page
    mentions), a group
    limit, top-k inside the kept groups, gates from the unbiased scores.

    The key s + bias and a group's top-2 sum are single fp32 additions
    (fp64 in the "f64" variant).
    """
    r32 = out_f32(prec)
    s = sigmoid_scores(logits, prec)
    T, E = s.shape
    key = s.copy() if score_bias is None else r32(s + as64(score_bias)[None, :])
    G = E // n_groups
    grp = key.reshape(T, n_groups, G)
    first = grp.max(axis=2)
    if G >= 2:
        at = np.argmax(grp, axis=2)
        rest = grp.copy()
        np.put_along_axis(rest, at[:, :, None], -np.inf, axis=2)
        gscore = r32(first + rest.max(axis=2))
    else:
        gscore = first
    keep = select_topk(gscore, topk_groups)
    gmask = np.zeros((T, n_groups), dtype=bool)
    np.put_along_axis(gmask, keep, True, axis=1)
    allowed = np.repeat(gmask, G, axis=1)
    idx = select_topk(key, k, allowed)
    ssel = np.take_along_axis(s, idx, axis=1)
    if renorm:
        w = ssel / ssel.sum(axis=1, keepdims=True)
    else:
        w = ssel
    return idx.astype(np.int32), r32(w)


def route(logits, k, score=SCORE_SOFTMAX, renorm=1, n_groups=1,
          topk_groups=1, score_bias=None, prec="f32"):
    if score == SCORE_SOFTMAX:
        return route_softmax(logits, k, renorm, prec)
    return route_sigmoid_grouped(logits, k, n_groups, topk_groups,
                                 score_bias, renorm, prec)


# --------------------------------------------------------------------------
# padding-free permutation
# --------------------------------------------------------------------------
def permute(x, topk_idx, topk_w, E):
    """Expert histogram, exclusive prefix sum, stable scatter.

    counts[e] = #{(t,j): idx[t,j] = e}; offsets = exclusive prefix sum;
    pos[t,j] = offsets[e] + #{t' < t : e in idx[t']}; row_token[pos] = t,
    token_row[t,j] = pos, row_gate[pos] = w[t,j], x_perm[pos] = x[t].
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    onehot = np.zeros((T, E), dtype=np.int64)
    for j in range(k):
        onehot[np.arange(T), idx[:, j]] += 1
    counts = onehot.sum(axis=0)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    before = np.cumsum(onehot, axis=0) - onehot   # #{t' < t : e in idx[t']}
    token_row = offsets[idx] + np.take_along_axis(before, idx, axis=1)
    R = T * k
    row_token = np.full(R, -1, dtype=np.int64)
    row_gate = np.zeros(R, dtype=F64)
    tt = np.repeat(np.arange(T), k)
    row_token[token_row.reshape(-1)] = tt
    row_gate[token_row.reshape(-1)] = as64(topk_w).reshape(-1)
    x_perm = None if x is None else as64(x)[row_token]
    return dict(counts=counts.astype(np.int32),
                offsets=offsets.astype(np.int32),
                row_token=row_token.astype(np.int32),
                token_row=token_row.astype(np.int32),
                row_gate=row_gate, x_perm=x_perm)


# --------------------------------------------------------------------------
# expert FFN (FC1 gate/up -> SwiGLU -> FC2 down)
# --------------------------------------------------------------------------
def silu(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_ffn(rows, wg, wu, wd, prec="bf16"):
    """One expert on its rows: g = rows.wg^T, u = rows.wu^T,
    h = silu(g)*u, y = h.wd^T (wg, wu [F, d]; wd [d, F]).

    The SwiGLU expert of the Primus blog (FC1 gate/up, SwiGLU, FC2 down) with
    the three matrices of the DeepSeek-V3 memory-model page (h x h_E twice,
    h_E x h).  h and y are materialised at ``prec``.
    """
    rnd = rounder(prec)
    rows = as64(rows)
    g = rows @ as64(wg).T
    u = rows @ as64(wu).T
    h = rnd(silu(g) * u)
    y = rnd(h @ as64(wd).T)
    return dict(g=g, u=u, h=h, y=y)


def grouped_ffn(x_perm, offsets, w_gate, w_up, w_down, prec="bf16",
                save_gu=False):
    """The grouped expert GEMM over ragged, expert-contiguous row ranges.

    Returns y_perm [R, d] (and gu_save [R, 2F] = rounded g | u when asked).
    Experts with no rows contribute nothing.
    """
    rnd = rounder(prec)
    x_perm = as64(x_perm)
    R, d = x_perm.shape
    E = len(offsets) - 1
    F = w_gate.shape[1]
    y_perm = np.zeros((R, d), dtype=F64)
    gu = np.zeros((R, 2 * F), dtype=F64) if save_gu else None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        r = swiglu_ffn(x_perm[a:b], w_gate[e], w_up[e], w_down[e], prec)
        y_perm[a:b] = r["y"]
        if save_gu:
            gu[a:b, :F] = rnd(r["g"])
            gu[a:b, F:] = rnd(r["u"])
    return y_perm, gu


def shared_ffn(x, ws_gate, ws_up, ws_down, prec="bf16"):
    """The shared expert, applied to every token (gate 1)."""
    return swiglu_ffn(x, ws_gate, ws_up, ws_down, prec)["y"]


# --------------------------------------------------------------------------
# MXFP8 (Primus blog, low-precision section: MXFP8 block scaling with E4M3
# elements, blocks of 32 and an E8M0 scale per block)
# --------------------------------------------------------------------------
E4M3_MAX = 448.0          # largest finite E4M3 value, 1.75 * 2^8
E4M3_EMAX = 8             # exponent of the largest power of two in E4M3
MX_BLOCK = 32


def e4m3_round(v):
    """Nearest E4M3 value (ties to even), saturating at +-448.

    E4M3: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; normal numbers
    from 2^-6, subnormals in steps of 2^-9.  A value's quantum is 2^(e-3)
    with e = max(floor(log2|v|), -6); rounding to that grid with ties to even
    is np.rint on v / quantum."""
    v = as64(v)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    q = np.exp2(e - 3.0)
    r = np.rint(a / q) * q
    return np.sign(v) * np.minimum(r, E4M3_MAX)


def mx_quantize(a, block=MX_BLOCK):
    """MX quantization along the last axis in blocks of `block` values.

    Per block the scale is 2^s with s = floor(log2(amax)) - 8 (the largest
    power of two of E4M3), amax the block's largest magnitude (s = -127, the
    smallest E8M0 scale, for an all-zero block); elements are
    e4m3_round(v / 2^s).  Returns (elements, s) with a ~ elements * 2^s."""
    a = as64(a)
    n = a.shape[-1]
    assert n % block == 0
    blk = a.reshape(*a.shape[:-1], n // block, block)
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        s = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, -127.0)
    s = np.clip(s, -127.0, 127.0)
    q = e4m3_round(blk / np.exp2(s)[..., None])
    return q.reshape(a.shape), s


def mx_dequantize(q, s, block=MX_BLOCK):
    q = as64(q)
    n = q.shape[-1]
    blk = q.reshape(*q.shape[:-1], n // block, block)
    return (blk * np.exp2(as64(s))[..., None]).reshape(q.shape)


def mx_round(a, block=MX_BLOCK):
    """a quantized to MXFP8 and back (the values an MXFP8 GEMM consumes)."""
    q, s = mx_quantize(a, block)
    return mx_dequantize(q, s, block)


def mx_round_rows(a, block=MX_BLOCK):
    """a [n, c] (one expert's rows) quantized to MXFP8 along its row axis:
    blocks of `block` consecutive rows starting at the expert's first row,
    the last block completed with zero rows (the Primus blog's low-precision
    section pads permuted tokens to the quantization block boundary when the
    contraction runs over tokens).  Zero rows change no block maximum and
    contribute nothing to a sum over rows; they are dropped again."""
    a = as64(a)
    n = a.shape[0]
    npad = -(-n // block) * block
    p = np.zeros((npad,) + a.shape[1:], dtype=F64)
    p[:n] = a
    return mx_round(p.T, block).T[:n]


def swiglu_ffn_mxfp8(rows, wg, wu, wd):
    """One expert with MXFP8 operands: the rows and the three weights are
    quantized along their contraction dimension (d for FC1, F for FC2), and
    h = silu(g) * u is quantized along F before FC2; products and sums are
    exact (fp64) on the dequantized values, y is rounded to bf16."""
    x = mx_round(rows)
    g = x @ mx_round(wg).T
    u = x @ mx_round(wu).T
    h = mx_round(silu(g) * u)
    return dict(g=g, u=u, h=h, y=round_bf16(h @ mx_round(wd).T))


def grouped_ffn_mxfp8(x_perm, offsets, w_gate, w_up, w_down):
    """grouped_ffn with MXFP8 operands (swiglu_ffn_mxfp8 per expert)."""
    x_perm = as64(x_perm)
    y = np.zeros((x_perm.shape[0], as64(w_down[0]).shape[0]), dtype=F64)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y[a:b] = swiglu_ffn_mxfp8(x_perm[a:b], w_gate[e], w_up[e], w_down[e])["y"]
    return y


def grouped_ffn_mxfp8_combine(x_perm, offsets, token_row, topk_w, w_gate, w_up,
                              w_down, shared=None):
    """The MXFP8 grouped FFN with the combine folded into FC2 (the Primus
    blog's MegaMoE section fuses the combine into the second grouped GEMM):
    per expert, hq as in swiglu_ffn_mxfp8, the expert output hq . mx(wd)^T
    kept exact (never materialised, so not rounded to bf16), then
    y[t] = ys[t] + sum_j w[t,j] * out[token_row[t,j]] rounded to fp32 once.
    ``shared`` is None or (x, ws_gate, ws_up, ws_down)."""
    x_perm = as64(x_perm)
    R = x_perm.shape[0]
    d = as64(w_down[0]).shape[0]
    out = np.zeros((R, d), dtype=F64)
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            h = swiglu_ffn_mxfp8(x_perm[a:b], w_gate[e], w_up[e], w_down[e])["h"]
            out[a:b] = h @ mx_round(as64(w_down[e])).T
    ys = None
    if shared is not None:
        xs, wsg, wsu, wsd = shared
        hs = swiglu_ffn_mxfp8(xs, wsg, wsu, wsd)["h"]
        ys = hs @ mx_round(as64(wsd)).T
    return combine(out, token_row, topk_w, ys, "f32")


# --------------------------------------------------------------------------
# unpermute-and-scale
# --------------------------------------------------------------------------
def combine(y_perm, token_row, topk_w, y_shared=None, prec="f32"):
    """y[t] = ys[t] + sum_j w[t,j] * y_perm[token_row[t,j]] (fp64 sum, fp32
    result): the final unpermute-and-scale of the Primus blog's MegaMoE
    section, which folds each token's k weighted expert outputs into its row."""
    y_perm = as64(y_perm)
    tr = np.asarray(token_row, dtype=np.int64)
    w = as64(topk_w)
    T, k = tr.shape
    acc = np.zeros((T, y_perm.shape[1]), dtype=F64)
    if y_shared is not None:
        acc += as64(y_shared)
    for j in range(k):
        acc += w[:, j:j + 1] * y_perm[tr[:, j]]
    return out_f32(prec)(acc)


def grouped_ffn_combine(x_perm, offsets, token_row, topk_w, w_gate, w_up,
                        w_down, shared=None, prec="bf16"):
    """The grouped FFN with the unpermute-and-scale folded into FC2 (the
    Primus blog's MegaMoE section fuses the combine into the second grouped
    GEMM): y[t] = ys[t] + sum_j w[t,j] * (h_r . wd[e]^T), r = token_row[t,j].

    h is materialised at ``prec`` as in the unfused layer; the expert outputs
    (and the shared expert's) are never materialised, so they are not
    rounded: they enter the fp64 sum exactly, and y is rounded to fp32 once.
    ``shared`` is None or (x, ws_gate, ws_up, ws_down).
    """
    x_perm = as64(x_perm)
    R, d = x_perm.shape
    E = len(offsets) - 1
    y_exp = np.zeros((R, d), dtype=F64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        h = swiglu_ffn(x_perm[a:b], w_gate[e], w_up[e], w_down[e], prec)["h"]
        y_exp[a:b] = h @ as64(w_down[e]).T
    ys = None
    if shared is not None:
        xs, wsg, wsu, wsd = shared
        hs = swiglu_ffn(xs, wsg, wsu, wsd, prec)["h"]
        ys = hs @ as64(wsd).T
    return combine(y_exp, token_row, topk_w, ys, prec)


# --------------------------------------------------------------------------
# backward
# --------------------------------------------------------------------------
def router_backward(d_gate, topk_idx, topk_w, logits, E, score=SCORE_SOFTMAX,
                    renorm=1, prec="f32"):
    """d_logits [T, E] from d_gate [T, k] through the gate function.

    Renormalised softmax over the picked set S: d_l[e_i] =
    w_i (dg_i - sum_j w_j dg_j).  Full softmax: d_l[b] = [b in S] p_b dg(b)
    - p_b sum_j dg_j p_{e_j}.  Sigmoid: d_s_i = (dg_i - sum_j w_j dg_j)/sum_S s
    (renormalised) or dg_i, then d_l_i = d_s_i s_i (1 - s_i).  The selection
    itself is piecewise constant and passes no gradient.
    """
    dg = as64(d_gate)
    idx = np.asarray(topk_idx, dtype=np.int64)
    w = as64(topk_w)
    l = as64(logits)
    T, k = idx.shape
    dl = np.zeros((T, E), dtype=F64)
    rows = np.arange(T)[:, None]
    if score == SCORE_SOFTMAX:
        if renorm:
            dot = (w * dg).sum(axis=1, keepdims=True)
            dl[rows, idx] = w * (dg - dot)
        else:
            m = l.max(axis=1, keepdims=True)
            p = np.exp(l - m)
            p /= p.sum(axis=1, keepdims=True)
            psel = np.take_along_axis(p, idx, axis=1)
            dot = (dg * psel).sum(axis=1, keepdims=True)
            dl = -p * dot
            dl[rows, idx] += psel * dg
    else:
        s = sigmoid_scores(l, prec)
        ssel = np.take_along_axis(s, idx, axis=1)
        if renorm:
            dot = (w * dg).sum(axis=1, keepdims=True)
            ds = (dg - dot) / ssel.sum(axis=1, keepdims=True)
        else:
            ds = dg
        dl[rows, idx] = ds * ssel * (1.0 - ssel)
    return out_f32(prec)(dl)


def expert_backward(dYe, xe, gu_e, wg, wu, wd, prec="bf16", mxfp8=False,
                    mx_wgrad=False):
    """One expert's backward on its rows (dYe [n, d], xe [n, d],
    gu_e [n, 2F]); wg, wu [F, d], wd [d, F].

    dh = dY . W_d; with s = sigmoid(g): dg = dh u s (1 + g (1 - s)),
    du = dh silu(g); h = silu(g) u recomputed from the saved g, u;
    dW_d = dY^T h, dW_g = dg^T x, dW_u = du^T x; dX = dg . W_g + du . W_u.

    mxfp8: the two data-gradient GEMMs take MXFP8 operands (the Primus
    blog's low-precision section runs the grouped expert GEMMs of forward
    and backward in MXFP8), each quantised along its contraction dimension:
    dY and W_d along d for dh; [dg | du] and [W_g; W_u] along F for dX
    (blocks never straddle g and u: F is a multiple of 32).  dh itself is
    not materialised (exact here); dg, du, h and dX are rounded as above.
    The weight gradients keep the unquantised operands unless mx_wgrad.

    mx_wgrad: the two weight-gradient GEMMs take MXFP8 operands too, each
    quantised along its contraction dimension, the expert's rows
    (mx_round_rows: 32-row blocks from the expert's first row, the last one
    padded with zero rows): dY and h for dW_down, [dg | du] and x for
    dW_gate | dW_up.  Their sums are exact on the dequantised values.
    """
    rnd = rounder(prec)
    gu_e = as64(gu_e)
    F = gu_e.shape[1] // 2
    g, u = gu_e[:, :F], gu_e[:, F:]
    dYe, xe = as64(dYe), as64(xe)
    if mxfp8:
        dh = mx_round(dYe) @ mx_round(as64(wd).T).T
    else:
        dh = dYe @ as64(wd)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    sg = g * sig
    dgt = rnd(dh * u * sig * (1.0 + g * (1.0 - sig)))
    dut = rnd(dh * sg)
    h = rnd(sg * u)
    if mxfp8:
        dgu = np.concatenate([dgt, dut], axis=1)
        wgu = np.concatenate([as64(wg), as64(wu)], axis=0)     # [2F, d]
        dX = rnd(mx_round(dgu) @ mx_round(wgu.T).T)
    else:
        dX = rnd(dgt @ as64(wg) + dut @ as64(wu))
    if mx_wgrad:
        xq = mx_round_rows(xe)
        return dict(dw_down=mx_round_rows(dYe).T @ mx_round_rows(h),
                    dw_gate=mx_round_rows(dgt).T @ xq, dw_up=mx_round_rows(dut).T @ xq,
                    dX=dX, dg=dgt, du=dut)
    return dict(dw_down=dYe.T @ h, dw_gate=dgt.T @ xe, dw_up=dut.T @ xe,
                dX=dX, dg=dgt, du=dut)


def dispatch_grad(dy, token_row, topk_w, R, prec="bf16"):
    """dY_perm[token_row[t,j]] = w[t,j] dy[t] (the dual of the combine)."""
    rnd = rounder(prec)
    dy = as64(dy)
    tr = np.asarray(token_row, dtype=np.int64)
    w = as64(topk_w)
    dY = np.zeros((R, dy.shape[1]), dtype=F64)
    for j in range(tr.shape[1]):
        dY[tr[:, j]] = rnd(w[:, j:j + 1] * dy)
    return dY


def gate_grad(dy, y_perm, token_row):
    """d_gate[t,j] = <dy[t], y_perm[token_row[t,j]]> (fp64 sum)."""
    dy = as64(dy)
    y_perm = as64(y_perm)
    tr = np.asarray(token_row, dtype=np.int64)
    return np.stack([(dy * y_perm[tr[:, j]]).sum(axis=1)
                     for j in range(tr.shape[1])], axis=1)


def ffn_backward(dy, x_perm, gu_save, y_perm, offsets, token_row, topk_idx,
                 topk_w, logits, w_gate, w_up, w_down, score=SCORE_SOFTMAX,
                 renorm=1, prec="bf16", shared=None, mxfp8=False, mx_wgrad=False):
    """Backward of the layer, from the saved tensors.

    The backward mirrors the forward through dispatch/combine duality, with
    the FC2 and FC1 data gradients and weight-gradient GEMMs over each expert's rows
    (Primus blog, MegaMoE section):
      dY_perm[pos] = w[t,j] dy[t];  d_gate[t,j] = <dy[t], y_perm[pos]>
      per expert: expert_backward;  dx[t] = sum_j dX_perm[pos[t,j]]
      d_logits from d_gate through the gate function.
    Weight gradients of experts with no rows are exactly zero.
    mxfp8: the data-gradient GEMMs on MXFP8 operands (expert_backward).
    mx_wgrad: the weight-gradient GEMMs on MXFP8 operands quantised along
    each expert's rows, padded per expert (expert_backward).

    ``shared`` (optional) = dict(x, gu, ws_gate, ws_up, ws_down) for the
    shared expert applied to every token: it adds ys[t] to y[t] with gate 1, so its
    backward is expert_backward on all T tokens with dY = dy; its data
    gradient is added to dx after the routed terms.
    """
    of32 = out_f32(prec)
    x_perm = as64(x_perm)
    gu = as64(gu_save)
    tr = np.asarray(token_row, dtype=np.int64)
    T, k = tr.shape
    R, d = x_perm.shape
    E = len(offsets) - 1
    F = gu.shape[1] // 2
    dY = dispatch_grad(dy, token_row, topk_w, R, prec)
    d_gate = gate_grad(dy, y_perm, token_row)
    dw_gate = np.zeros((E, F, d), dtype=F64)
    dw_up = np.zeros((E, F, d), dtype=F64)
    dw_down = np.zeros((E, d, F), dtype=F64)
    dX = np.zeros((R, d), dtype=F64)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        r = expert_backward(dY[a:b], x_perm[a:b], gu[a:b], w_gate[e],
                            w_up[e], w_down[e], prec, mxfp8, mx_wgrad)
        dw_down[e], dw_gate[e], dw_up[e] = r["dw_down"], r["dw_gate"], r["dw_up"]
        dX[a:b] = r["dX"]
    dx = np.zeros((T, d), dtype=F64)
    for j in range(k):
        dx += dX[tr[:, j]]
    out = {}
    if shared is not None:
        rs = expert_backward(dy, shared["x"], shared["gu"], shared["ws_gate"],
                             shared["ws_up"], shared["ws_down"], prec, mxfp8, mx_wgrad)
        dx = dx + rs["dX"]
        out = dict(dws_gate=of32(rs["dw_gate"]), dws_up=of32(rs["dw_up"]),
                   dws_down=of32(rs["dw_down"]), dX_shared=rs["dX"])
    d_logits = router_backward(d_gate, topk_idx, topk_w, logits,
                               as64(logits).shape[1], score, renorm, prec)
    return dict(dx=of32(dx), dw_gate=of32(dw_gate), dw_up=of32(dw_up),
                dw_down=of32(dw_down), d_gate=of32(d_gate),
                d_logits=d_logits, dY_perm=dY, dX_perm=dX, **out)


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------
def forward(inp, cfg, prec=None, logits=None, save_gu=False):
    """Route -> permute -> grouped SwiGLU -> combine for one workload.

    ``inp`` holds the tensors of moe_inputs.make_inputs; ``cfg`` a MoEConfig.
    When ``logits`` is given (e.g. the GPU's fp32 router scores), routing
    starts from them instead of the oracle's own.
    """
    if prec is None:
        prec = "f32" if cfg.dtype == 0 else "bf16"
    own_logits = router_logits(inp["x"], inp["w_router"],
                               inp.get("router_bias"), prec)
    l = own_logits if logits is None else as64(logits)
    idx, w = route(l, cfg.k, cfg.score, cfg.renorm, cfg.n_groups,
                   cfg.topk_groups, inp.get("score_bias"), prec)
    p = permute(inp["x"], idx, w, cfg.E)
    y_perm, gu = grouped_ffn(p["x_perm"], p["offsets"], inp["w_gate"],
                             inp["w_up"], inp["w_down"], prec, save_gu)
    ys = gu_s = None
    if cfg.F_shared > 0:
        r = swiglu_ffn(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], prec)
        ys = r["y"]
        if save_gu:
            rnd = rounder(prec)
            gu_s = np.concatenate([rnd(r["g"]), rnd(r["u"])], axis=1)
    y = combine(y_perm, p["token_row"], w, ys, prec)
    return dict(logits=own_logits, route_logits=l, topk_idx=idx, topk_w=w,
                y_perm=y_perm, gu_save=gu, y_shared=ys, gu_shared=gu_s, y=y, **p)
