"""GPU parity of the MXFP8 entry points (moe_mx_quantize, moe_grouped_ffn_mxfp8)
against the oracle's MX functions, on seeded inputs both sides receive.

Quantisation decides integers (codes and scale bytes) from bf16 inputs that
are exact in fp32 and fp64 alike, so it must match bit for bit.  The grouped
FFN computes the same quantised model as the oracle (exact products of the
dequantised operands there, fp32 accumulation here); h = silu(g) * u is
quantised from fp32 on the GPU and from fp64 in the oracle, so a code may
differ by one step where the two straddle a rounding boundary, which the bf16
tolerance of the layer covers."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import CONFIGS, MoEConfig, SCORE_SIGMOID, make_inputs, random_topk
from parity_util import assert_close, assert_equal_int, np64, route_and_check, sample_tokens

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _lib():
    import mixture_experts_layer_logits_amd as M
    return M


def _decode(q):
    """E4M3 codes to values (torch's float8_e4m3fn is the OCP E4M3 format)."""
    return q.cpu().view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _quantize(M, src):
    rows, cols = src.shape
    q = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    s = torch.empty(rows, cols // 32, dtype=torch.uint8, device="cuda")
    M.moe_mx_quantize(src, rows, cols, q, s)
    return q, s


def _mx_matrix(rows, cols, seed):
    """bf16 [rows, cols]: per block of 32 a random decade in 1e-6 .. 1e6,
    plus blocks that are all zero, fp32-subnormal, huge, exact rounding ties,
    negative zeros, and values at E4M3's saturation edge."""
    g = torch.Generator().manual_seed(seed)
    nb = rows * cols // 32
    v = torch.randn(nb, 32, generator=g, dtype=torch.float64)
    v *= 10.0 ** (torch.rand(nb, 1, generator=g, dtype=torch.float64) * 12 - 6)
    special = [
        torch.zeros(32, dtype=torch.float64),
        torch.randn(32, generator=g, dtype=torch.float64) * 1e-39,
        torch.randn(32, generator=g, dtype=torch.float64) * 1e30,
        # amax 256 gives scale 1: 1.0625, 3.125, 19, 3 * 2^-10, 1.1875, 9.5
        # sit halfway between E4M3 neighbours
        torch.tensor([256.0, 1.0625, -1.0625, 3.125, -19.0, 0.0029296875, 1.1875, 9.5] * 4,
                     dtype=torch.float64),
        torch.tensor([-0.0] * 31 + [1.0], dtype=torch.float64),
        # amax 470 (scale 1): 470 and 464 saturate, 440 rounds up to 448,
        # 432 is the tie between 416 and 448
        torch.tensor([470.0, 464.0, 440.0, 432.0, -470.0, -432.0, 400.0, 7.0] * 4,
                     dtype=torch.float64),
    ]
    for i, blk in enumerate(special):
        if i < nb:
            v[(i * 7) % nb] = blk
    return v.view(rows, cols).to(torch.bfloat16)


QUANT_CASES = [(1, 32), (3, 64), (37, 96), (256, 7168), (1000, 2048), (0, 64)]


@pytest.mark.parametrize("rows,cols", QUANT_CASES)
def test_mx_quantize_bit_exact(rows, cols):
    _log(f"[mx quantize] {rows}x{cols}")
    M = _lib()
    src = _mx_matrix(rows, cols, seed=rows * 31 + cols)
    q, s = _quantize(M, src.cuda())
    torch.cuda.synchronize()
    ref_q, ref_s = O.mx_quantize(np64(src))
    got_q = _decode(q)
    assert np.array_equal(got_q, ref_q), np.argwhere(got_q != ref_q)[:5]
    got_s = s.cpu().numpy().astype(np.int64) - 127
    assert np.array_equal(got_s, ref_s.astype(np.int64)), np.argwhere(got_s != ref_s)[:5]
    # 0x7f and 0xff (NaN) are never written
    assert not ((q == 0x7F) | (q == 0xFF)).any()


MX_FFN_CASES = [
    # name, T, d, E, k, F, Fs, skew
    # d = 384: FC1 runs 6 K steps (4-step loop and a 2-step tail), FC2 has
    # a half-empty 256-column tile
    ("mx_t300_d384", 300, 384, 4, 2, 256, 0, False),
    ("mx_shared_t200", 200, 256, 8, 2, 128, 256, False),
    ("mx_skewed_empty_t500", 500, 512, 16, 4, 384, 0, True),
    ("mx_single_expert_t70", 70, 128, 1, 1, 128, 128, False),
    ("mx_no_tokens", 0, 256, 4, 2, 128, 128, False),
    # K >= 512 loads scales eight K steps at a time: FC1 K = 1024 is two
    # groups; FC2 K = 768 (and the shared expert's 640) ends in a group whose
    # 16-byte window is moved back to the row's end
    ("mx_scale_groups_t256", 256, 1024, 4, 2, 768, 0, False),
    ("mx_scale_groups_shared_t256", 256, 1024, 4, 2, 768, 640, False),
]


def _quantized_weights(M, inp, names):
    out = []
    for n in names:
        if n not in inp or inp[n] is None:
            out += [None, None]
            continue
        w = inp[n]
        out += list(_quantize(M, w.reshape(-1, w.shape[-1])))
    return out


@pytest.mark.parametrize("case", MX_FFN_CASES, ids=[c[0] for c in MX_FFN_CASES])
def test_grouped_ffn_mxfp8(case):
    name, T, d, E, k, F, Fs, skew = case
    _log(f"[mx ffn] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=F, F_shared=Fs, dtype=1)
    inp = make_inputs(cfg, device="cuda")
    wts = [1.0 / (r + 1) ** 6 for r in range(E)] if skew else None
    idx = random_topk(T, E, k, seed=T + 11, weights=wts)
    p = O.permute(None, idx.numpy(), np.ones((T, k)), E)
    if skew:
        assert (np.diff(p["offsets"]) == 0).any()
    xq, xs = _quantize(M, inp["x"])
    wq = _quantized_weights(M, inp, ("w_gate", "w_up", "w_down"))
    sq = _quantized_weights(M, inp, ("ws_gate", "ws_up", "ws_down")) if Fs else [None] * 6
    yp = torch.empty(cfg.R, d, dtype=torch.bfloat16, device="cuda")
    ys = torch.empty(T, d, dtype=torch.bfloat16, device="cuda") if Fs else None
    shape = M.make_shape(cfg)
    n = M.moe_workspace_size(shape, 5)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    M.moe_grouped_ffn_mxfp8(shape, xq, xs, torch.as_tensor(p["row_token"]).cuda(),
                            torch.as_tensor(p["offsets"]).cuda(), *wq, *sq, yp, ys, ws, n)
    torch.cuda.synchronize()
    if T == 0:
        return
    x = np64(inp["x"])
    ref = O.grouped_ffn_mxfp8(x[p["row_token"]], p["offsets"], np64(inp["w_gate"]),
                              np64(inp["w_up"]), np64(inp["w_down"]))
    assert_close("y_perm", yp, ref, "bf16")
    if Fs:
        ref_s = O.swiglu_ffn_mxfp8(x, np64(inp["ws_gate"]), np64(inp["ws_up"]),
                                   np64(inp["ws_down"]))["y"]
        assert_close("y_shared", ys, ref_s, "bf16")


# Rows per expert around every tile-height boundary (full 256-row tiles, the
# 128-row x 2BN tail tiles, tails of <= 64 rows, empty experts), routed rows
# drawn as a seeded permutation of the tokens.
TAIL_COUNTS = (0, 1, 63, 64, 65, 127, 128, 129, 192, 255, 256, 257, 320, 384,
               511, 512, 600)
MX_TAIL_CASES = [
    # d = 256, F = 384: per-step scale dwords; FC2's tail tiles (512 columns)
    # run half past N = 256
    ("mx_tail_classes_d256_f384", 256, 384),
    # d = 512, F = 768: grouped scales, FC2's last group window moved back
    ("mx_tail_classes_d512_f768", 512, 768),
]


@pytest.mark.parametrize("name,d,F", MX_TAIL_CASES)
def test_grouped_ffn_mxfp8_tail_classes(name, d, F):
    _log(f"[mx ffn tails] {name}")
    M = _lib()
    counts = np.array(TAIL_COUNTS)
    E, T = len(counts), int(counts.sum())
    cfg = MoEConfig(name, T=T, d=d, E=E, k=1, F=F, dtype=1)
    inp = make_inputs(cfg, device="cuda")
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_token = np.random.default_rng(5).permutation(T).astype(np.int32)
    xq, xs = _quantize(M, inp["x"])
    wq = _quantized_weights(M, inp, ("w_gate", "w_up", "w_down"))
    yp = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    shape = M.make_shape(cfg)
    n = M.moe_workspace_size(shape, 5)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
    M.moe_grouped_ffn_mxfp8(shape, xq, xs, torch.as_tensor(row_token).cuda(),
                            torch.as_tensor(offsets).cuda(), *wq, *([None] * 6), yp, None, ws, n)
    torch.cuda.synchronize()
    ref = O.grouped_ffn_mxfp8(np64(inp["x"])[row_token], offsets, np64(inp["w_gate"]),
                              np64(inp["w_up"]), np64(inp["w_down"]))
    assert_close("y_perm", yp, ref, "bf16")
    # rows of every expert checked on their own too (a wrong tail tile would
    # hide in the Frobenius norm of the whole output)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            assert_close(f"y_perm[expert {e}]", yp[a:b], ref[a:b], "bf16")


# --------------------------------------------------------------------------
# The layer's MXFP8 forward: route -> maps-only permute -> quantise x ->
# MXFP8 grouped FFN -> combine, against the oracle routing from its own
# fp64 scores and running the MX expert FFN on its own permutation.
# --------------------------------------------------------------------------
MX_LAYER = {
    "mx_softmax_t300": MoEConfig("mx_softmax_t300", T=300, d=256, E=8, k=2, F=384),
    "mx_sigmoid_groups_shared_t200": MoEConfig(
        "mx_sigmoid_groups_shared_t200", T=200, d=128, E=64, k=8, F=128, F_shared=256,
        n_groups=8, topk_groups=4, score=SCORE_SIGMOID, score_bias_std=0.1),
}


def _mx_layer(cfg):
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    layer.quantize_weights(inp)
    out = layer.forward_mxfp8(inp)
    torch.cuda.synchronize()
    return inp, layer, out


@pytest.mark.parametrize("name", list(MX_LAYER))
def test_layer_mxfp8_forward(name):
    cfg = MX_LAYER[name]
    _log(f"[mx layer] {name}")
    inp, layer, out = _mx_layer(cfg)
    idx, w, amb, same = route_and_check(cfg, inp, out)
    x = np64(inp["x"])
    p = O.permute(x, idx, w, cfg.E)
    ref_yp = O.grouped_ffn_mxfp8(p["x_perm"], p["offsets"], np64(inp["w_gate"]),
                                 np64(inp["w_up"]), np64(inp["w_down"]))
    ref_ys = None
    if cfg.F_shared:
        ref_ys = O.swiglu_ffn_mxfp8(x, np64(inp["ws_gate"]), np64(inp["ws_up"]),
                                    np64(inp["ws_down"]))["y"]
        assert_close("y_shared", out["y_shared"], ref_ys, "bf16")
    if same:
        assert_equal_int("expert_offsets", out["expert_offsets"], p["offsets"])
        assert_equal_int("row_token", out["row_token"], p["row_token"])
        assert_close("y_perm", out["y_perm"], ref_yp, "bf16")
    ref_y = O.combine(ref_yp, p["token_row"], w, ref_ys, "bf16")
    ok = ~amb | same
    assert_close("y", out["y"][torch.as_tensor(ok).cuda()], ref_y[ok], "bf16")


# sampled tokens per full-size shape: the oracle's cost is one weight
# quantisation per expert reached (about 3 s at the DeepSeek-V3 shape, 11 s
# at Mixtral's), so the 8-expert Mixtral shape takes many more tokens
MX_FULL_SAMPLE = {"deepseek_v3_t8192": 4, "mixtral_t4096": 32}


@pytest.mark.parametrize("name", ["deepseek_v3_t8192", "mixtral_t4096"])
def test_layer_mxfp8_full_size_sampled(name):
    """Full-size MXFP8 forward: sampled tokens (y_perm rows, y_shared, y), and
    every row of two whole experts (the heaviest and the median one by the
    oracle's counts; compared when the routing matches the oracle's bit for
    bit, so that the oracle's own permutation names the rows).  The oracle
    runs each expert it needs once, on just the rows needed."""
    cfg = CONFIGS[name]
    _log(f"[mx layer full] {name}")
    inp, layer, out = _mx_layer(cfg)
    idx, w, amb, same = route_and_check(cfg, inp, out)
    toks = np.array([t for t in sample_tokens(cfg.T, MX_FULL_SAMPLE[name]) if not amb[t]])
    p = O.permute(None, idx, w, cfg.E)
    counts = np.diff(p["offsets"])
    order = np.argsort(-counts, kind="stable")
    whole = [int(order[0]), int(order[np.count_nonzero(counts) // 2])] if same else []
    _log(f"  {len(toks)} sampled tokens; whole experts {whole} "
         f"({[int(counts[e]) for e in whole]} rows)")
    x_all = inp["x"]
    idx_s, w_s = np.asarray(idx)[toks], np.asarray(w)[toks]
    y_rows = np.zeros((len(toks), cfg.k, cfg.d))
    for e in sorted(set(np.unique(idx_s).tolist()) | set(whole)):
        sel = np.argwhere(idx_s == e)
        a, b = int(p["offsets"][e]), int(p["offsets"][e + 1])
        seg = p["row_token"][a:b] if e in whole else np.zeros(0, dtype=np.int64)
        rows_t = np.concatenate([toks[sel[:, 0]], seg]).astype(np.int64)
        xe = np64(x_all[torch.as_tensor(rows_t, device="cuda")])
        ye = O.swiglu_ffn_mxfp8(xe, np64(inp["w_gate"][e]), np64(inp["w_up"][e]),
                                np64(inp["w_down"][e]))["y"]
        y_rows[sel[:, 0], sel[:, 1]] = ye[:len(sel)]
        if e in whole:
            assert_close(f"y_perm[expert {e}]", out["y_perm"][a:b], ye[len(sel):], "bf16")
    tt = torch.as_tensor(toks, device="cuda")
    rows = out["token_row"][tt].reshape(-1).long()
    assert_close("y_perm[sample]", out["y_perm"][rows], y_rows.reshape(-1, cfg.d), "bf16")
    acc = np.zeros((len(toks), cfg.d))
    if cfg.F_shared:
        x = np64(x_all[tt])
        ys = O.swiglu_ffn_mxfp8(x, np64(inp["ws_gate"]), np64(inp["ws_up"]),
                                np64(inp["ws_down"]))["y"]
        assert_close("y_shared[sample]", out["y_shared"][tt], ys, "bf16")
        acc += ys
    for j in range(cfg.k):
        acc += w_s[:, j:j + 1] * y_rows[:, j]
    assert_close("y[sample]", out["y"][tt], acc, "bf16")
    del layer, out, inp
    torch.cuda.empty_cache()


# --------------------------------------------------------------------------
# The MXFP8 forward with the combine in FC2's epilogue
# (moe_grouped_ffn_mxfp8_combine), against grouped_ffn_mxfp8_combine.
# --------------------------------------------------------------------------
MX_COMBINE = dict(MX_LAYER)
MX_COMBINE["mx_skewed_empty_t520"] = MoEConfig("mx_skewed_empty_t520", T=520, d=384, E=32,
                                               k=2, F=256, zipf_s=1.2)


@pytest.mark.parametrize("name", list(MX_COMBINE))
def test_layer_mxfp8_combined(name):
    cfg = MX_COMBINE[name]
    _log(f"[mx combined] {name}")
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    layer.quantize_weights(inp)
    out = layer.forward_mxfp8_combined(inp)
    torch.cuda.synchronize()
    idx, w, amb, same = route_and_check(cfg, inp, out)
    x = np64(inp["x"])
    p = O.permute(x, idx, w, cfg.E)
    sh = None
    if cfg.F_shared:
        sh = (x, np64(inp["ws_gate"]), np64(inp["ws_up"]), np64(inp["ws_down"]))
    ref = O.grouped_ffn_mxfp8_combine(p["x_perm"], p["offsets"], p["token_row"], w,
                                      np64(inp["w_gate"]), np64(inp["w_up"]),
                                      np64(inp["w_down"]), sh)
    ok = ~amb
    assert_close("y", out["y"][torch.as_tensor(ok).cuda()], ref[ok], "bf16")
    if cfg.zipf_s > 0:
        assert (np.diff(p["offsets"]) == 0).any()
    # k = 2 without a shared expert: two addends per element, bitwise repeatable
    y1 = out["y"].clone()
    layer.ffn_mxfp8_combine(inp)
    torch.cuda.synchronize()
    if cfg.k <= 2 and not cfg.F_shared:
        assert torch.equal(out["y"], y1)
    else:
        assert_close("y (second run)", out["y"], y1, "f32")


def test_layer_mxfp8_combined_full_size_sampled():
    """Mixtral shape: sampled tokens, each expert they reach evaluated once by
    the oracle on just their rows, expert outputs kept exact."""
    cfg = CONFIGS["mixtral_t4096"]
    _log(f"[mx combined full] {cfg.name}")
    from mixture_experts_layer_logits_amd import MoELayer
    inp = make_inputs(cfg, device="cuda")
    layer = MoELayer(cfg)
    layer.quantize_weights(inp)
    out = layer.forward_mxfp8_combined(inp)
    torch.cuda.synchronize()
    idx, w, amb, same = route_and_check(cfg, inp, out)
    toks = np.array([t for t in sample_tokens(cfg.T, 32) if not amb[t]])
    x = np64(inp["x"][torch.as_tensor(toks, device="cuda")])
    idx_s, w_s = np.asarray(idx)[toks], np.asarray(w)[toks]
    acc = np.zeros((len(toks), cfg.d))
    for e in np.unique(idx_s):
        sel = np.argwhere(idx_s == e)
        h = O.swiglu_ffn_mxfp8(x[sel[:, 0]], np64(inp["w_gate"][int(e)]),
                               np64(inp["w_up"][int(e)]), np64(inp["w_down"][int(e)]))["h"]
        ye = h @ O.mx_round(np64(inp["w_down"][int(e)])).T
        for n, (t, j) in enumerate(sel):
            acc[t] += w_s[t, j] * ye[n]
    tt = torch.as_tensor(toks, device="cuda")
    assert_close("y[sample]", out["y"][tt], O.round_f32(acc), "bf16")
    del layer, out, inp
    torch.cuda.empty_cache()
