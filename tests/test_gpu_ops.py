"""GPU parity of each C-ABI entry point against the CPU oracle, on seeded
synthetic inputs that both sides receive (nothing the GPU computes is fed to
the oracle).  Integer outputs must match bit for bit; float outputs within
the tolerance of the storage type."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import (CONFIGS, MoEConfig, SCORE_SIGMOID, child_seed, expert_weight,
                        make_inputs, normal, random_gates, random_logits, random_topk)
from parity_util import assert_close, assert_equal_int, np64, prec_of, sample_tokens

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _lib():
    import mixture_experts_layer_logits_amd as M
    return M


def _ws(M, shape, op):
    n = M.moe_workspace_size(shape, op)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda"), n


# --------------------------------------------------------------------------
# moe_route_topk with the scores given as input: bit-exact selection
# --------------------------------------------------------------------------
ROUTE_CASES = [
    # name, cfg overrides, logits std, tie quantum
    ("softmax_top2_of_8", dict(T=1000, E=8, k=2), 1.0, 0.0),
    ("softmax_near_uniform", dict(T=4096, E=8, k=2), 0.064, 0.0),
    ("softmax_ties", dict(T=2000, E=16, k=4), 1.0, 0.25),
    ("softmax_full_probs", dict(T=700, E=40, k=5, renorm=0), 1.0, 0.0),
    ("softmax_top8_of_128", dict(T=3000, E=128, k=8), 1.0, 0.0),
    ("softmax_k_equals_E", dict(T=300, E=6, k=6), 1.0, 0.5),
    ("softmax_top8_of_512", dict(T=500, E=512, k=8), 1.0, 0.0),
    ("softmax_k64_of_1024", dict(T=64, E=1024, k=64), 1.0, 0.0),
    ("sigmoid_groups_256", dict(T=3000, E=256, k=8, n_groups=8, topk_groups=4,
                                score=SCORE_SIGMOID, score_bias_std=0.1), 1.7, 0.0),
    ("sigmoid_groups_ties", dict(T=1000, E=64, k=6, n_groups=8, topk_groups=3,
                                 score=SCORE_SIGMOID, score_bias_std=0.1), 1.0, 0.5),
    ("sigmoid_single_group_norenorm", dict(T=500, E=32, k=4, score=SCORE_SIGMOID,
                                           renorm=0), 1.0, 0.0),
]


@pytest.mark.parametrize("name,over,std,quantum", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_route_topk_from_given_scores(name, over, std, quantum):
    _log(f"[route] {name}")
    M = _lib()
    cfg = MoEConfig(name, d=64, F=64, **over)
    logits = random_logits(cfg.T, cfg.E, seed=len(name), std=std, quantum=quantum)
    sb = None
    if cfg.score_bias_std > 0:
        sb = normal((cfg.E,), cfg.score_bias_std, torch.float32, "cpu",
                    child_seed(7, "score_bias"))
        if quantum > 0:
            sb = torch.round(sb / quantum) * quantum
    ref_idx, ref_w = O.route(logits, cfg.k, cfg.score, cfg.renorm, cfg.n_groups,
                             cfg.topk_groups, sb, "f32")
    lg = logits.cuda()
    sbg = None if sb is None else sb.cuda()
    idx = torch.empty(cfg.T, cfg.k, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, cfg.k, dtype=torch.float32, device="cuda")
    M.moe_route_topk(M.make_shape(cfg), None, None, None, lg, sbg, idx, w)
    torch.cuda.synchronize()
    assert_equal_int("topk_idx", idx, ref_idx)
    assert_close("topk_w", w, ref_w, "f32")
    assert torch.equal(lg.cpu(), logits)  # an input stays untouched


# bf16 with d % 64 == 0 runs the MFMA kernel, split in K when its tiles are
# few (64 x 64 tiles for E <= 128, 256 x 256 above); the rest runs the generic kernel
@pytest.mark.parametrize("dtype,d,E", [(0, 128, 8), (1, 4096, 8), (1, 7168, 256), (1, 200, 24),
                                       (0, 37, 5), (1, 2048, 128), (1, 512, 96)])
def test_router_logits_gemm(dtype, d, E):
    _log(f"[router gemm] dtype={dtype} d={d} E={E}")
    M = _lib()
    cfg = MoEConfig("router", T=700, d=d, E=E, k=2, F=64, dtype=dtype, zipf_s=1.2)
    inp = make_inputs(cfg, device="cuda", with_weights=False)
    prec = prec_of(cfg)
    logits = torch.empty(cfg.T, E, device="cuda")
    idx = torch.empty(cfg.T, 2, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, 2, device="cuda")
    shape = M.make_shape(cfg)
    ws, n = _ws(M, shape, 0)          # the split router GEMM's partial sums
    M.moe_route_topk(shape, inp["x"], inp["w_router"], inp["router_bias"],
                     logits, None, idx, w, ws, n)
    torch.cuda.synchronize()
    ref = O.router_logits(inp["x"], inp["w_router"], inp["router_bias"], "f32")
    # fp32 outputs of an fp32 (or exact bf16-product) accumulation
    assert_close("logits", logits, ref, "f32")


# --------------------------------------------------------------------------
# moe_permute on synthetic routing
# --------------------------------------------------------------------------
PERMUTE_CASES = [
    ("uniform_t4096_e8_k2", 4096, 8, 2, None, 1, 64),
    ("skewed_t3000_e128_k8", 3000, 128, 8, "zipf", 1, 256),
    ("ragged_t777_e13_k3", 777, 13, 3, None, 0, 36),
    ("all_experts_t300_e6_k6", 300, 6, 6, None, 1, 64),
    ("one_expert_t257_e1_k1", 257, 1, 1, None, 1, 16),
    ("one_token_t1_e64_k8", 1, 64, 8, None, 1, 128),
    ("many_experts_t600_e1024_k4", 600, 1024, 4, "zipf", 1, 24),
    ("odd_row_bytes_t100_e7_k2", 100, 7, 2, None, 1, 13),
    # 79 blocks of 256 tokens: the separate scan kernel (the maps kernel does
    # the scan itself only up to 64 blocks and 16384 block counts)
    ("scan_kernel_t20000_e16_k2", 20000, 16, 2, None, 1, 32),
    ("fused_scan_limit_t16384_e256_k4", 16384, 256, 4, "zipf", 1, 16),
]


@pytest.mark.parametrize("name,T,E,k,skew,dtype,d", PERMUTE_CASES, ids=[c[0] for c in PERMUTE_CASES])
def test_permute_maps_and_rows(name, T, E, k, skew, dtype, d):
    _log(f"[permute] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=64, dtype=dtype)
    wts = [1.0 / (r + 1) ** 1.2 for r in range(E)] if skew else None
    idx = random_topk(T, E, k, seed=T + E, weights=wts)
    gates = random_gates(T, k, seed=T)
    x = normal((T, d), 1.0, cfg.torch_dtype, "cpu", child_seed(3, "x"))
    ref = O.permute(None, idx.numpy(), gates.numpy(), E)
    R = T * k
    dev = lambda *s, dt=torch.int32: torch.empty(*s, dtype=dt, device="cuda")
    offs, rt, tr = dev(E + 1), dev(R), dev(T, k)
    rg = dev(R, dt=torch.float32)
    xp = dev(R, d, dt=cfg.torch_dtype)
    shape = M.make_shape(cfg)
    ws, n = _ws(M, shape, 1)
    M.moe_permute(shape, x.cuda(), idx.cuda(), gates.cuda(), offs, rt, tr, rg, xp, ws, n)
    torch.cuda.synchronize()
    assert_equal_int("expert_offsets", offs, ref["offsets"])
    assert_equal_int("row_token", rt, ref["row_token"])
    assert_equal_int("token_row", tr, ref["token_row"])
    assert np.array_equal(rg.cpu().numpy(), ref["row_gate"].astype(np.float32))
    assert torch.equal(xp.cpu(), x[torch.as_tensor(ref["row_token"]).long()])


def test_permute_no_tokens():
    M = _lib()
    cfg = MoEConfig("empty", T=0, d=64, E=8, k=2, F=64)
    shape = M.make_shape(cfg)
    offs = torch.full((9,), 7, dtype=torch.int32, device="cuda")
    e = torch.empty(0, device="cuda")
    ws, n = _ws(M, shape, 1)
    M.moe_permute(shape, e, e, e, offs, e, e, e, e, ws, n)
    torch.cuda.synchronize()
    assert offs.cpu().tolist() == [0] * 9


# --------------------------------------------------------------------------
# moe_grouped_ffn on synthetic expert-contiguous rows
# --------------------------------------------------------------------------
TAIL_COUNTS = (0, 1, 63, 64, 65, 127, 128, 129, 192, 255, 256, 257, 320, 384,
               511, 512, 600)

FFN_CASES = [
    # name, T, d, E, k, F, Fs, dtype, skew
    ("mfma_splitk_t300", 300, 256, 8, 2, 384, 0, 1, None),
    ("mfma_shared_t200", 200, 128, 64, 8, 128, 192, 1, None),
    ("mfma_skewed_empty_t600", 600, 192, 32, 4, 256, 0, 1, "zipf"),
    ("generic_bf16_t77", 77, 200, 6, 2, 96, 40, 1, None),
    ("fp32_t256", 256, 128, 8, 2, 256, 0, 0, None),
    ("fp32_odd_t37", 37, 20, 5, 3, 12, 8, 0, None),
    ("single_expert_t65", 65, 64, 1, 1, 64, 0, 1, None),
    # explicit rows per expert around every tile-height boundary (full
    # 256-row tiles, 128-row tail tiles, tails of <= 64 rows, empty experts);
    # N = 384 and d = 256 leave half of the wide tail tiles past N
    ("mfma_tail_classes_splitk", None, 256, None, 1, 384, 0, 1, TAIL_COUNTS),
    ("mfma_tail_classes_shared", None, 512, None, 1, 256, 128, 1, TAIL_COUNTS),
    # the largest expert count: the tile schedule's total sits at index 1024
    ("mfma_e1024_t300", 300, 256, 1024, 4, 256, 0, 1, None),
    ("generic_e1024_t300", 300, 96, 1024, 4, 64, 0, 1, None),
]


GATHER_CASES = [
    # name, T, d, E, k, F, Fs, dtype: FC1 reads x[row_token[r]] (x_perm NULL)
    ("mfma_gather_t500", 500, 256, 8, 4, 384, 0, 1),
    ("mfma_gather_shared_t300", 300, 128, 16, 2, 128, 64, 1),
    ("generic_gather_t77", 77, 200, 6, 2, 96, 40, 1),
    ("fp32_gather_t50", 50, 24, 5, 3, 16, 0, 0),
]


@pytest.mark.parametrize("case", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_grouped_ffn_gathered_rows(case):
    """The permutation fused into FC1's operand load: rows come from
    x[row_token[r]]; the result must equal the FFN of the gathered rows."""
    name, T, d, E, k, F, Fs, dtype = case
    _log(f"[ffn gather] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=F, F_shared=Fs, dtype=dtype)
    prec = prec_of(cfg)
    idx = random_topk(T, E, k, seed=T + 3)
    p = O.permute(None, idx.numpy(), np.ones((T, k)), E)
    inp = make_inputs(cfg, device="cuda")
    dt = cfg.torch_dtype
    yp = torch.empty(cfg.R, d, dtype=dt, device="cuda")
    ys = torch.empty(T, d, dtype=dt, device="cuda") if Fs else None
    shape = M.make_shape(cfg)
    ws, n = _ws(M, shape, 2)
    rt = torch.as_tensor(p["row_token"]).cuda()
    M.moe_grouped_ffn(shape, None, rt, torch.as_tensor(p["offsets"]).cuda(), inp["w_gate"],
                      inp["w_up"], inp["w_down"], inp["x"], inp["ws_gate"], inp["ws_up"],
                      inp["ws_down"], yp, ys, None, ws, n)
    torch.cuda.synchronize()
    xg = np64(inp["x"])[p["row_token"]]
    ref_y, _ = O.grouped_ffn(xg, p["offsets"], np64(inp["w_gate"]), np64(inp["w_up"]),
                             np64(inp["w_down"]), prec)
    assert_close("y_perm", yp, ref_y, prec)
    if Fs:
        assert_close("y_shared", ys, O.shared_ffn(inp["x"], inp["ws_gate"], inp["ws_up"],
                                                  inp["ws_down"], prec), prec)


def _ffn_inputs(cfg, skew):
    if isinstance(skew, tuple):
        p = {"offsets": np.concatenate([[0], np.cumsum(skew)]).astype(np.int32)}
        inp = make_inputs(cfg, device="cuda")
        xp = normal((cfg.R, cfg.d), 1.0, cfg.torch_dtype, "cuda", child_seed(5, "rows"))
        return p, inp, xp
    wts = [1.0 / (r + 1) ** 6 for r in range(cfg.E)] if skew else None
    idx = random_topk(cfg.T, cfg.E, cfg.k, seed=cfg.T, weights=wts)
    p = O.permute(None, idx.numpy(), np.ones((cfg.T, cfg.k)), cfg.E)
    inp = make_inputs(cfg, device="cuda")
    xp = normal((cfg.R, cfg.d), 1.0, cfg.torch_dtype, "cuda", child_seed(5, "rows"))
    return p, inp, xp


@pytest.mark.parametrize("case", FFN_CASES, ids=[c[0] for c in FFN_CASES])
def test_grouped_ffn(case):
    name, T, d, E, k, F, Fs, dtype, skew = case
    if isinstance(skew, tuple):
        T, E = int(sum(skew)), len(skew)
    _log(f"[ffn] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=F, F_shared=Fs, dtype=dtype)
    prec = prec_of(cfg)
    p, inp, xp = _ffn_inputs(cfg, skew)
    if skew:
        assert (np.diff(p["offsets"]) == 0).any()
    dt = cfg.torch_dtype
    yp = torch.empty(cfg.R, d, dtype=dt, device="cuda")
    ys = torch.empty(T, d, dtype=dt, device="cuda") if Fs else None
    # g | u of the routed rows [R, 2F], then of the shared expert [T, 2Fs]
    n_r = cfg.R * 2 * F
    gu_all = torch.empty(n_r + T * 2 * Fs, dtype=dt, device="cuda")
    gu = gu_all[:n_r].view(cfg.R, 2 * F)
    shape = M.make_shape(cfg)
    ws, n = _ws(M, shape, 2)
    M.moe_grouped_ffn(shape, xp, None, torch.as_tensor(p["offsets"]).cuda(), inp["w_gate"],
                      inp["w_up"], inp["w_down"], inp["x"] if Fs else None, inp["ws_gate"],
                      inp["ws_up"], inp["ws_down"], yp, ys, gu_all, ws, n)
    torch.cuda.synchronize()
    ref_y, ref_gu = O.grouped_ffn(xp, p["offsets"], np64(inp["w_gate"]), np64(inp["w_up"]),
                                  np64(inp["w_down"]), prec, save_gu=True)
    assert_close("y_perm", yp, ref_y, prec)
    assert_close("gu_save", gu, ref_gu, prec)
    if Fs:
        r = O.swiglu_ffn(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"], prec)
        assert_close("y_shared", ys, r["y"], prec)
        rnd = O.rounder(prec)
        assert_close("gu_shared", gu_all[n_r:].view(T, 2 * Fs),
                     np.concatenate([rnd(r["g"]), rnd(r["u"])], axis=1), prec)


# --------------------------------------------------------------------------
# moe_unpermute_combine on synthetic rows
# --------------------------------------------------------------------------
# The vector kernel gathers a token's rows in batches of 1, 2, 4 or 8 (the
# largest not above k): k = 1, 2, 4 fill their batches, k = 5 and 12 leave
# padding slots in a second batch, and the fp32 case takes the same path.
@pytest.mark.parametrize("T,d,E,k,shared,dtype", [(1000, 512, 8, 2, False, 1), (333, 96, 16, 4, True, 1),
                                                  (100, 20, 5, 3, True, 0), (50, 13, 4, 2, False, 1),
                                                  (120, 64, 4, 1, False, 1), (200, 64, 16, 5, True, 1),
                                                  (150, 256, 32, 12, False, 1), (90, 40, 8, 3, True, 0)])
def test_unpermute_combine(T, d, E, k, shared, dtype):
    _log(f"[combine] T={T} d={d} k={k} shared={shared}")
    M = _lib()
    cfg = MoEConfig("combine", T=T, d=d, E=E, k=k, F=64, F_shared=64 if shared else 0, dtype=dtype)
    idx = random_topk(T, E, k, seed=d)
    gates = random_gates(T, k, seed=d)
    p = O.permute(None, idx.numpy(), gates.numpy(), E)
    dt = cfg.torch_dtype
    yp = normal((cfg.R, d), 1.0, dt, "cuda", child_seed(9, "rows"))
    ys = normal((T, d), 1.0, dt, "cuda", child_seed(9, "x")) if shared else None
    y = torch.empty(T, d, device="cuda")
    M.moe_unpermute_combine(M.make_shape(cfg), yp, torch.as_tensor(p["token_row"]).cuda(),
                            gates.cuda(), ys, y)
    torch.cuda.synchronize()
    ref = O.combine(yp, p["token_row"], gates.numpy(), None if ys is None else ys, "f32")
    assert_close("y", y, ref, "f32")


# --------------------------------------------------------------------------
# moe_ffn_backward on synthetic saved tensors
# --------------------------------------------------------------------------
def _bwd_inputs(cfg, skew=None, dev="cuda"):
    """Saved forward tensors drawn directly (the backward is defined for any
    values of them): routing from synthetic scores, x_perm, g | u, y_perm
    and dy as seeded normals with the layer's typical scales."""
    dt = cfg.torch_dtype
    logits = random_logits(cfg.T, cfg.E, seed=cfg.T + 1)
    if skew:
        logits = logits + torch.tensor([-8.0 * np.log(r + 1) for r in range(cfg.E)],
                                       dtype=torch.float32)
    idx, w = O.route(logits, cfg.k, cfg.score, cfg.renorm, cfg.n_groups, cfg.topk_groups,
                     None, "f32")
    p = O.permute(None, idx, w, cfg.E)
    g = dict(logits=logits, idx=idx, w=w, p=p)
    g["x_perm"] = normal((cfg.R, cfg.d), 1.0, dt, dev, child_seed(11, "rows"))
    # one buffer: routed g | u [R, 2F], then the shared expert's [T, 2Fs]
    n = cfg.R * 2 * cfg.F
    g["gu_all"] = normal((n + cfg.T * 2 * cfg.F_shared,), 1.3, dt, dev, child_seed(12, "rows"))
    g["gu"] = g["gu_all"][:n].view(cfg.R, 2 * cfg.F)
    g["gu_s"] = g["gu_all"][n:].view(cfg.T, 2 * cfg.F_shared) if cfg.F_shared else None
    g["y_perm"] = normal((cfg.R, cfg.d), 0.1, dt, dev, child_seed(13, "rows"))
    g["dy"] = normal((cfg.T, cfg.d), 1.0, dt, dev, child_seed(14, "rows"))
    return g


def _run_bwd(M, cfg, inp, g):
    dev = "cuda"
    f32 = torch.float32
    wt = torch.bfloat16 if cfg.wgrad_dtype == 1 else f32
    out = dict(dx=torch.empty(cfg.T, cfg.d, device=dev),
               dw_gate=torch.empty(cfg.E, cfg.F, cfg.d, device=dev, dtype=wt),
               dw_up=torch.empty(cfg.E, cfg.F, cfg.d, device=dev, dtype=wt),
               dw_down=torch.empty(cfg.E, cfg.d, cfg.F, device=dev, dtype=wt),
               d_gate=torch.empty(cfg.T, cfg.k, device=dev),
               d_logits=torch.empty(cfg.T, cfg.E, device=dev))
    fs = cfg.F_shared
    if fs:
        out.update(dws_gate=torch.empty(fs, cfg.d, device=dev, dtype=wt),
                   dws_up=torch.empty(fs, cfg.d, device=dev, dtype=wt),
                   dws_down=torch.empty(cfg.d, fs, device=dev, dtype=wt))
    for v in out.values():
        v.fill_(float("nan"))
    shape = M.make_shape(cfg)
    ws, n = _ws(M, shape, 4)
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32)).cuda()
    M.moe_ffn_backward(shape, g["dy"], g["x_perm"], g["gu_all"], g["y_perm"],
                       i32(g["p"]["offsets"]), i32(g["p"]["row_token"]),
                       i32(g["p"]["token_row"]), i32(g["idx"]),
                       torch.as_tensor(g["w"], dtype=f32).cuda(), g["logits"].cuda(),
                       inp["w_gate"], inp["w_up"], inp["w_down"],
                       inp["x"] if fs else None, inp["ws_gate"], inp["ws_up"], inp["ws_down"],
                       out["dx"], out["dw_gate"], out["dw_up"], out["dw_down"],
                       out.get("dws_gate"), out.get("dws_up"), out.get("dws_down"),
                       out["d_gate"], out["d_logits"], ws, n)
    torch.cuda.synchronize()
    return out


BWD_CASES = [
    # name, T, d, E, k, F, dtype, score, renorm, skew[, F_shared]
    ("mfma_softmax_t300", 300, 256, 8, 2, 256, 1, 0, 1, False),
    # with a shared expert: direct-to-LDS, MFMA, generic bf16 and fp32 paths
    ("dma_shared_sigmoid_t300", 300, 256, 16, 4, 256, 1, 1, 1, False, 512),
    ("mfma_shared_t200", 200, 128, 8, 2, 128, 1, 0, 1, True, 128),
    ("generic_shared_t77", 77, 200, 6, 2, 96, 1, 0, 1, False, 40),
    ("fp32_shared_t64", 64, 32, 4, 2, 16, 0, 1, 1, False, 24),
    ("dma_skewed_tails_t500", 500, 256, 16, 4, 512, 1, 0, 1, True),
    ("dma_sigmoid_t333", 333, 512, 24, 3, 256, 1, 1, 1, False),
    ("mfma_skewed_empty_t400", 400, 128, 16, 4, 128, 1, 0, 1, True),
    ("mfma_sigmoid_t200", 200, 128, 32, 4, 128, 1, 1, 1, False),
    ("generic_bf16_t77", 77, 200, 6, 2, 96, 1, 0, 0, False),
    ("fp32_t128", 128, 64, 8, 2, 64, 0, 0, 1, False),
    ("fp32_odd_full_probs_t37", 37, 20, 5, 3, 12, 0, 0, 0, True),
    # weight gradients stored as bf16 (direct-to-LDS with a shared expert,
    # MFMA with empty experts, generic)
    ("dma_shared_wgrad_bf16_t300", 300, 256, 16, 4, 256, 1, 1, 1, False, 512, 1),
    ("mfma_skewed_wgrad_bf16_t400", 400, 128, 16, 4, 128, 1, 0, 1, True, 0, 1),
    ("generic_wgrad_bf16_t77", 77, 200, 6, 2, 96, 1, 0, 0, False, 40, 1),
    # k above one gather batch (the dispatch gradient and the dx gather take
    # a token's rows 8 at a time) and k = 5 (a batch of 4, then a padded one)
    ("dma_k12_t150", 150, 256, 32, 12, 256, 1, 0, 1, False),
    ("mfma_k5_t200", 200, 128, 16, 5, 128, 1, 0, 1, True),
    # 1024 experts (the largest count): direct-to-LDS and MFMA kernels
    ("dma_e1024_t300", 300, 256, 1024, 4, 256, 1, 0, 1, False),
    ("mfma_e1024_t300", 300, 128, 1024, 4, 128, 1, 0, 1, True),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_ffn_backward(case):
    name, T, d, E, k, F, dtype, score, renorm, skew = case[:10]
    Fs = case[10] if len(case) > 10 else 0
    wgrad = case[11] if len(case) > 11 else 0
    _log(f"[backward] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=F, F_shared=Fs, dtype=dtype, score=score,
                    renorm=renorm, backward=True, wgrad_dtype=wgrad)
    prec = prec_of(cfg)
    inp = make_inputs(cfg, device="cuda")
    g = _bwd_inputs(cfg, skew)
    out = _run_bwd(M, cfg, inp, g)
    shared = None
    if Fs:
        shared = dict(x=np64(inp["x"]), gu=np64(g["gu_s"]), ws_gate=np64(inp["ws_gate"]),
                      ws_up=np64(inp["ws_up"]), ws_down=np64(inp["ws_down"]))
    ref = O.ffn_backward(g["dy"], g["x_perm"], g["gu"], g["y_perm"], g["p"]["offsets"],
                         g["p"]["token_row"], g["idx"], g["w"], g["logits"], np64(inp["w_gate"]),
                         np64(inp["w_up"]), np64(inp["w_down"]), score, renorm, prec,
                         shared=shared)
    keys = ["d_gate", "d_logits", "dx", "dw_gate", "dw_up", "dw_down"]
    if Fs:
        keys += ["dws_gate", "dws_up", "dws_down"]
    for key in keys:
        assert_close(key, out[key], ref[key], "f32" if prec == "f32" else "bf16")
    counts = np.diff(g["p"]["offsets"])
    for e in np.nonzero(counts == 0)[0]:
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert torch.all(out[key][int(e)] == 0), (key, e)
    if skew:
        assert (counts == 0).any()


@pytest.mark.parametrize("name", ["qwen3_235b_train_t8192", "deepseek_v3_train_t8192"])
def test_ffn_backward_full_size_sampled(name):
    """A training workload's shape: sampled tokens for d_gate, d_logits and
    dx; three whole experts (first, middle, last) for the weight gradients;
    with a shared expert, its whole weight gradients too."""
    cfg = CONFIGS[name]
    _log(f"[backward full] {cfg.name}")
    M = _lib()
    inp = make_inputs(cfg, device="cuda")
    g = _bwd_inputs(cfg)
    out = _run_bwd(M, cfg, inp, g)
    p = g["p"]
    tr, rt = p["token_row"], p["row_token"]
    w = np.asarray(g["w"], dtype=np.float64)
    toks = sample_tokens(cfg.T, 64)
    dy = np64(g["dy"][torch.as_tensor(toks).cuda()])

    def dY_rows(rows):
        """dY_perm for permuted rows, from the oracle's dispatch gradient on
        just those rows (row i of the result is routed row rows[i])."""
        t = rt[rows]
        j = np.argmax(tr[t] == rows[:, None], axis=1)
        dyt = np64(g["dy"][torch.as_tensor(t).cuda()])
        n = len(rows)
        return O.dispatch_grad(dyt, np.arange(n)[:, None], w[t, j][:, None], n, "bf16")

    # d_gate and d_logits on sampled tokens
    rows = tr[toks]
    yp = np64(g["y_perm"][torch.as_tensor(rows.reshape(-1)).cuda()]).reshape(len(toks), cfg.k, cfg.d)
    d_gate = np.einsum("td,tjd->tj", dy, yp)
    assert_close("d_gate[sample]", out["d_gate"][torch.as_tensor(toks).cuda()], d_gate, "bf16")
    d_l = O.router_backward(d_gate, g["idx"][toks], g["w"][toks], g["logits"][toks], cfg.E,
                            cfg.score, cfg.renorm)
    assert_close("d_logits[sample]", out["d_logits"][torch.as_tensor(toks).cuda()], d_l, "bf16")
    # dx on sampled tokens: each row's dX depends on that row only
    flat = rows.reshape(-1)
    ex = np.searchsorted(p["offsets"], flat, side="right") - 1
    dX = np.zeros((len(flat), cfg.d))
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        rr = torch.as_tensor(flat[sel]).cuda()
        r = O.expert_backward(dY_rows(flat[sel]), g["x_perm"][rr], g["gu"][rr],
                              np64(inp["w_gate"][int(e)]), np64(inp["w_up"][int(e)]),
                              np64(inp["w_down"][int(e)]), "bf16")
        dX[sel] = r["dX"]
    dx = dX.reshape(len(toks), cfg.k, cfg.d).sum(axis=1)
    tt = torch.as_tensor(toks).cuda()
    if cfg.F_shared:
        rs = O.expert_backward(dy, np64(inp["x"][tt]), np64(g["gu_s"][tt]),
                               np64(inp["ws_gate"]), np64(inp["ws_up"]),
                               np64(inp["ws_down"]), "bf16")
        dx = dx + rs["dX"]
    assert_close("dx[sample]", out["dx"][tt], dx, "bf16")
    # weight gradients of whole experts
    for e in (0, cfg.E // 2, cfg.E - 1):
        a, b = int(p["offsets"][e]), int(p["offsets"][e + 1])
        rr = torch.arange(a, b, device="cuda")
        r = O.expert_backward(dY_rows(np.arange(a, b)), g["x_perm"][rr], g["gu"][rr],
                              np64(inp["w_gate"][e]), np64(inp["w_up"][e]),
                              np64(inp["w_down"][e]), "bf16")
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert_close(f"{key}[{e}]", out[key][e], r[key], "bf16")
    if cfg.F_shared:
        rs = O.expert_backward(np64(g["dy"]), np64(inp["x"]), np64(g["gu_s"]),
                               np64(inp["ws_gate"]), np64(inp["ws_up"]),
                               np64(inp["ws_down"]), "bf16")
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert_close(f"dws_{key[3:]}", out["dws_" + key[3:]], rs[key], "bf16")
