"""GPU parity of the MXFP8 backward (moe_mx_quantize_t, moe_ffn_backward_mxfp8)
against the oracle's ffn_backward with mxfp8=True, on saved forward tensors
drawn directly (the backward is defined for any values of them).

The transposed quantisation decides codes and scale bytes from bf16 inputs
that are exact on both sides, so it must match bit for bit.  In the
backward, dg | du are rounded to bf16 from an fp32 dh on the GPU and from an
exact dh in the oracle, so a bf16 value, and then the E4M3 code it takes,
can differ by one step; the layer's bf16 tolerance covers this."""
import numpy as np
import pytest
import torch

import oracle as O
from moe_inputs import CONFIGS, MoEConfig, make_inputs
from parity_util import assert_close, np64, sample_tokens
from test_gpu_mxfp8 import _decode, _mx_matrix
from test_gpu_ops import _bwd_inputs

pytestmark = pytest.mark.gpu


def _log(msg):
    print(msg, flush=True)


def _lib():
    import mixture_experts_layer_logits_amd as M
    return M


QT_CASES = [
    # batches, rows, cols, ldq, column offset of the output rows
    (1, 32, 1, 32, 0),
    (3, 64, 100, 64, 0),        # a ragged 64-column block
    (2, 96, 128, 256, 128),     # written into the second half of wider rows
    (4, 256, 384, 256, 0),
]


@pytest.mark.parametrize("batches,rows,cols,ldq,off", QT_CASES)
def test_mx_quantize_t_bit_exact(batches, rows, cols, ldq, off):
    """Codes and scales of the transposed quantisation equal the oracle's
    mx_quantize of each matrix's transpose; the rest of the output rows is
    left untouched."""
    _log(f"[mx quantize_t] {batches}x{rows}x{cols} ldq {ldq} +{off}")
    M = _lib()
    # special blocks along the quantised axis: build them as rows of the transpose
    src = torch.stack([_mx_matrix(cols, rows, seed=97 * b + rows).t().contiguous()
                       for b in range(batches)]).cuda()
    q = torch.full((batches, cols, ldq), 0x55, dtype=torch.uint8, device="cuda")
    s = torch.full((batches, cols, ldq // 32), 0x55, dtype=torch.uint8, device="cuda")
    M.moe_mx_quantize_t(src, batches, rows, cols, ldq, q.view(-1)[off:], s.view(-1)[off // 32:])
    torch.cuda.synchronize()
    for b in range(batches):
        ref_q, ref_s = O.mx_quantize(np64(src[b]).T)
        got = q[b, :, off:off + rows]
        assert np.array_equal(_decode(got.contiguous()), ref_q)
        gs = s[b, :, off // 32:off // 32 + rows // 32].cpu().numpy().astype(np.int64) - 127
        assert np.array_equal(gs, ref_s.astype(np.int64))
    # bytes outside the written columns keep their fill
    mask = torch.ones(ldq, dtype=torch.bool)
    mask[off:off + rows] = False
    assert torch.all(q[:, :, mask.cuda()] == 0x55)


def mx_weights_t(M, cfg, inp):
    """Weights quantised for the backward's data gradients, as the layer
    builds them: w_down along d [E, F, d]; w_gate | w_up along F [E, d, 2F]."""
    u8 = torch.uint8

    def pair(E, d, F, wd, wg, wu):
        wd_q = torch.empty(E, F, d, dtype=u8, device="cuda")
        wd_s = torch.empty(E, F, d // 32, dtype=u8, device="cuda")
        M.moe_mx_quantize_t(wd, E, d, F, d, wd_q, wd_s)
        gu_q = torch.empty(E, d, 2 * F, dtype=u8, device="cuda")
        gu_s = torch.empty(E, d, 2 * F // 32, dtype=u8, device="cuda")
        M.moe_mx_quantize_t(wg, E, F, d, 2 * F, gu_q, gu_s)
        M.moe_mx_quantize_t(wu, E, F, d, 2 * F, gu_q.view(-1)[F:], gu_s.view(-1)[F // 32:])
        return [wd_q, wd_s, gu_q, gu_s]

    routed = pair(cfg.E, cfg.d, cfg.F, inp["w_down"], inp["w_gate"], inp["w_up"])
    shared = (pair(1, cfg.d, cfg.F_shared, inp["ws_down"], inp["ws_gate"], inp["ws_up"])
              if cfg.F_shared else [None] * 4)
    return routed, shared


def run_bwd_mx(M, cfg, inp, g):
    dev, f32 = "cuda", torch.float32
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
    from mixture_experts_layer_logits_amd import _lib as L
    n = M.moe_workspace_size(shape, L.MOE_OP_BACKWARD_MXFP8)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    routed, shared = mx_weights_t(M, cfg, inp)
    i32 = lambda a: torch.as_tensor(np.asarray(a, dtype=np.int32)).cuda()
    M.moe_ffn_backward_mxfp8(
        shape, g["dy"], g["x_perm"], g["gu_all"], g["y_perm"], i32(g["p"]["offsets"]),
        i32(g["p"]["row_token"]), i32(g["p"]["token_row"]), i32(g["idx"]),
        torch.as_tensor(g["w"], dtype=f32).cuda(), g["logits"].cuda(), *routed,
        inp["x"] if fs else None, *shared, out["dx"], out["dw_gate"], out["dw_up"],
        out["dw_down"], out.get("dws_gate"), out.get("dws_up"), out.get("dws_down"),
        out["d_gate"], out["d_logits"], ws, n)
    torch.cuda.synchronize()
    return out


MXB_CASES = [
    # name, T, d, E, k, F, score, renorm, skew, F_shared, wgrad_dtype
    ("mxb_softmax_t300", 300, 256, 8, 2, 256, 0, 1, False, 0, 0),
    # shared expert and sigmoid scores
    ("mxb_shared_sigmoid_t300", 300, 256, 16, 4, 256, 1, 1, False, 256, 0),
    # empty experts; dh's K = d = 128 takes the per-step scale loads
    ("mxb_skewed_empty_t400", 400, 128, 16, 4, 128, 0, 1, True, 0, 0),
    # d = F = 384: half-empty 256-column tiles in both GEMMs, MFMA-register
    # weight-gradient kernels, bf16 weight gradients
    ("mxb_d384_shared_wgrad_bf16_t500", 500, 384, 12, 4, 384, 0, 1, True, 128, 1),
    # K = 1024 for dh (two groups of eight scale steps); dX's K = 1536 and,
    # for the shared expert, 1280 (a last group moved back to the row's end)
    ("mxb_scale_groups_t256", 256, 1024, 4, 2, 768, 0, 1, False, 640, 0),
]


@pytest.mark.parametrize("case", MXB_CASES, ids=[c[0] for c in MXB_CASES])
def test_ffn_backward_mxfp8(case):
    name, T, d, E, k, F, score, renorm, skew, Fs, wgrad = case
    _log(f"[backward mxfp8] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=F, F_shared=Fs, score=score,
                    renorm=renorm, backward=True, wgrad_dtype=wgrad)
    inp = make_inputs(cfg, device="cuda")
    g = _bwd_inputs(cfg, skew)
    out = run_bwd_mx(M, cfg, inp, g)
    shared = None
    if Fs:
        shared = dict(x=np64(inp["x"]), gu=np64(g["gu_s"]), ws_gate=np64(inp["ws_gate"]),
                      ws_up=np64(inp["ws_up"]), ws_down=np64(inp["ws_down"]))
    ref = O.ffn_backward(g["dy"], g["x_perm"], g["gu"], g["y_perm"], g["p"]["offsets"],
                         g["p"]["token_row"], g["idx"], g["w"], g["logits"],
                         np64(inp["w_gate"]), np64(inp["w_up"]), np64(inp["w_down"]),
                         score, renorm, "bf16", shared=shared, mxfp8=True)
    keys = ["d_gate", "d_logits", "dx", "dw_gate", "dw_up", "dw_down"]
    if Fs:
        keys += ["dws_gate", "dws_up", "dws_down"]
    for key in keys:
        assert_close(key, out[key], ref[key], "bf16")
    counts = np.diff(g["p"]["offsets"])
    for e in np.nonzero(counts == 0)[0]:
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert torch.all(out[key][int(e)] == 0), (key, e)
    if skew:
        assert (counts == 0).any()


MXW_CASES = [
    # name, T, d, E, k, F, score, renorm, skew, F_shared, wgrad_dtype: the
    # MXFP8 weight gradients (operands quantised along each expert's rows,
    # padded to 128); row counts that are no multiple of 32
    ("mxw_softmax_t300", 300, 256, 8, 2, 256, 0, 1, False, 0, 0),
    # the shared expert's 300 rows pad to 384; sigmoid scores
    ("mxw_shared_sigmoid_t300", 300, 256, 16, 4, 256, 1, 1, False, 256, 0),
    # empty experts: zero K steps, exactly zero gradients
    ("mxw_skewed_empty_t400", 400, 128, 16, 4, 128, 0, 1, True, 0, 0),
    # d = F = 384: the last row and column tiles half past the output;
    # bf16 weight gradients
    ("mxw_d384_shared_wgrad_bf16_t500", 500, 384, 12, 4, 384, 0, 1, True, 128, 1),
    # about 500 rows per expert: several 128-row blocks, 8 K steps
    ("mxw_long_k_t1000", 1000, 256, 4, 2, 256, 0, 1, False, 0, 0),
]


@pytest.mark.parametrize("case", MXW_CASES, ids=[c[0] for c in MXW_CASES])
def test_ffn_backward_mxfp8_weight_gradients(case):
    name, T, d, E, k, F, score, renorm, skew, Fs, wgrad = case
    _log(f"[backward mxfp8 wgrad] {name}")
    M = _lib()
    cfg = MoEConfig(name, T=T, d=d, E=E, k=k, F=F, F_shared=Fs, score=score,
                    renorm=renorm, backward=True, wgrad_dtype=wgrad, wgrad_mx=1)
    inp = make_inputs(cfg, device="cuda")
    g = _bwd_inputs(cfg, skew)
    out = run_bwd_mx(M, cfg, inp, g)
    shared = None
    if Fs:
        shared = dict(x=np64(inp["x"]), gu=np64(g["gu_s"]), ws_gate=np64(inp["ws_gate"]),
                      ws_up=np64(inp["ws_up"]), ws_down=np64(inp["ws_down"]))
    ref = O.ffn_backward(g["dy"], g["x_perm"], g["gu"], g["y_perm"], g["p"]["offsets"],
                         g["p"]["token_row"], g["idx"], g["w"], g["logits"],
                         np64(inp["w_gate"]), np64(inp["w_up"]), np64(inp["w_down"]),
                         score, renorm, "bf16", shared=shared, mxfp8=True, mx_wgrad=True)
    keys = ["d_gate", "d_logits", "dx", "dw_gate", "dw_up", "dw_down"]
    if Fs:
        keys += ["dws_gate", "dws_up", "dws_down"]
    for key in keys:
        assert_close(key, out[key], ref[key], "bf16")
    counts = np.diff(g["p"]["offsets"])
    for e in range(E):
        for key in ("dw_gate", "dw_up", "dw_down"):
            if counts[e] == 0:
                assert torch.all(out[key][e] == 0), (key, e)
            else:      # each expert on its own (a wrong block would hide in the whole)
                assert_close(f"{key}[{e}]", out[key][e], ref[key][e], "bf16")
    if skew:
        assert (counts == 0).any()


@pytest.mark.parametrize("wgrad_mx", [0, 1], ids=["bf16_wgrad", "mxfp8_wgrad"])
def test_ffn_backward_mxfp8_full_size_sampled(wgrad_mx):
    """The Qwen3-235B training shape: sampled tokens for dx, d_gate and
    d_logits; three whole experts for the weight gradients (bf16, or MXFP8
    along each expert's padded rows)."""
    cfg = CONFIGS["qwen3_235b_train_t8192"].replace(wgrad_mx=wgrad_mx)
    _log(f"[backward mxfp8 full] {cfg.name} wgrad_mx={wgrad_mx}")
    M = _lib()
    inp = make_inputs(cfg, device="cuda")
    g = _bwd_inputs(cfg)
    out = run_bwd_mx(M, cfg, inp, g)
    p = g["p"]
    tr, rt = p["token_row"], p["row_token"]
    w = np.asarray(g["w"], dtype=np.float64)
    toks = sample_tokens(cfg.T, 48)
    tt = torch.as_tensor(toks).cuda()

    def dY_rows(rows):
        """dY_perm of routed rows, from the oracle's dispatch gradient on
        just those rows."""
        t = rt[rows]
        j = np.argmax(tr[t] == rows[:, None], axis=1)
        dyt = np64(g["dy"][torch.as_tensor(t).cuda()])
        n = len(rows)
        return O.dispatch_grad(dyt, np.arange(n)[:, None], w[t, j][:, None], n, "bf16")

    def expert(e, rows):
        rr = torch.as_tensor(rows).cuda()
        return O.expert_backward(dY_rows(rows), g["x_perm"][rr], g["gu"][rr],
                                 np64(inp["w_gate"][e]), np64(inp["w_up"][e]),
                                 np64(inp["w_down"][e]), "bf16", mxfp8=True,
                                 mx_wgrad=bool(wgrad_mx))

    rows = tr[toks].reshape(-1)
    ex = np.searchsorted(p["offsets"], rows, side="right") - 1
    dX = np.zeros((len(rows), cfg.d))
    for e in np.unique(ex):
        sel = np.nonzero(ex == e)[0]
        dX[sel] = expert(int(e), rows[sel])["dX"]       # each row's dX is its own
    dx = dX.reshape(len(toks), cfg.k, cfg.d).sum(axis=1)
    assert_close("dx[sample]", out["dx"][tt], dx, "bf16")
    for e in (0, cfg.E // 2, cfg.E - 1):
        a, b = int(p["offsets"][e]), int(p["offsets"][e + 1])
        r = expert(e, np.arange(a, b))
        for key in ("dw_gate", "dw_up", "dw_down"):
            assert_close(f"{key}[{e}]", out[key][e], r[key], "bf16")
    del out, inp, g
    torch.cuda.empty_cache()
