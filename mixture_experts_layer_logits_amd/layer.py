"""The layer on one GPU: torch allocates device buffers once, the C ABI does
every step.

    layer = MoELayer(cfg)            # cfg: the layer's parameters
    out = layer.forward(inputs)      # route -> permute -> grouped FFN -> combine
    grads = layer.backward(inputs, out, dy)
"""
from __future__ import annotations

import torch

from . import _lib as L


class MoELayer:
    def __init__(self, cfg, device="cuda", save_gu=None, recompute=False):
        """recompute: train without keeping g | u from the forward; the
        backward runs FC1 again (selective rematerialisation)."""
        self.cfg = cfg
        self.shape = L.make_shape(cfg)
        self.device = torch.device(device)
        self.recompute = bool(recompute)
        if self.recompute:
            save_gu = False
        self.save_gu = bool(getattr(cfg, "backward", False)) if save_gu is None else save_gu
        T, d, E, k, F, Fs = cfg.T, cfg.d, cfg.E, cfg.k, cfg.F, cfg.F_shared
        R = T * k
        dt = torch.bfloat16 if cfg.dtype == L.MOE_DTYPE_BF16 else torch.float32
        dev = self.device
        ops = [L.MOE_OP_ROUTE, L.MOE_OP_PERMUTE, L.MOE_OP_FFN,
               L.MOE_OP_COMBINE, L.MOE_OP_FFN_COMBINE]
        if self.save_gu:
            ops.append(L.MOE_OP_BACKWARD)
        if self.recompute:
            ops.append(L.MOE_OP_BACKWARD_RECOMPUTE)
        # one scratch buffer serves every call: they are ordered on one stream
        self.ws_bytes = max(L.moe_workspace_size(self.shape, op) for op in ops)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        e = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=dev)
        i32, f32 = torch.int32, torch.float32
        self.buf = dict(
            logits=e(T, E, dtype=f32), topk_idx=e(T, k, dtype=i32),
            topk_w=e(T, k, dtype=f32), expert_offsets=e(E + 1, dtype=i32),
            row_token=e(R, dtype=i32), token_row=e(T, k, dtype=i32),
            row_gate=e(R, dtype=f32), x_perm=e(R, d), y_perm=e(R, d),
            y_shared=e(T, d) if Fs > 0 else None,
            # routed g | u [R, 2F], then the shared expert's [T, 2Fs]
            gu_save=e(R * 2 * F + T * 2 * Fs) if self.save_gu else None,
            y=e(T, d, dtype=f32))
        self.grad = None

    # ------------------------------------------------------------------
    def route(self, inp, stream=None):
        """Router scores from x and w_router, or, when inp holds "logits"
        (fp32 [T, E]), top-k and gates from those given scores."""
        b = self.buf
        given = inp.get("logits")
        if given is not None:
            b["logits"].copy_(given)
            L.moe_route_topk(self.shape, None, None, None, b["logits"],
                             inp.get("score_bias"), b["topk_idx"], b["topk_w"],
                             self.ws, self.ws_bytes, stream)
            return
        L.moe_route_topk(self.shape, inp["x"], inp["w_router"],
                         inp.get("router_bias"), b["logits"],
                         inp.get("score_bias"), b["topk_idx"], b["topk_w"],
                         self.ws, self.ws_bytes, stream)

    def permute(self, inp, stream=None, maps_only=False):
        b = self.buf
        L.moe_permute(self.shape, None if maps_only else inp["x"], b["topk_idx"],
                      b["topk_w"], b["expert_offsets"], b["row_token"],
                      b["token_row"], b["row_gate"],
                      None if maps_only else b["x_perm"], self.ws, self.ws_bytes,
                      stream)

    def ffn(self, inp, stream=None, fused=False):
        """fused: FC1 gathers its rows from x through row_token (after a
        maps-only permute) instead of reading x_perm."""
        b = self.buf
        L.moe_grouped_ffn(self.shape, None if fused else b["x_perm"],
                          b["row_token"], b["expert_offsets"],
                          inp["w_gate"], inp["w_up"], inp["w_down"],
                          inp["x"] if (fused or self.cfg.F_shared > 0) else None,
                          inp.get("ws_gate"), inp.get("ws_up"),
                          inp.get("ws_down"), b["y_perm"], b["y_shared"],
                          b["gu_save"], self.ws, self.ws_bytes, stream)

    def combine(self, inp, stream=None):
        b = self.buf
        L.moe_unpermute_combine(self.shape, b["y_perm"], b["token_row"],
                                b["topk_w"], b["y_shared"], b["y"], self.ws,
                                self.ws_bytes, stream)

    def ffn_combine(self, inp, stream=None, gather=True):
        """The grouped FFN with the combine in FC2's epilogue: y straight
        from the expert GEMMs, no y_perm.  gather: FC1 reads its rows from x
        (after a maps-only permute), else from x_perm."""
        b = self.buf
        L.moe_grouped_ffn_combine(self.shape, None if gather else b["x_perm"],
                                  b["row_token"], b["row_gate"], b["expert_offsets"],
                                  inp["w_gate"], inp["w_up"], inp["w_down"],
                                  inp["x"] if (gather or self.cfg.F_shared > 0) else None,
                                  inp.get("ws_gate"), inp.get("ws_up"),
                                  inp.get("ws_down"), b["y"], self.ws, self.ws_bytes,
                                  stream)

    def forward_combined(self, inp, stream=None):
        """route -> maps-only permute -> FFN with the combine in FC2's
        epilogue (inference: the backward's x_perm, y_perm and g | u are not
        produced)."""
        self.route(inp, stream)
        self.permute(inp, stream, maps_only=True)
        self.ffn_combine(inp, stream)
        return self.buf

    def forward(self, inp, stream=None, fused=False):
        """fused=True skips x_perm: the permutation only builds the maps and
        FC1 gathers its rows from x (not for training, whose backward reads
        x_perm)."""
        if fused and self.save_gu:
            raise ValueError("the fused forward keeps no x_perm for the backward")
        self.route(inp, stream)
        self.permute(inp, stream, maps_only=fused)
        self.ffn(inp, stream, fused=fused)
        self.combine(inp, stream)
        return self.buf

    # ------------------------------------------------------------------
    # MXFP8 forward
    def quantize_weights(self, inp, stream=None):
        """E4M3 codes and E8M0 scales of every expert weight, along its
        contraction dimension; kept for every later MXFP8 forward (the
        weights change only at an optimizer step)."""
        dev = self.device
        out = {}
        names = ["w_gate", "w_up", "w_down"]
        if self.cfg.F_shared > 0:
            names += ["ws_gate", "ws_up", "ws_down"]
        for n in names:
            w = inp[n]
            cols = w.shape[-1]
            rows = w.numel() // cols
            q = torch.empty(w.shape, dtype=torch.uint8, device=dev)
            sc = torch.empty(*w.shape[:-1], cols // 32, dtype=torch.uint8, device=dev)
            L.moe_mx_quantize(w, rows, cols, q, sc, stream)
            out[n] = (q, sc)
        self.mx_weights = out
        return out

    def _mx_buffers(self):
        if getattr(self, "mx_buf", None) is None:
            c = self.cfg
            n = L.moe_workspace_size(self.shape, L.MOE_OP_FFN_MXFP8)
            self.mx_buf = dict(
                xq=torch.empty(c.T, c.d, dtype=torch.uint8, device=self.device),
                xs=torch.empty(c.T, c.d // 32, dtype=torch.uint8, device=self.device),
                ws=torch.empty(max(n, 256), dtype=torch.uint8, device=self.device),
                ws_bytes=n)
        return self.mx_buf

    def quantize_x(self, inp, stream=None):
        """x [T, d] to MXFP8 (codes and block scales along d)."""
        m = self._mx_buffers()
        L.moe_mx_quantize(inp["x"], self.cfg.T, self.cfg.d, m["xq"], m["xs"], stream)

    def ffn_mxfp8(self, inp, stream=None):
        """The MXFP8 grouped FFN on the quantised x, routed rows gathered
        through row_token (needs quantize_weights() and quantize_x())."""
        if getattr(self, "mx_weights", None) is None:
            raise RuntimeError("call quantize_weights() before the MXFP8 FFN")
        b, m, w = self.buf, self._mx_buffers(), self.mx_weights
        none = (None, None)
        L.moe_grouped_ffn_mxfp8(
            self.shape, m["xq"], m["xs"], b["row_token"], b["expert_offsets"],
            *w["w_gate"], *w["w_up"], *w["w_down"], *w.get("ws_gate", none),
            *w.get("ws_up", none), *w.get("ws_down", none), b["y_perm"],
            b["y_shared"], m["ws"], m["ws_bytes"], stream)

    def ffn_mxfp8_combine(self, inp, stream=None):
        """The MXFP8 grouped FFN with the combine in FC2's epilogue: y
        straight from the expert GEMMs (needs quantize_weights() and
        quantize_x())."""
        if getattr(self, "mx_weights", None) is None:
            raise RuntimeError("call quantize_weights() before the MXFP8 FFN")
        b, m, w = self.buf, self._mx_buffers(), self.mx_weights
        none = (None, None)
        L.moe_grouped_ffn_mxfp8_combine(
            self.shape, m["xq"], m["xs"], b["row_token"], b["row_gate"],
            b["expert_offsets"], *w["w_gate"], *w["w_up"], *w["w_down"],
            *w.get("ws_gate", none), *w.get("ws_up", none), *w.get("ws_down", none),
            b["y"], m["ws"], m["ws_bytes"], stream)

    def forward_mxfp8_combined(self, inp, stream=None):
        """route -> permute (maps only) -> quantise x -> MXFP8 FFN with the
        combine in FC2, with the cached quantised weights."""
        self.route(inp, stream)
        self.permute(inp, stream, maps_only=True)
        self.quantize_x(inp, stream)
        self.ffn_mxfp8_combine(inp, stream)
        return self.buf

    def forward_mxfp8(self, inp, stream=None):
        """route -> permute (maps only) -> quantise x -> MXFP8 grouped FFN ->
        combine, with the cached quantised weights."""
        self.route(inp, stream)
        self.permute(inp, stream, maps_only=True)
        self.quantize_x(inp, stream)
        self.ffn_mxfp8(inp, stream)
        self.combine(inp, stream)
        return self.buf

    # ------------------------------------------------------------------
    def _alloc_grad(self):
        c = self.cfg
        dev, f32 = self.device, torch.float32
        wt = torch.bfloat16 if getattr(c, "wgrad_dtype", 0) == L.MOE_DTYPE_BF16 else f32
        self.grad = dict(
            dx=torch.empty(c.T, c.d, dtype=f32, device=dev),
            dw_gate=torch.empty(c.E, c.F, c.d, dtype=wt, device=dev),
            dw_up=torch.empty(c.E, c.F, c.d, dtype=wt, device=dev),
            dw_down=torch.empty(c.E, c.d, c.F, dtype=wt, device=dev),
            d_gate=torch.empty(c.T, c.k, dtype=f32, device=dev),
            d_logits=torch.empty(c.T, c.E, dtype=f32, device=dev))
        fs = c.F_shared
        self.grad.update(
            dws_gate=torch.empty(fs, c.d, dtype=wt, device=dev) if fs else None,
            dws_up=torch.empty(fs, c.d, dtype=wt, device=dev) if fs else None,
            dws_down=torch.empty(c.d, fs, dtype=wt, device=dev) if fs else None)

    def gu_views(self):
        """(routed [R, 2F], shared [T, 2Fs] or None) views of gu_save."""
        c, gu = self.cfg, self.buf["gu_save"]
        if gu is None:
            return None, None
        n = c.T * c.k * 2 * c.F
        routed = gu[:n].view(c.T * c.k, 2 * c.F)
        shared = gu[n:].view(c.T, 2 * c.F_shared) if c.F_shared else None
        return routed, shared

    def backward(self, inp, dy, stream=None):
        if self.grad is None:
            self._alloc_grad()
        b, g = self.buf, self.grad
        sh = self.cfg.F_shared > 0
        L.moe_ffn_backward(self.shape, dy, b["x_perm"], b["gu_save"],
                           b["y_perm"], b["expert_offsets"], b["row_token"],
                           b["token_row"], b["topk_idx"], b["topk_w"],
                           b["logits"], inp["w_gate"], inp["w_up"],
                           inp["w_down"], inp["x"] if sh else None,
                           inp.get("ws_gate"), inp.get("ws_up"),
                           inp.get("ws_down"), g["dx"], g["dw_gate"],
                           g["dw_up"], g["dw_down"], g["dws_gate"],
                           g["dws_up"], g["dws_down"], g["d_gate"],
                           g["d_logits"], self.ws, self.ws_bytes, stream)
        return g

    # ------------------------------------------------------------------
    # MXFP8 backward (data-gradient GEMMs in MXFP8, weight gradients bf16)
    def quantize_weights_t(self, inp, stream=None):
        """The weights quantised along the dimension the backward's data
        gradients contract: w_down along d ([E, F, d]) and w_gate | w_up
        along F ([E, d, 2F]); kept until the weights change."""
        c, dev = self.cfg, self.device
        u8 = torch.uint8

        def pair(E, d, F, wd, wg, wu):
            wd_q = torch.empty(E, F, d, dtype=u8, device=dev)
            wd_s = torch.empty(E, F, d // 32, dtype=u8, device=dev)
            L.moe_mx_quantize_t(wd, E, d, F, d, wd_q, wd_s, stream)
            gu_q = torch.empty(E, d, 2 * F, dtype=u8, device=dev)
            gu_s = torch.empty(E, d, 2 * F // 32, dtype=u8, device=dev)
            L.moe_mx_quantize_t(wg, E, F, d, 2 * F, gu_q, gu_s, stream)
            L.moe_mx_quantize_t(wu, E, F, d, 2 * F, gu_q.view(-1)[F:], gu_s.view(-1)[F // 32:],
                                stream)
            return wd_q, wd_s, gu_q, gu_s

        out = {"routed": pair(c.E, c.d, c.F, inp["w_down"], inp["w_gate"], inp["w_up"])}
        if c.F_shared:
            out["shared"] = pair(1, c.d, c.F_shared, inp["ws_down"], inp["ws_gate"], inp["ws_up"])
        self.mx_weights_t = out
        return out

    def backward_mxfp8(self, inp, dy, stream=None):
        """The backward with MXFP8 data-gradient GEMMs (needs
        quantize_weights_t() and a forward that saved g | u)."""
        if getattr(self, "mx_weights_t", None) is None:
            raise RuntimeError("call quantize_weights_t() before the MXFP8 backward")
        if self.grad is None:
            self._alloc_grad()
        if getattr(self, "mx_bwd_ws", None) is None:
            n = L.moe_workspace_size(self.shape, L.MOE_OP_BACKWARD_MXFP8)
            self.mx_bwd_ws = (torch.empty(max(n, 256), dtype=torch.uint8, device=self.device), n)
        b, g, w = self.buf, self.grad, self.mx_weights_t
        ws, nws = self.mx_bwd_ws
        sh = self.cfg.F_shared > 0
        shw = w["shared"] if sh else (None, None, None, None)
        L.moe_ffn_backward_mxfp8(
            self.shape, dy, b["x_perm"], b["gu_save"], b["y_perm"],
            b["expert_offsets"], b["row_token"], b["token_row"], b["topk_idx"],
            b["topk_w"], b["logits"], *w["routed"], inp["x"] if sh else None, *shw,
            g["dx"], g["dw_gate"], g["dw_up"], g["dw_down"], g["dws_gate"],
            g["dws_up"], g["dws_down"], g["d_gate"], g["d_logits"], ws, nws, stream)
        return g
