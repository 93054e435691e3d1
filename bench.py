"""Throughput of one GPU's MoE layer (tokens/s) with the grouped-GEMM rate.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--headline-only]

A step is one pass of the whole layer over one batch of seeded synthetic
tokens already resident in HBM: router GEMM + top-k, permutation, grouped
SwiGLU FFN (FC1 + FC2, plus the shared expert where the workload has one),
combine, and the backward where the workload is a training step.  The
default workload is the largest configuration, the Qwen3-235B-shape training
step (forward + backward).  W untimed warm-up steps, then K timed steps
between two device synchronisations.  Per stage, HIP events recorded on the
stream the library launches on give the mean, median and minimum duration;
inside the grouped FFN and backward calls the library records events around
each main kernel (moe_set_phase_events), and every such kernel is priced
against the MI355X roofline; the longest one is the line's `roofline`.  The
bandwidth stages (permute, combine) are also timed on their own, after a
scratch write that evicts the caches and back to back, beside this box's
plain device-copy rate.  The CPU oracle is timed on a bounded sample of the
same workload on the host cores.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

# Kernel sources per phase; traffic figures recorded in profiles/ are used
# only while these files are byte-identical to the ones profiled.
_CSRC = "mixture_experts_layer_logits_amd/csrc/"
FFN_SOURCES = (_CSRC + "ffn.hip", _CSRC + "gemm_tiles.h", _CSRC + "moe_common.h")
BWD_SOURCES = (_CSRC + "backward.hip", _CSRC + "gemm_tiles.h", _CSRC + "moe_common.h")


def ffn_flops(c):
    R = c.T * c.k
    return 6.0 * R * c.d * c.F + 6.0 * c.T * c.d * c.F_shared


def ffn_bytes(c, counts_nonzero):
    """Algorithmic HBM bytes of one grouped-FFN call: every expert weight
    with rows read once, x_perm read, h written and read back, y_perm
    written (plus the shared expert's x, weights, h and output)."""
    b = 2 if c.dtype == 1 else 4
    R = c.T * c.k
    w = 3.0 * counts_nonzero * c.d * c.F * b
    act = (R * c.d + 2 * R * c.F + R * c.d) * b
    if c.F_shared:
        w += 3.0 * c.d * c.F_shared * b
        act += (c.T * c.d + 2 * c.T * c.F_shared + c.T * c.d) * b
    if c.backward:
        act += (2 * R * c.F + 2 * c.T * c.F_shared) * b   # gu_save
    return w + act


def phase_figures(c, counts_nonzero):
    """Algorithmic FLOPs and HBM bytes of one launch of each phase kernel
    (the MOE_PHASE_* kernels of the routed experts), R = T k routed rows,
    E' = experts with rows, b = storage bytes, wb = weight-gradient bytes:
      fc1          4 R d F flops; W_g, W_u of E' experts, x_perm read, h
                   written (+ g | u when training)
      fc2          2 R F d; W_d of E' experts, h read, y_perm written
      bwd_dispatch dy and y_perm read, dY_perm written (+ fp32 logits read,
                   d_logits written)
      bwd_dh       2 R d F; dY_perm, W_d, g | u read; dg | du and h written
      bwd_dw_down  2 R d F; dY_perm and h read; dW_down of all E written
      bwd_dx       4 R F d; dg | du, W_g, W_u read; dX_perm written
      bwd_dw_gate_up 4 R d F; dg | du and x_perm read; dW_gate, dW_up of all
                   E written
      bwd_gather   dX_perm read, fp32 dx written
    The shared expert's work counts where it shares the launch (fc1, fc2)."""
    b = 2 if c.dtype == 1 else 4
    wb = 2 if c.wgrad_dtype == 1 else 4
    R, T, d, F, E, Fs = c.T * c.k, c.T, c.d, c.F, c.E, c.F_shared
    En = counts_nonzero
    f = {}
    f["fc1"] = (4.0 * R * d * F + 4.0 * T * d * Fs,
                (2.0 * En * F * d + R * d + R * F + (2 * R * F if c.backward else 0)) * b +
                ((2.0 * Fs * d + T * d + T * Fs + (2 * T * Fs if c.backward else 0)) * b
                 if Fs else 0))
    f["fc2"] = (2.0 * R * F * d + 2.0 * T * Fs * d,
                (En * d * F + R * F + R * d) * b + ((Fs * d + T * Fs + T * d) * b if Fs else 0))
    if c.backward:
        f["bwd_dispatch"] = (2.0 * R * d, (T * d + 2.0 * R * d) * b + 8.0 * T * E + 8.0 * T * c.k)
        f["bwd_dh"] = (2.0 * R * d * F, (R * d + En * d * F + 2 * R * F + 2 * R * F + R * F) * b)
        f["bwd_dw_down"] = (2.0 * R * d * F, (R * d + R * F) * b + 1.0 * E * d * F * wb)
        f["bwd_dx"] = (4.0 * R * F * d, (2.0 * R * F + 2.0 * En * F * d + R * d) * b)
        f["bwd_dw_gate_up"] = (4.0 * R * d * F, (2.0 * R * F + R * d) * b + 2.0 * E * F * d * wb)
        f["bwd_gather"] = (1.0 * R * d, R * d * b + 4.0 * T * d)
    return f


# The kernel behind each phase (names as a kernel trace prints them, for the
# headline bf16 shapes: d and F multiples of 256; {jb} is the row batch of
# the per-token gathers, the largest of 1, 2, 4, 8 not above k).
PHASE_KERNELS = {
    "fc1": "gemm_bf16_mfma_kernel<256, 128, 2, 1, 4, 2, 1> (FC1 + SwiGLU)",
    "fc2": "gemm_bf16_mfma_kernel<256, 256, 1, 0, 4, 2, 1> (FC2) + splitk_reduce_kernel",
    "bwd_dispatch": "bwd_dispatch_kernel<unsigned short, {jb}>",
    "bwd_dh": "bwd_dma_kernel<0> (dh + SwiGLU backward)",
    "bwd_dw_down": "bwd_wgrad_kernel<2> (dW_down, persistent)",
    "bwd_dx": "bwd_dma_kernel<1> (dX_perm)",
    "bwd_dw_gate_up": "bwd_wgrad_kernel<3> (dW_gate | dW_up, persistent)",
    "bwd_gather": "bwd_gather_kernel<unsigned short, {jb}>",
}


def phase_kernel(name, k):
    jb = 8 if k >= 8 else 4 if k >= 4 else 2 if k >= 2 else 1
    return PHASE_KERNELS[name].replace("{jb}", str(jb))


def price(flops, nbytes, ms):
    """Roofline of one kernel: the bound is the resource whose peak time is
    longer; achieved = algorithmic work / measured time against that peak."""
    t = ms / 1e3
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        a = flops / t / 1e12
        return {"bound": "mfma", "achieved": round(a, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / PEAK_BF16_TFLOPS, 4)}
    a = nbytes / t / 1e9
    return {"bound": "hbm", "achieved": round(a, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(a / PEAK_HBM_GBS, 4)}


def permute_bytes(c):
    """Algorithmic HBM bytes of moe_permute: topk_idx and topk_w read, x read
    once, the four maps and x_perm written."""
    b = 2 if c.dtype == 1 else 4
    R = c.T * c.k
    return 2 * R * 4 + c.T * c.d * b + (c.E + 1) * 4 + 3 * R * 4 + R * c.d * b


def combine_bytes(c):
    """Algorithmic HBM bytes of moe_unpermute_combine: y_perm, token_row and
    topk_w read (y_shared too when present), fp32 y written."""
    b = 2 if c.dtype == 1 else 4
    R = c.T * c.k
    extra = c.T * c.d * b if c.F_shared else 0
    return R * c.d * b + 2 * R * 4 + extra + c.T * c.d * 4


def sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload, kernel="moe_grouped_ffn", sources=FFN_SOURCES):
    """HBM bytes per launch of `kernel` from the committed FETCH_SIZE /
    WRITE_SIZE summary of this workload, or None when there is none or the
    kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("record:"):
                for kv in line.split()[1:]:
                    key, _, v = kv.partition("=")
                    vals[key] = v
    if vals.get("sources") != sources_digest(sources):
        return None
    try:
        return int(vals["bytes_per_call"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """A plain device copy of 1 GiB, three times, for scaling the FETCH_SIZE
    and WRITE_SIZE counters (each copy reads and writes exactly 1 GiB)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n} bytes 3 times", flush=True)


def _oracle_pass(cfg, inp, T):
    import oracle as O
    sub = cfg.replace(T=T)
    host = {}
    for k, v in inp.items():
        if v is None:
            host[k] = None
        elif k in ("x", "dy"):
            host[k] = v[:T].cpu()
        else:
            host[k] = v.cpu()
    t0 = time.perf_counter()
    out = O.forward(host, sub, save_gu=cfg.backward)
    if cfg.backward:
        shared = None
        if cfg.F_shared:
            shared = dict(x=host["x"], gu=out["gu_shared"], ws_gate=host["ws_gate"],
                          ws_up=host["ws_up"], ws_down=host["ws_down"])
        O.ffn_backward(host["dy"], out["x_perm"], out["gu_save"], out["y_perm"],
                       out["offsets"], out["token_row"], out["topk_idx"],
                       out["topk_w"], out["route_logits"], host["w_gate"],
                       host["w_up"], host["w_down"], cfg.score, cfg.renorm,
                       shared=shared)
    return time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def device_record(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1)}


def cpu_baseline(cfg, inp, sample_tokens=None, target_s=15.0):
    """The oracle, as it stands, on the first tokens of the same workload.
    Without a fixed sample size, passes on growing samples run until one
    takes at least target_s / 2 seconds (or covers the whole workload); the
    last pass is the one reported."""
    from threadpoolctl import threadpool_limits

    # the host cores this process may run on; the oracle's BLAS uses them all
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores, user_api="blas"):
        if sample_tokens:
            T = min(sample_tokens, cfg.T)
            dt = _oracle_pass(cfg, inp, T)
        else:
            # grow the sample (at most 8x a pass: fixed costs dominate small ones)
            T = min(cfg.T, 64)
            dt = _oracle_pass(cfg, inp, T)
            while dt < target_s / 2 and T < cfg.T:
                T = min(cfg.T, max(T + 1, int(T * min(8.0, target_s / max(dt, 1e-3)))))
                dt = _oracle_pass(cfg, inp, T)
    kind = "forward+backward" if cfg.backward else "forward"
    return {"value": round(T / dt, 2), "unit": "tokens/s", "cores": int(cores),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"first {T} of {cfg.T} tokens of the same workload, whole "
                      f"{kind} layer in the fp64 oracle ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3_235b_train_t8192",
                    help="the Qwen3-235B-shape training step (forward + backward), "
                         "the largest configuration, by default")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline step (no isolated stages, fused, "
                         "MXFP8 or other variants), so that a kernel trace of the run "
                         "holds the headline form's kernels alone")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling "
                         "the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU's layer; --gpus {args.gpus} is not "
              "supported (the layer is built and measured on a single GPU)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ctypes

    from mixture_experts_layer_logits_amd import MoELayer
    from mixture_experts_layer_logits_amd import _lib as L
    from moe_inputs import CONFIGS, make_inputs

    cfg = CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(cfg, device=dev)
    layer = MoELayer(cfg, device=dev)
    stream = torch.cuda.current_stream()
    stages = ["route", "permute", "ffn", "combine"] + (["backward"] if cfg.backward else [])

    def step(evs=None):
        for i, st in enumerate(stages):
            if evs is not None:
                evs[i].record(stream)
            if st == "backward":
                layer.backward(inp, inp["dy"])
            else:
                getattr(layer, st)(inp)
        if evs is not None:
            evs[len(stages)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
           for _ in range(args.steps)]
    # Per-kernel events: the library records pair p of a step's array around
    # phase p's kernels (moe_set_phase_events), on the stream it launches on.
    nph = 2 * L.MOE_PHASE_COUNT
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(nph)]
           for _ in range(args.steps)]
    for row in pev:
        for ev in row:
            ev.record(stream)          # creates the HIP event behind it
    parr = [(ctypes.c_void_p * nph)(*[ev.cuda_event for ev in row]) for row in pev]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        L.moe_set_phase_events(parr[s])
        step(evs[s])
    L.moe_set_phase_events(None)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    stage_samples = {st: [evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps)]
                     for i, st in enumerate(stages)}
    per_stage = {st: float(np.mean(v)) for st, v in stage_samples.items()}
    phase_ms = {}
    for p_, name in enumerate(L.PHASE_NAMES):
        if name.startswith("bwd") and not cfg.backward:
            continue
        v = [pev[s][2 * p_].elapsed_time(pev[s][2 * p_ + 1]) for s in range(args.steps)]
        phase_ms[name] = (float(np.mean(v)), float(np.median(v)), float(np.min(v)))

    # The bandwidth stages on their own, each repetition after a 512 MiB
    # scratch write that evicts the L2s and the 256 MB MALL ("flushed"), and
    # back to back with their inputs left in the caches ("cache_resident").
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    isolated = {}
    for st in (() if args.headline_only else ("permute", "combine")):
        fn = getattr(layer, st)
        res = {}
        for label, flush in (("flushed", True), ("cache_resident", False)):
            fn(inp)
            pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(args.steps)]
            for s_ in range(args.steps):
                if flush:
                    scratch.fill_(s_ & 255)
                pev[s_][0].record(stream)
                fn(inp)
                pev[s_][1].record(stream)
            torch.cuda.synchronize()
            res[label] = [pev[s_][0].elapsed_time(pev[s_][1]) for s_ in range(args.steps)]
        isolated[st] = res
    # This box's plain device copy of 1 GiB (read + write), the practical
    # ceiling of a copy-shaped stage such as permute and combine.
    copy_gbs = None
    if not args.headline_only:
        src = scratch[: 256 << 20]
        dst = torch.empty_like(src)
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(3):
            dst.copy_(src)
        cev[0].record(stream)
        for _ in range(10):
            dst.copy_(src)
        cev[1].record(stream)
        torch.cuda.synchronize()
        copy_gbs = 2 * src.numel() * 10 / (cev[0].elapsed_time(cev[1]) / 1e3) / 1e9
        del src, dst
    del scratch
    torch.cuda.empty_cache()

    # The same forward with the permutation fused into FC1's operand load
    # (maps-only permute, rows gathered from x; no x_perm), timed the same way.
    fused = None
    if not cfg.backward and not args.headline_only:
        def fused_step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            layer.route(inp)
            layer.permute(inp, maps_only=True)
            if ev is not None:
                ev[1].record(stream)
            layer.ffn(inp, fused=True)
            if ev is not None:
                ev[2].record(stream)
            layer.combine(inp)
            if ev is not None:
                ev[3].record(stream)
        for _ in range(args.warmup):
            fused_step()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        f0 = time.perf_counter()
        for s_ in range(args.steps):
            fused_step(fev[s_])
        torch.cuda.synchronize()
        fwall = (time.perf_counter() - f0) * 1e3 / args.steps
        fms = lambda a, b: float(np.mean([fev[s_][a].elapsed_time(fev[s_][b])
                                          for s_ in range(args.steps)]))
        fused = {"ms_per_step": round(fwall, 4),
                 "tokens_per_s": round(cfg.T / (fwall / 1e3), 1),
                 "stage_ms": {"route+permute_maps": round(fms(0, 1), 4),
                              "ffn_gathered": round(fms(1, 2), 4),
                              "combine": round(fms(2, 3), 4)}}
    # The forward with the combine folded into FC2's epilogue as well: route,
    # maps-only permute, then one FFN call that adds each gate-scaled expert
    # output into y (no y_perm, no combine launch).
    combined = None
    if not cfg.backward and not args.headline_only:
        def comb_step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            layer.route(inp)
            layer.permute(inp, maps_only=True)
            if ev is not None:
                ev[1].record(stream)
            layer.ffn_combine(inp)
            if ev is not None:
                ev[2].record(stream)
        for _ in range(args.warmup):
            comb_step()
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for s_ in range(args.steps):
            comb_step(cev[s_])
        torch.cuda.synchronize()
        cwall = (time.perf_counter() - c0) * 1e3 / args.steps
        cms = lambda a, b: float(np.mean([cev[s_][a].elapsed_time(cev[s_][b])
                                          for s_ in range(args.steps)]))
        combined = {"ms_per_step": round(cwall, 4),
                    "tokens_per_s": round(cfg.T / (cwall / 1e3), 1),
                    "stage_ms": {"route+permute_maps": round(cms(0, 1), 4),
                                 "ffn_combine": round(cms(1, 2), 4)}}
    # The forward with MXFP8 expert GEMMs (E4M3, blocks of 32, E8M0 scales):
    # weights quantised once and cached (outside the timed steps, reported
    # on its own), x quantised every step, rows gathered from the quantised x.
    mx = None
    if (not cfg.backward and not args.headline_only and cfg.dtype == 1 and
            all(v % 128 == 0 for v in (cfg.d, cfg.F, cfg.F_shared))):
        q0, q1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        q0.record(stream)
        layer.quantize_weights(inp)
        q1.record(stream)

        def mx_step(ev=None):
            parts = (lambda: (layer.route(inp), layer.permute(inp, maps_only=True)),
                     lambda: layer.quantize_x(inp), lambda: layer.ffn_mxfp8(inp),
                     lambda: layer.combine(inp))
            for i, fn in enumerate(parts):
                if ev is not None:
                    ev[i].record(stream)
                fn()
            if ev is not None:
                ev[len(parts)].record(stream)
        for _ in range(args.warmup):
            mx_step()
        mev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        m0 = time.perf_counter()
        for s_ in range(args.steps):
            mx_step(mev[s_])
        torch.cuda.synchronize()
        mwall = (time.perf_counter() - m0) * 1e3 / args.steps
        mms = lambda a, b: float(np.mean([mev[s_][a].elapsed_time(mev[s_][b])
                                          for s_ in range(args.steps)]))
        t_mx = mms(2, 3) / 1e3
        mx = {"ms_per_step": round(mwall, 4),
              "tokens_per_s": round(cfg.T / (mwall / 1e3), 1),
              "stage_ms": {"route+permute_maps": round(mms(0, 1), 4),
                           "quantize_x": round(mms(1, 2), 4),
                           "ffn_mxfp8": round(mms(2, 3), 4),
                           "combine": round(mms(3, 4), 4)},
              "ffn_tflops": round(ffn_flops(cfg) / t_mx / 1e12, 2),
              "ffn_frac_of_fp8_peak": round(ffn_flops(cfg) / t_mx / 1e12 / PEAK_FP8_TFLOPS, 4),
              "weight_quantize_ms_once": round(q0.elapsed_time(q1), 4)}

        # ... and with the combine in the MXFP8 FC2's epilogue (no y_perm)
        def mxc_step(ev=None):
            layer.route(inp)
            layer.permute(inp, maps_only=True)
            layer.quantize_x(inp)
            if ev is not None:
                ev[0].record(stream)
            layer.ffn_mxfp8_combine(inp)
            if ev is not None:
                ev[1].record(stream)
        for _ in range(args.warmup):
            mxc_step()
        cev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                for _ in range(args.steps)]
        torch.cuda.synchronize()
        c0 = time.perf_counter()
        for s_ in range(args.steps):
            mxc_step(cev2[s_])
        torch.cuda.synchronize()
        cwall2 = (time.perf_counter() - c0) * 1e3 / args.steps
        mx["with_combine_in_fc2"] = {
            "ms_per_step": round(cwall2, 4), "tokens_per_s": round(cfg.T / (cwall2 / 1e3), 1),
            "ffn_mxfp8_combine_ms": round(float(np.mean([cev2[s_][0].elapsed_time(cev2[s_][1])
                                                         for s_ in range(args.steps)])), 4)}
    # Training with selective rematerialisation: the forward keeps no g | u
    # and the backward reruns FC1 (same kernels) before its own GEMMs.
    remat = None
    if cfg.backward and not args.headline_only:
        rl = MoELayer(cfg, device=dev, recompute=True)

        def remat_step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            rl.forward(inp)
            if ev is not None:
                ev[1].record(stream)
            rl.backward(inp, inp["dy"])
            if ev is not None:
                ev[2].record(stream)
        for _ in range(args.warmup):
            remat_step()
        rev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        r0 = time.perf_counter()
        for s_ in range(args.steps):
            remat_step(rev[s_])
        torch.cuda.synchronize()
        rwall = (time.perf_counter() - r0) * 1e3 / args.steps
        rms = lambda a, b: float(np.mean([rev[s_][a].elapsed_time(rev[s_][b])
                                          for s_ in range(args.steps)]))
        esz = 2 if cfg.dtype == 1 else 4
        fc1r = {"ms_per_step": round(rwall, 4),
                "tokens_per_s": round(cfg.T / (rwall / 1e3), 1),
                "stage_ms": {"forward": round(rms(0, 1), 4),
                             "backward_with_fc1_recompute": round(rms(1, 2), 4)},
                "gu_bytes_not_kept": int((cfg.T * cfg.k * 2 * cfg.F + cfg.T * 2 * cfg.F_shared) * esz)}
        del rl
        torch.cuda.empty_cache()
        # The same training step with the weight gradients stored as bf16.
        bl = MoELayer(cfg.replace(wgrad_dtype=1), device=dev)
        for _ in range(args.warmup):
            bl.forward(inp)
            bl.backward(inp, inp["dy"])
        bev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        b0 = time.perf_counter()
        for s_ in range(args.steps):
            bl.forward(inp)
            bev[s_][0].record(stream)
            bl.backward(inp, inp["dy"])
            bev[s_][1].record(stream)
        torch.cuda.synchronize()
        bwall = (time.perf_counter() - b0) * 1e3 / args.steps
        remat = {"fc1_recomputed": fc1r}
        remat["bf16_weight_gradients"] = {
            "ms_per_step": round(bwall, 4), "tokens_per_s": round(cfg.T / (bwall / 1e3), 1),
            "backward_ms": round(float(np.mean([bev[s_][0].elapsed_time(bev[s_][1])
                                                for s_ in range(args.steps)])), 4)}
        del bl
        torch.cuda.empty_cache()
        # The same training step with the backward's data-gradient GEMMs in
        # MXFP8 (weights quantised for them once, outside the timed steps).
        if cfg.dtype == 1 and all(v % 128 == 0 for v in (cfg.d, cfg.F, cfg.F_shared)):
            ml = MoELayer(cfg, device=dev)
            q0, q1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
            q0.record(stream)
            ml.quantize_weights_t(inp)
            q1.record(stream)
            for _ in range(args.warmup):
                ml.forward(inp)
                ml.backward_mxfp8(inp, inp["dy"])
            mev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(args.steps)]
            torch.cuda.synchronize()
            m0 = time.perf_counter()
            for s_ in range(args.steps):
                ml.forward(inp)
                mev[s_][0].record(stream)
                ml.backward_mxfp8(inp, inp["dy"])
                mev[s_][1].record(stream)
            torch.cuda.synchronize()
            mwall = (time.perf_counter() - m0) * 1e3 / args.steps
            remat["mxfp8_data_gradients"] = {
                "ms_per_step": round(mwall, 4), "tokens_per_s": round(cfg.T / (mwall / 1e3), 1),
                "backward_ms": round(float(np.mean([mev[s_][0].elapsed_time(mev[s_][1])
                                                    for s_ in range(args.steps)])), 4),
                "weight_quantize_ms_once": round(q0.elapsed_time(q1), 4)}
            del ml
            torch.cuda.empty_cache()
            # ... and with the weight-gradient GEMMs in MXFP8 too (operands
            # quantised along each expert's rows, padded to the block): every
            # GEMM of the backward on MXFP8 operands
            ml = MoELayer(cfg.replace(wgrad_mx=1), device=dev)
            ml.quantize_weights_t(inp)
            for _ in range(args.warmup):
                ml.forward(inp)
                ml.backward_mxfp8(inp, inp["dy"])
            nph = 2 * L.MOE_PHASE_COUNT
            xev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 + nph)]
                   for _ in range(args.steps)]
            for row in xev:
                for ev in row:
                    ev.record(stream)
            xarr = [(ctypes.c_void_p * nph)(*[ev.cuda_event for ev in row[2:]]) for row in xev]
            torch.cuda.synchronize()
            m0 = time.perf_counter()
            for s_ in range(args.steps):
                ml.forward(inp)
                L.moe_set_phase_events(xarr[s_])
                xev[s_][0].record(stream)
                ml.backward_mxfp8(inp, inp["dy"])
                xev[s_][1].record(stream)
                L.moe_set_phase_events(None)
            torch.cuda.synchronize()
            mwall = (time.perf_counter() - m0) * 1e3 / args.steps
            pms = lambda p_: round(float(np.mean([xev[s_][2 + 2 * p_].elapsed_time(
                xev[s_][3 + 2 * p_]) for s_ in range(args.steps)])), 4)
            remat["mxfp8_backward"] = {
                "ms_per_step": round(mwall, 4), "tokens_per_s": round(cfg.T / (mwall / 1e3), 1),
                "backward_ms": round(float(np.mean([xev[s_][0].elapsed_time(xev[s_][1])
                                                    for s_ in range(args.steps)])), 4),
                "dw_down_ms (token-axis quantise + GEMM)": pms(L.MOE_PHASE_BWD_DW_DOWN),
                "dw_gate_up_ms (token-axis quantise + GEMM)": pms(L.MOE_PHASE_BWD_DW_GATE_UP)}
            del ml
            torch.cuda.empty_cache()
    ms_step = float(np.mean([evs[s][0].elapsed_time(evs[s][-1])
                             for s in range(args.steps)]))
    ms_wall = wall * 1e3 / args.steps
    tokens_per_s = cfg.T / (ms_wall / 1e3)

    counts = torch.diff(layer.buf["expert_offsets"]).cpu().numpy()
    n_nonzero = int((counts > 0).sum())
    flops = ffn_flops(cfg)
    t_ffn = per_stage["ffn"] / 1e3
    tflops = flops / t_ffn / 1e12
    bytes_ = ffn_bytes(cfg, n_nonzero)
    # the forward's grouped FFN call as a whole (FC1 + FC2 and their helpers)
    ffn_roof = price(flops, bytes_, per_stage["ffn"])
    ffn_roof["traffic"] = recorded_traffic(cfg.name)
    ffn_roof["algorithmic_bytes"] = int(bytes_)
    ffn_roof["kernel"] = ("moe_grouped_ffn: one call = tile schedule, FC1+SwiGLU "
                          "and FC2 grouped GEMM launches (+ split-K reduce)")
    # every phase kernel priced on its own; the dominant one (longest mean
    # launch) is the line's roofline
    figs = phase_figures(cfg, n_nonzero)
    kernels = {}
    for name, (mean, med, mn) in phase_ms.items():
        fl, nb = figs[name]
        r = price(fl, nb, mean)
        r.update({"kernel": phase_kernel(name, cfg.k), "ms_mean": round(mean, 4),
                  "ms_median": round(med, 4), "ms_min": round(mn, 4),
                  "algorithmic_flops": fl, "algorithmic_bytes": int(nb)})
        kernels[name] = r
    dom = max(kernels, key=lambda k_: kernels[k_]["ms_mean"])
    roof = {k_: kernels[dom][k_] for k_ in ("bound", "achieved", "peak", "unit", "frac")}
    roof["traffic"] = recorded_traffic(cfg.name, dom, BWD_SOURCES if dom.startswith("bwd")
                                       else FFN_SOURCES)
    roof.update({"kernel": kernels[dom]["kernel"], "phase": dom,
                 "ms_per_launch": kernels[dom]["ms_mean"],
                 "algorithmic_flops": kernels[dom]["algorithmic_flops"],
                 "algorithmic_bytes": kernels[dom]["algorithmic_bytes"]})

    hbm = {"copy_ceiling_GBs": None if copy_gbs is None else round(copy_gbs, 1)}
    for st, nb in (("permute", permute_bytes(cfg)), ("combine", combine_bytes(cfg))):
        gbs = nb / (per_stage[st] / 1e3) / 1e9
        hbm[st] = {"bytes": int(nb), "GB/s": round(gbs, 1),
                   "frac": round(gbs / PEAK_HBM_GBS, 4)}
        for label, v in isolated.get(st, {}).items():
            med = float(np.median(v))
            g = nb / (med / 1e3) / 1e9
            hbm[st][label] = {"ms_median": round(med, 4), "ms_min": round(float(np.min(v)), 4),
                              "GB/s": round(g, 1), "frac": round(g / PEAK_HBM_GBS, 4)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, args.cpu_sample_tokens)

    rec = {
        "metric": "MoE-layer tokens/sec + grouped-GEMM TFLOPS (fraction of peak) on 1 MI355X",
        "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_wall, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == 1 else "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "E": cfg.E, "k": cfg.k,
                   "F": cfg.F, "F_shared": cfg.F_shared,
                   "router": "sigmoid+groups" if cfg.score == 1 else "softmax",
                   "pass": "fwd+bwd" if cfg.backward else "fwd",
                   "parallelism": "single GPU"},
        "grouped_gemm_tflops": round(tflops, 2),
        "grouped_gemm_frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "stage_ms": {k: round(v, 4) for k, v in per_stage.items()},
        "stage_ms_median": {k: round(float(np.median(v)), 4) for k, v in stage_samples.items()},
        "stage_ms_min": {k: round(float(np.min(v)), 4) for k, v in stage_samples.items()},
        "stage_hbm": hbm,
        "event_ms_per_step": round(ms_step, 4),
        "fused_permute_forward": fused,
        "fused_permute_and_combine_forward": combined,
        "mxfp8_forward": mx,
        "training_variants": remat,
        "roofline": roof,
        "ffn_roofline": ffn_roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "device": device_record(torch),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
