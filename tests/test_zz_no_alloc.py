"""moe_permute_noalloc (the permutation with its scratch in a fixed device
array of the library, for callers that cannot allocate) against moe_permute
with a caller workspace: every map and x_perm bit for bit, on two calls in a
row, the second with a smaller input (the fixed array keeps the first call's
contents, which the second must not depend on).  Shapes beyond the array's
limit are refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from moe_inputs import MoEConfig, child_seed, normal, random_gates, random_topk

pytestmark = pytest.mark.gpu


def _bufs(cfg):
    dev = lambda *s, dt=torch.int32: torch.full(s, -7, dtype=dt, device="cuda")
    R = cfg.T * cfg.k
    return dict(offs=dev(cfg.E + 1), rt=dev(R), tr=dev(cfg.T, cfg.k),
                rg=dev(R, dt=torch.float32), xp=dev(R, cfg.d, dt=cfg.torch_dtype))


def _run(M, cfg, idx, gates, x, noalloc):
    b = _bufs(cfg)
    shape = M.make_shape(cfg)
    if noalloc:
        M.moe_permute_noalloc(shape, x, idx, gates, b["offs"], b["rt"], b["tr"], b["rg"], b["xp"])
    else:
        n = M.moe_workspace_size(shape, 1)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device="cuda")
        M.moe_permute(shape, x, idx, gates, b["offs"], b["rt"], b["tr"], b["rg"], b["xp"], ws, n)
    torch.cuda.synchronize()
    return b


@pytest.mark.parametrize("first,second", [
    # (T, E, k, skewed) of the two calls; the second is smaller each time
    ((20000, 64, 4, True), (3000, 64, 4, False)),     # separate scan launch, then fused scan
    ((16384, 256, 8, False), (700, 96, 2, True)),     # at the fused-scan limit, then small
    ((65536, 1024, 2, True), (1, 8, 1, False)),       # the array's limit, then one token
])
def test_permute_noalloc_matches_workspace_call(first, second):
    import mixture_experts_layer_logits_amd as M
    for i, (T, E, k, skew) in enumerate((first, second)):
        print(f"[noalloc] call {i}: T={T} E={E} k={k} skewed={skew}", flush=True)
        cfg = MoEConfig(f"noalloc_{i}", T=T, d=64, E=E, k=k, F=64)
        wts = [1.0 / (r + 1) ** 1.2 for r in range(E)] if skew else None
        idx = random_topk(T, E, k, seed=T + E + i, weights=wts).cuda()
        gates = random_gates(T, k, seed=T + i).cuda()
        x = normal((T, cfg.d), 1.0, cfg.torch_dtype, "cuda", child_seed(i, "x"))
        want = _run(M, cfg, idx, gates, x, noalloc=False)
        got = _run(M, cfg, idx, gates, x, noalloc=True)
        for key in ("offs", "rt", "tr", "rg", "xp"):
            assert torch.equal(got[key], want[key]), (i, key)
        # the maps are the permutation's: offsets are the counts' prefix sums
        counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=E)
        assert np.array_equal(got["offs"].cpu().numpy(),
                              np.concatenate([[0], np.cumsum(counts)]))


def test_permute_noalloc_refuses_shapes_beyond_its_array():
    """E * ceil(T / 256) above 2^18 is refused before any launch (the
    pointers are never dereferenced)."""
    import mixture_experts_layer_logits_amd as M
    from mixture_experts_layer_logits_amd import _lib as L
    p = 0x100000
    ok = M.make_shape(MoEConfig("at_limit", T=65536, d=64, E=1024, k=2, F=64))
    big = M.make_shape(MoEConfig("beyond", T=65536 + 1, d=64, E=1024, k=2, F=64))
    lib = L.load()
    st = lib.moe_permute_noalloc(ctypes.byref(big), p, p, p, p, p, p, p, p, 0)
    assert st == L.MOE_ERR_WORKSPACE
    # a bad argument is still an argument error at the limit
    st = lib.moe_permute_noalloc(ctypes.byref(ok), p, None, p, p, p, p, p, p, 0)
    assert st == L.MOE_ERR_INVALID_ARG
