"""attn_bwd_noalloc (the backward with the library's static scratch as its
workspace, for callers that cannot allocate) against attn_bwd with a caller
workspace, on the same inputs: bitwise equal results on two calls in a row,
the second with a smaller problem (the scratch keeps the first call's
contents); shapes beyond the scratch are rejected."""
import numpy as np
import pytest

from attn_inputs import DenseConfig, make_dense_inputs
from _util import say, to_dev

pytestmark = pytest.mark.gpu

CASES = [DenseConfig("na_big", 1, 2, 2000, 128, True, seed=31),
         DenseConfig("na_small", 1, 1, 333, 128, True, seed=32),
         DenseConfig("na_nc64", 2, 2, 700, 64, False, seed=33)]


def _run(lib, cfg):
    import torch
    inp = make_dense_inputs(cfg)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd(q, k, v, cfg.causal, cfg.scale)
    D = lib.attn_bwd_preprocess(o, do)
    ref = lib.attn_bwd(q, k, v, do, lse, D, cfg.causal, cfg.scale)
    out = tuple(torch.full_like(q, float("nan")) for _ in range(3))
    lib.attn_bwd_noalloc(q, k, v, do, lse, D, cfg.causal, *out, scale=cfg.scale)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_attn_bwd_twice(lib):
    import torch
    for cfg in CASES:                      # the second and third calls are smaller than the first
        need = lib.attn_bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d, cfg.causal)
        assert need <= lib.attn_bwd_noalloc_max_workspace_bytes()
        say(f"[noalloc] {cfg.name} B{cfg.B} H{cfg.H} N{cfg.N} d{cfg.d} causal={cfg.causal}: {need} bytes")
        ref, out = _run(lib, cfg)
        for n, a, b in zip(("dq", "dk", "dv"), ref, out):
            assert torch.equal(a, b), n


def test_noalloc_rejects_shapes_beyond_the_scratch(lib):
    import torch
    B, H, N, d = 1, 8, 4096, 128
    assert lib.attn_bwd_workspace_bytes(B, H, N, d, True) > lib.attn_bwd_noalloc_max_workspace_bytes()
    x = torch.zeros((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    st = torch.zeros((B, H, N), dtype=torch.float32, device="cuda")
    outs = tuple(torch.empty_like(x) for _ in range(3))
    with pytest.raises(lib.AttnError, match="static scratch"):
        lib.attn_bwd_noalloc(x, x, x, x, st, st, True, *outs)
