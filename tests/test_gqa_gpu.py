"""GPU parity of grouped-query attention (H query heads on Hkv K/V heads)
through the C ABI against the fp64 oracle (``oracle.gqa_forward`` /
``oracle.gqa_backward``) on the same seeded bf16 inputs, element by element:
O, L, D, dQ per query head and dK, dV per K/V head (summed over the query
heads that share it).  Cases cover d = 64 and 128, causal and not, ragged
lengths over several tiles, MQA (Hkv = 1) and G = 1 through the grouped entry
points, plus full-length cases (N = 4096) through the fused kernel and
through the separate dK/dV and dQ kernels, with the group sums of the first
and last K/V head checked against the oracle.
"""
import numpy as np
import pytest

import oracle
from attn_inputs import DenseConfig, bf16_bits_to_f64, make_gqa_inputs
from _util import assert_close, assert_lse, from_dev, say, to_dev

pytestmark = pytest.mark.gpu

CASES = [
    (DenseConfig("gqa4_c128", 1, 8, 300, 128, True, seed=21), 2),
    (DenseConfig("mqa_n64", 2, 4, 200, 64, False, seed=22), 1),
    (DenseConfig("gqa4_n128", 1, 16, 520, 128, False, seed=23), 4),
    (DenseConfig("gqa2_c64", 1, 6, 129, 64, True, seed=24), 3),
    (DenseConfig("gqa1_c128", 2, 4, 100, 128, True, seed=25), 4),
    (DenseConfig("mqa_c128", 1, 8, 257, 128, True, seed=26), 1),
]


def _run(lib, inp, cfg):
    import torch
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, lse = lib.attn_fwd_gqa(q, k, v, cfg.causal, cfg.scale, o=o, lse=lse)
    D = lib.attn_bwd_preprocess(o, do)
    dq, dk, dv = torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    lib.attn_bwd_gqa(q, k, v, do, lse, D, cfg.causal, cfg.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "D": D, "dq": dq, "dk": dk, "dv": dv}


@pytest.mark.parametrize("cfg,hkv", CASES, ids=[c.name for c, _ in CASES])
def test_gqa_end_to_end(lib, cfg, hkv):
    say(f"[parity-gqa] {cfg.name} B{cfg.B} H{cfg.H} Hkv{hkv} N{cfg.N} d{cfg.d} causal={cfg.causal}")
    inp = make_gqa_inputs(cfg, hkv)
    out = _run(lib, inp, cfg)
    f = {n: bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "do")}
    ref = oracle.gqa_backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, causal=cfg.causal)
    for n in ("o", "D", "dq", "dk", "dv"):
        assert_close(n, from_dev(out[n]), ref[n])
    assert_lse(from_dev(out["lse"]), ref["lse"])


FULL = [
    # causal d = 128 runs the fused kernel, one item per (query head, key
    # tile), each writing fp32 dK / dV partials that the group reduction sums:
    # 8 query heads per K/V head, then 4 with many K/V heads
    (DenseConfig("gqa8_c128_4k", 1, 16, 4096, 128, True, seed=27), 2),
    (DenseConfig("gqa4_c128_b8", 8, 32, 4096, 128, True, seed=28), 8),
    # the separate dK/dV and dQ kernels: 4 query heads per K/V head, two per
    # workgroup at d = 128 (two partials), all four in one workgroup at d = 64
    # (no partials)
    (DenseConfig("gqa4_n128_b8", 8, 32, 4096, 128, False, seed=30), 8),
    (DenseConfig("gqa4_n64_b8", 8, 32, 4096, 64, False, seed=29), 8),
]


@pytest.mark.parametrize("cfg,hkv", FULL, ids=[c.name for c, _ in FULL])
def test_gqa_full_length_group_sums(lib, cfg, hkv):
    """The whole GPU path at full length; dK / dV of the first and last K/V
    head (each the sum over its query heads) and dQ, O, L of the first and last
    query head of those groups checked element by element."""
    say(f"[parity-gqa-full] {cfg.name} B{cfg.B} H{cfg.H} Hkv{hkv} N{cfg.N} d{cfg.d} causal={cfg.causal}")
    inp = make_gqa_inputs(cfg, hkv)
    out = _run(lib, inp, cfg)
    import torch
    for n in ("o", "lse", "D", "dq", "dk", "dv"):
        assert not torch.isnan(out[n]).any().item(), f"{n} has NaN (unwritten sentinel)"
    G = cfg.H // hkv
    q4 = lambda n: inp[n].reshape(cfg.B * cfg.H, cfg.N, cfg.d)          # noqa: E731
    k4 = lambda n: inp[n].reshape(cfg.B * hkv, cfg.N, cfg.d)            # noqa: E731
    res = {n: from_dev(out[n]).reshape((-1,) + tuple(out[n].shape[2:])) for n in out}
    for c in sorted({0, cfg.B * hkv - 1}):
        hs = slice(c * G, (c + 1) * G)                                  # its query heads (flattened)
        f = {"q": bf16_bits_to_f64(q4("q")[hs])[None], "do": bf16_bits_to_f64(q4("do")[hs])[None],
             "k": bf16_bits_to_f64(k4("k")[c])[None, None], "v": bf16_bits_to_f64(k4("v")[c])[None, None]}
        ref = oracle.gqa_backward(f["q"], f["k"], f["v"], f["do"], cfg.scale, causal=cfg.causal)
        assert_close(f"dk[{c}]", res["dk"][c], ref["dk"][0, 0])
        assert_close(f"dv[{c}]", res["dv"][c], ref["dv"][0, 0])
        for h in (0, G - 1):
            for n in ("o", "D", "dq"):
                assert_close(f"{n}[{c * G + h}]", res[n][c * G + h], ref[n][0, h])
            assert_lse(res["lse"][c * G + h], ref["lse"][0, h])


@pytest.mark.parametrize("B,H,hkv,N", [(1, 8, 2, 300), (8, 16, 2, 4096)])
def test_gqa_fused_control_block(lib, B, H, hkv, N):
    """Grouped-query causal d = 128 runs the persistent fused kernel with the
    query heads as its items: after a call its control block shows what the
    one-query-head-per-K/V-head case shows (every item published its last
    query tile, no wait reached its bound, every workgroup checked in, each
    queue's ticket counter ran one failed claim per workgroup of its XCD plus
    the sweep's past its items, and the sweep found nothing left)."""
    import torch
    cfg = DenseConfig("gqa_ctrl", B, H, N, 128, True, seed=35)
    say(f"[gqa-ctrl] B{B} H{H} Hkv{hkv} N{N}")
    inp = make_gqa_inputs(cfg, hkv)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd_gqa(q, k, v, True, cfg.scale)
    D = lib.attn_bwd_preprocess(o, do)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(B, H, N, 128, True, hkv), dtype=torch.uint8, device="cuda")
    lib.attn_bwd_gqa(q, k, v, do, lse, D, True, cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    tc2 = -(-N // 256)
    BH = B * H
    nq = [(BH - qq + 7) // 8 if qq < BH else 0 for qq in range(8)]    # query heads of queue qq, in pairs
    items = [(n + 1) // 2 * 2 * tc2 for n in nq]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = min(8 * max(items), max(8, cus // 8 * 8))
    ctrl = ws[: (64 + BH * tc2) * 4].view(torch.int32).cpu().numpy()
    say(f"  grid {grid} tickets {ctrl[:8].tolist()} finished {ctrl[8]} wait-bound {ctrl[9]} swept {ctrl[10]}")
    assert ctrl[8] == grid
    assert ctrl[9] == 0 and ctrl[10] == 0
    assert ctrl[:8].tolist() == [items[qq] + grid // 8 + 1 for qq in range(8)]
    prog = ctrl[64:].reshape(BH, tc2)
    assert np.array_equal(prog, np.tile(4 * np.arange(tc2), (BH, 1))), prog
