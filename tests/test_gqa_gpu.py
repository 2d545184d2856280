"""GPU parity of grouped-query attention (H query heads on Hkv K/V heads)
through the C ABI against the fp64 oracle (``oracle.gqa_forward`` /
``oracle.gqa_backward``) on the same seeded bf16 inputs, element by element:
O, L, D, dQ per query head and dK, dV per K/V head (summed over the query
heads that share it).  Cases cover d = 64 and 128, causal and not, ragged
lengths over several tiles, MQA (Hkv = 1) and G = 1 through the grouped entry
points, plus a full-length causal case (N = 4096) with the group sums of the
first and last K/V head checked against the oracle.
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


def test_gqa_full_length_group_sums(lib):
    """B1 H16 Hkv2 N4096 d128 causal: the whole GPU path at full length; dK / dV
    of K/V heads 0 and 1 (each the sum over 8 query heads) and dQ, O, L of the
    first and last query head checked element by element."""
    cfg = DenseConfig("gqa8_c128_4k", 1, 16, 4096, 128, True, seed=27)
    hkv = 2
    say(f"[parity-gqa-full] B1 H16 Hkv2 N4096 d128 causal")
    inp = make_gqa_inputs(cfg, hkv)
    out = _run(lib, inp, cfg)
    import torch
    for n in ("o", "lse", "D", "dq", "dk", "dv"):
        assert not torch.isnan(out[n]).any().item(), f"{n} has NaN (unwritten sentinel)"
    f = {n: bf16_bits_to_f64(inp[n]) for n in ("q", "k", "v", "do")}
    G = cfg.H // hkv
    for c in range(hkv):
        sl = slice(c * G, (c + 1) * G)
        ref = oracle.gqa_backward(f["q"][:, sl], f["k"][:, c:c + 1], f["v"][:, c:c + 1], f["do"][:, sl],
                                  cfg.scale, causal=True)
        assert_close(f"dk[{c}]", from_dev(out["dk"])[:, c:c + 1], ref["dk"])
        assert_close(f"dv[{c}]", from_dev(out["dv"])[:, c:c + 1], ref["dv"])
        for h in (0, G - 1):
            for n in ("o", "D", "dq"):
                assert_close(f"{n}[{c * G + h}]", from_dev(out[n])[:, c * G + h], ref[n][:, h])
            assert_lse(from_dev(out["lse"])[:, c * G + h], ref["lse"][:, h])
