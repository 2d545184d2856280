"""The backward paths captured in a HIP graph and replayed.

Callers under stream capture (serving loops, graph-replayed training steps)
need every launch of a call to be capturable and every replay to start from a
clean state: the fused causal backward's ticket counters and progress flags
are reset by the prep kernel inside the call (a fill kernel, no memset node),
and nothing else in a workspace is read before it is written.  Each test
captures one call, then replays the graph several times with the program's own
eager work and synchronizations between the replays (the outputs are poisoned
with NaN before each replay), and checks every replay bit for bit against the
same call run eagerly: no floating-point atomics, so the results are
reproducible.
"""
import numpy as np
import pytest

from attn_inputs import DenseConfig, SparseConfig, make_dense_inputs, make_sparse_inputs
from _util import say, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _replay_and_compare(run_eager, run_captured, outs):
    """run_captured() enqueues the call writing into `outs` (a dict of
    tensors); run_eager() returns the same call's results as a dict."""
    import torch
    ref = {n: t.clone() for n, t in run_eager().items()}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_captured()                           # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        run_captured()
    for r in range(REPLAYS):
        for t in outs.values():
            t.fill_(float("nan"))                # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), f"replay {r}: {n} differs from the eager call"
    say(f"  {REPLAYS} replays bit-identical to the eager call ({', '.join(outs)})")


@pytest.mark.parametrize("causal,d", [(True, 128), (False, 128), (True, 64)],
                         ids=["fused_c128", "pair_n128", "pair_c64"])
def test_dense_backward_in_a_graph(lib, causal, d):
    import torch
    cfg = DenseConfig("graph", 1, 4, 600, d, causal, seed=31)
    say(f"[graph] attn_bwd B{cfg.B} H{cfg.H} N{cfg.N} d{d} causal={causal}")
    inp = make_dense_inputs(cfg)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd(q, k, v, causal, cfg.scale)
    D = lib.attn_bwd_preprocess(o, do)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, d, causal), dtype=torch.uint8,
                     device="cuda")
    outs = {n: torch.empty_like(q) for n in ("dq", "dk", "dv")}

    def eager():
        dq, dk, dv = lib.attn_bwd(q, k, v, do, lse, D, causal, cfg.scale, workspace=ws)
        return {"dq": dq, "dk": dk, "dv": dv}

    def captured():
        lib.attn_bwd(q, k, v, do, lse, D, causal, cfg.scale, dq=outs["dq"], dk=outs["dk"], dv=outs["dv"],
                     workspace=ws)

    _replay_and_compare(eager, captured, outs)


def test_forward_and_preprocess_in_a_graph(lib):
    import torch
    cfg = DenseConfig("graph_fwd", 2, 8, 700, 128, True, seed=32)
    say(f"[graph] attn_fwd + attn_bwd_preprocess B{cfg.B} H{cfg.H} N{cfg.N} causal")
    inp = make_dense_inputs(cfg)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    outs = {"o": torch.empty_like(q), "lse": torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda"),
            "D": torch.empty((cfg.B, cfg.H, cfg.N), dtype=torch.float32, device="cuda")}

    def eager():
        o, lse = lib.attn_fwd(q, k, v, True, cfg.scale)
        return {"o": o, "lse": lse, "D": lib.attn_bwd_preprocess(o, do)}

    def captured():
        lib.attn_fwd(q, k, v, True, cfg.scale, o=outs["o"], lse=outs["lse"])
        lib.attn_bwd_preprocess(outs["o"], do, D=outs["D"])

    _replay_and_compare(eager, captured, outs)


def test_noalloc_backward_in_a_graph(lib):
    """The scratch-free entry point is the one meant for capture."""
    import torch
    cfg = DenseConfig("graph_na", 1, 2, 500, 128, True, seed=33)
    say(f"[graph] attn_bwd_noalloc B{cfg.B} H{cfg.H} N{cfg.N} causal")
    inp = make_dense_inputs(cfg)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd(q, k, v, True, cfg.scale)
    D = lib.attn_bwd_preprocess(o, do)
    outs = {n: torch.empty_like(q) for n in ("dq", "dk", "dv")}

    def eager():
        dq, dk, dv = lib.attn_bwd(q, k, v, do, lse, D, True, cfg.scale)
        return {"dq": dq, "dk": dk, "dv": dv}

    def captured():
        lib.attn_bwd_noalloc(q, k, v, do, lse, D, True, outs["dq"], outs["dk"], outs["dv"], cfg.scale)

    _replay_and_compare(eager, captured, outs)


def test_sparse_backward_in_a_graph(lib):
    import torch
    cfg = SparseConfig("graph_sp", 64, 200, 300, 576, 512, 100, seed=34)
    say(f"[graph] attn_sparse_bwd Hq{cfg.Hq} Nq{cfg.Nq} Nkv{cfg.Nkv} topk{cfg.topk}")
    inp = make_sparse_inputs(cfg)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    idx = torch.from_numpy(np.ascontiguousarray(inp["idx"])).cuda()
    tl = torch.from_numpy(np.ascontiguousarray(inp["topk_len"])).cuda()
    o, lse = lib.attn_sparse_fwd(q, k, v, idx, tl, cfg.scale)
    D = lib.attn_bwd_preprocess(o[None], do[None])[0]
    ws = torch.empty(lib.attn_sparse_bwd_workspace_bytes(cfg.Hq, cfg.Nq, cfg.Nkv, cfg.topk), dtype=torch.uint8,
                     device="cuda")
    outs = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}

    def eager():
        dq, dk, dv = lib.attn_sparse_bwd(q, k, v, do, lse, D, idx, tl, cfg.scale, workspace=ws)
        return {"dq": dq, "dk": dk, "dv": dv}

    def captured():
        lib.attn_sparse_bwd(q, k, v, do, lse, D, idx, tl, cfg.scale, dq=outs["dq"], dk=outs["dk"],
                            dv=outs["dv"], workspace=ws)

    _replay_and_compare(eager, captured, outs)


def test_grouped_query_backward_in_a_graph(lib):
    """Causal d = 128 grouped-query heads: the fused kernel with fp32 partials
    and the group reduction after it, captured together."""
    import torch
    from attn_inputs import make_gqa_inputs
    cfg = DenseConfig("graph_gqa", 1, 8, 500, 128, True, seed=37)
    hkv = 2
    say(f"[graph] attn_bwd_gqa B{cfg.B} H{cfg.H} Hkv{hkv} N{cfg.N} causal")
    inp = make_gqa_inputs(cfg, hkv)
    q, k, v, do = (to_dev(inp[n]) for n in ("q", "k", "v", "do"))
    o, lse = lib.attn_fwd_gqa(q, k, v, True, cfg.scale)
    D = lib.attn_bwd_preprocess(o, do)
    ws = torch.empty(lib.attn_bwd_workspace_bytes(cfg.B, cfg.H, cfg.N, cfg.d, True, hkv), dtype=torch.uint8,
                     device="cuda")
    outs = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v)}

    def eager():
        dq, dk, dv = lib.attn_bwd_gqa(q, k, v, do, lse, D, True, cfg.scale, workspace=ws)
        return {"dq": dq, "dk": dk, "dv": dv}

    def captured():
        lib.attn_bwd_gqa(q, k, v, do, lse, D, True, cfg.scale, dq=outs["dq"], dk=outs["dk"], dv=outs["dv"],
                         workspace=ws)

    _replay_and_compare(eager, captured, outs)
