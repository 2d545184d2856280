"""The FLOP and byte conventions of bench.py, pinned to numbers the pages print.

Each (latency, TFLOPS) pair in tests/golden/page_timings.csv must be
reproduced by bench.py's FLOP count for that workload, within the rounding of
the two printed figures.  The byte count of the dense backward is pinned to
the read / write totals of the attention-backward page's Appendix C (roofline
model), and its FLOP count to the 1.374 TFLOP printed there.
"""
import csv
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_timings.csv")


def _rows():
    with open(GOLDEN) as f:
        return list(csv.DictReader(line for line in f if not line.startswith("#")))


def _half_unit(text):
    """Half a unit in the last printed digit of a decimal number."""
    frac = text.split(".")[1] if "." in text else ""
    return 0.5 * 10.0 ** (-len(frac))


def _flops(r):
    B, H, N = int(r["B"]), int(r["H"]), int(r["N"])
    dqk, dv, topk, causal = int(r["d_qk"]), int(r["d_v"]), int(r["topk"]), r["causal"] == "1"
    if r["kind"] == "dense_bwd":
        return bench.bwd_flops(B, H, N, dqk, causal)
    if r["kind"] == "dense_fwd":
        return bench.fwd_flops(B, H, N, dqk, causal)
    assert r["kind"] == "sparse_bwd" and B == 1
    return bench.sparse_bwd_flops(H, N, topk, dqk, dv)


ROWS = _rows()


def test_golden_table_is_complete():
    kinds = [r["kind"] for r in ROWS]
    assert kinds.count("dense_bwd") == 5
    assert kinds.count("dense_fwd") == 6
    assert kinds.count("sparse_bwd") == 32      # 4 configs x 4 top-k x (old, new)


@pytest.mark.parametrize("row", ROWS, ids=lambda r: f'{r["kind"]}-{r["label"]}-{r["topk"]}')
def test_printed_throughput_follows_from_flop_count(row):
    flops = _flops(row)
    ms, hm = float(row["ms"]), _half_unit(row["ms"])
    t, ht = float(row["tflops"]), _half_unit(row["tflops"])
    lo = bench.tflops(flops, ms + hm) - ht
    hi = bench.tflops(flops, ms - hm) + ht
    assert lo <= t <= hi, (row, bench.tflops(flops, ms))


def test_a_wrong_convention_fails_the_pin():
    # N(N+1)/2 causal pairs instead of N^2/2, or 4 products instead of 5, must
    # not reproduce the printed backward throughput
    r = next(r for r in ROWS if r["label"] == "v3")
    ms, t = float(r["ms"]), float(r["tflops"])
    B, H, N, d = 8, 16, 4096, 128
    exact_pairs = 2 * 5 * B * H * (N * (N + 1) / 2) * d
    assert abs(bench.tflops(exact_pairs, ms) - t) > 0.01
    assert abs(bench.tflops(0.8 * bench.bwd_flops(B, H, N, d, True), ms) - t) > 1.0


def test_dense_backward_flops_and_bytes_match_appendix_c():
    B, H, N, d = 8, 16, 4096, 128
    assert round(bench.bwd_flops(B, H, N, d, True) / 1e12, 3) == 1.374
    b = bench.bwd_min_bytes(B, H, N, d)
    assert round(b["read"] / 1e6) == 673
    assert round(b["write"] / 1e6) == 403
    assert round((b["read"] + b["write"]) / 1e9, 3) == 1.076
    # the roofline times printed beside them (209.5 TFLOP/s, 1.792 TB/s)
    assert round(bench.bwd_flops(B, H, N, d, True) / 209.5e12 * 1e3, 2) == 6.56
    assert round((b["read"] + b["write"]) / 1.792e12 * 1e3, 2) == 0.60
