"""Seeded synthetic inputs for exact attention, shared by the oracle tests,
the GPU parity tests and the benchmark.

This module holds no attention arithmetic: it only draws random numbers,
rounds them to bfloat16 and builds top-k index sets. Both sides of every
parity check start from the same bfloat16 bit patterns produced here: the
GPU path uploads the bits, the fp64 oracle upcasts the same bits exactly.

Workloads (all seeded; standard normal Q, K, V, dO drawn in that order):

* ``tiny_causal``   B=1  H=1  N=128   d=64   causal
* ``noncausal``     B=2  H=8  N=1024  d=64   non-causal
* ``headline``      B=8  H=16 N=4096  d=128  causal   (the backward benchmark)
* ``long8k``        B=1  H=16 N=8192  d=128  non-causal
* ``long16k``       B=1  H=16 N=16384 d=128  non-causal
* ``sparse_topk``   Nq=Nkv=4096, 64 query heads sharing one K/V head,
                    d_qk=576, d_v=512, top-k 512 per query row

The shapes and the causal setting of ``headline`` follow the setup of
"Writing Speed-of-Light Attention Backward Kernel for 5090 in CUDA"
(hoanh.space, section "Setup"); the sparse shape follows the D576/H64/top-k 512
cell of the benchmark matrix in cudnn-frontend PR #684 ("Improve performance
of SM100 DSA backward kernel").  The two adversarial regimes ``wide_logits``
and ``late_spike`` follow the validation description of the
s-samchenko/flash_attention_cuda README (its validate.py paragraph).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "DenseConfig", "SparseConfig", "DENSE_CONFIGS", "SPARSE_CONFIGS",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_bits_to_f64",
    "make_dense_inputs", "make_sparse_inputs", "make_topk_indices",
]


@dataclasses.dataclass(frozen=True)
class DenseConfig:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def with_(self, **kw) -> "DenseConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class SparseConfig:
    name: str
    Hq: int
    Nq: int
    Nkv: int
    dqk: int
    dv: int
    topk: int
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dqk)

    def with_(self, **kw) -> "SparseConfig":
        return dataclasses.replace(self, **kw)


DENSE_CONFIGS = {
    "tiny_causal": DenseConfig("tiny_causal", 1, 1, 128, 64, True),
    "noncausal": DenseConfig("noncausal", 2, 8, 1024, 64, False),
    "headline": DenseConfig("headline", 8, 16, 4096, 128, True),
    "long8k": DenseConfig("long8k", 1, 16, 8192, 128, False),
    "long16k": DenseConfig("long16k", 1, 16, 16384, 128, False),
}

SPARSE_CONFIGS = {
    "sparse_topk": SparseConfig("sparse_topk", 64, 4096, 4096, 576, 512, 512),
}


# ----------------------------------------------------------------------------
# bfloat16 bit conversion (round to nearest, ties to even)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs must be finite (the generators never produce NaN or Inf)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.shape, dtype=np.uint16)
    step = 1 << 20                               # chunks that stay in cache
    for s in range(0, u.size, step):
        c = u[s:s + step]
        t = c >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)                   # round half to even
        t += c
        t >>= np.uint32(16)
        out[s:s + step] = t
    return out.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


# ----------------------------------------------------------------------------
# Dense inputs
# ----------------------------------------------------------------------------
def make_dense_inputs(cfg: DenseConfig, regime: str = "gaussian") -> dict:
    """Q, K, V, dO of shape [B, H, N, d] as bfloat16 bits (uint16).

    One generator per workload (``numpy.random.default_rng(cfg.seed)``) draws
    float32 standard normals for Q, K, V and dO in that order.

    ``regime``:
      * ``gaussian``    i.i.d. N(0, 1).
      * ``wide_logits`` Q and K multiplied by 3, so logits have a standard
                        deviation near 9 and softmax rows are very peaked.
      * ``late_spike``  every query gets +1 and the keys of the final 64-key
                        tile get +1.5 in every feature, so the largest logits of
                        every row that sees that tile sit in the last tile; a
                        wrong running-max rescale shows up there.
    """
    rng = np.random.default_rng(cfg.seed)
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    do = rng.standard_normal(shape, dtype=np.float32)
    if regime == "gaussian":
        pass
    elif regime == "wide_logits":
        q *= np.float32(3.0)
        k *= np.float32(3.0)
    elif regime == "late_spike":
        q += np.float32(1.0)
        last = max(0, cfg.N - 64)
        k[:, :, last:, :] += np.float32(1.5)
    else:
        raise ValueError(f"unknown regime {regime!r}")
    return {
        "q": f32_to_bf16_bits(q),
        "k": f32_to_bf16_bits(k),
        "v": f32_to_bf16_bits(v),
        "do": f32_to_bf16_bits(do),
    }


def make_gqa_inputs(cfg: DenseConfig, hkv: int) -> dict:
    """Grouped-query inputs: Q and dO [B, H, N, d], K and V [B, Hkv, N, d], as
    bfloat16 bits.  One generator (``default_rng(cfg.seed)``) draws float32
    standard normals for Q, K, V and dO in that order."""
    rng = np.random.default_rng(cfg.seed)
    qs = (cfg.B, cfg.H, cfg.N, cfg.d)
    ks = (cfg.B, hkv, cfg.N, cfg.d)
    q = rng.standard_normal(qs, dtype=np.float32)
    k = rng.standard_normal(ks, dtype=np.float32)
    v = rng.standard_normal(ks, dtype=np.float32)
    do = rng.standard_normal(qs, dtype=np.float32)
    return {n: f32_to_bf16_bits(x) for n, x in (("q", q), ("k", k), ("v", v), ("do", do))}


# ----------------------------------------------------------------------------
# Sparse (top-k) inputs
# ----------------------------------------------------------------------------
def make_topk_indices(rng: np.random.Generator, nq: int, nkv: int, topk: int):
    """Per query row i, ``topk`` key indices drawn uniformly without replacement
    from [0, min(i, nkv - 1)] (all of that range when it is shorter than
    ``topk``), sorted ascending, int32, padded with -1.  Also returns the
    per-row count of valid entries (int32)."""
    idx = np.full((nq, topk), -1, dtype=np.int32)
    cnt = np.zeros((nq,), dtype=np.int32)
    for i in range(nq):
        n_allowed = min(i, nkv - 1) + 1
        if n_allowed <= topk:
            idx[i, :n_allowed] = np.arange(n_allowed, dtype=np.int32)
            cnt[i] = n_allowed
        else:
            pick = rng.choice(n_allowed, size=topk, replace=False)
            pick.sort()
            idx[i, :] = pick.astype(np.int32)
            cnt[i] = topk
    return idx, cnt


def make_sparse_inputs(cfg: SparseConfig) -> dict:
    """Sparse workload: q [Hq, Nq, dqk], k [Nkv, dqk], v [Nkv, dv],
    do [Hq, Nq, dv] as bfloat16 bits, then idx [Nq, topk] int32 (-1 padded)
    and topk_len [Nq] int32.  Draw order: Q, K, V, dO, then the indices."""
    rng = np.random.default_rng(cfg.seed)
    q = rng.standard_normal((cfg.Hq, cfg.Nq, cfg.dqk), dtype=np.float32)
    k = rng.standard_normal((cfg.Nkv, cfg.dqk), dtype=np.float32)
    v = rng.standard_normal((cfg.Nkv, cfg.dv), dtype=np.float32)
    do = rng.standard_normal((cfg.Hq, cfg.Nq, cfg.dv), dtype=np.float32)
    idx, cnt = make_topk_indices(rng, cfg.Nq, cfg.Nkv, cfg.topk)
    return {
        "q": f32_to_bf16_bits(q),
        "k": f32_to_bf16_bits(k),
        "v": f32_to_bf16_bits(v),
        "do": f32_to_bf16_bits(do),
        "idx": idx,
        "topk_len": cnt,
    }
