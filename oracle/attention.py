"""Exact scaled-dot-product attention, forward and backward: the fp64 CPU oracle.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from it: the two share no code.  Inputs reach both
sides from the seeded generators in ``attn_inputs``.

What it computes is the plain definition, in float64, with every N x N matrix
(S, P, dP, dS) materialised per (batch, head).  It follows

* "Writing Speed-of-Light Attention Backward Kernel for 5090 in CUDA"
  (hoanh.space), section "Mathematical Formulation": the forward
  S = Q K^T / sqrt(d) + M, L_i = log sum_j exp(S_ij), P_ij = exp(S_ij - L_i),
  O = P V; and the backward dV = P^T dO, dP = dO V^T, D = rowsum(dO o O),
  dS = P o (dP - D 1^T), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d);
* the same page, Appendix B ("Softmax Backward Derivation"), for the row form
  ds = p o (dp - (p^T dp) 1);
* the same page, section "Mathematical Formulation" / pseudocode comments, for
  the causal mask: key index > query index is masked (score -inf, P = dS = 0);
* cudnn-frontend PR #684 ("Improve performance of SM100 DSA backward kernel"),
  summary and benchmark configuration, for the sparse top-k variant: each query
  row attends only to the keys its index list names, all query heads share one
  key/value head, and the key/value gradients are sums over heads.

``scale`` is the softmax scale (1/sqrt(d) on the pages); it is an argument so
that the oracle does not hard-code it.  Readings of points the pages leave
open:

* L is the natural-log log-sum-exp of the *scaled, masked* scores.
* A row with no visible key has O = 0, L = -inf and zero gradients.
* The backward recomputes P by normalising exp(S - max) by its row sum; it
  does not use L, so a kernel's L-based recomputation is checked, not copied.
* Top-k entries that are negative, or at or beyond the row's valid count, are
  ignored.  A repeated index counts as often as it appears (a gather).

Every function is pinned by tests that do not retype it: central finite
differences, a library routine (PyTorch CPU float64 attention with autograd),
closed forms and exact gradient identities.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "causal_allowed", "scores", "row_logsumexp", "softmax_rows",
    "attention_forward", "bwd_preprocess", "softmax_backward",
    "attention_backward", "topk_allowed", "sparse_forward", "sparse_backward",
    "gqa_forward", "gqa_backward", "attention_backward_sampled",
]


# ----------------------------------------------------------------------------
# Masks
# ----------------------------------------------------------------------------
def causal_allowed(n_q: int, n_k: int, row0: int = 0) -> np.ndarray:
    """Boolean [n_q, n_k]: True where key j may be seen by query i (j <= i,
    top-left aligned; the pages only use n_q == n_k).  Rows are the queries
    row0 .. row0 + n_q - 1 (a block of a taller mask)."""
    i = np.arange(row0, row0 + n_q)[:, None]
    j = np.arange(n_k)[None, :]
    return j <= i


# ----------------------------------------------------------------------------
# Forward (Mathematical Formulation: S, L, P, O)
# ----------------------------------------------------------------------------
def scores(q: np.ndarray, k: np.ndarray, scale: float, allowed=None) -> np.ndarray:
    """S = scale * Q K^T + M, where M is 0 on allowed pairs and -inf elsewhere.
    q: [..., Nq, d], k: [..., Nk, d] -> [..., Nq, Nk] float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if allowed is not None:
        s = np.where(allowed, s, -np.inf)
    return s


def row_logsumexp(s: np.ndarray) -> np.ndarray:
    """L_i = log sum_j exp(S_ij), evaluated as m + log sum exp(S - m) with the
    row maximum m; -inf for a row whose entries are all -inf."""
    m = np.max(s, axis=-1, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe)                      # exp(-inf) = 0 on masked entries
    total = np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        lse = np.where(finite, m_safe + np.log(total), -np.inf)
    return lse[..., 0]


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """P = row softmax of S: exp(S - max) / rowsum.  Rows with no finite entry
    give P = 0."""
    m = np.max(s, axis=-1, keepdims=True)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    e = np.exp(s - m_safe)
    total = np.sum(e, axis=-1, keepdims=True)
    return np.where(finite, e / np.where(finite, total, 1.0), 0.0)


def attention_forward(q, k, v, scale: float, causal: bool = False, allowed=None):
    """Forward pass.  q, k: [..., N, d]; v: [..., N, dv].

    Returns (O [..., Nq, dv] float64, L [..., Nq] float64) with
    L_i = log sum_j exp(S_ij) and P_ij = exp(S_ij - L_i), O = P V."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if causal:
        c = causal_allowed(q.shape[-2], k.shape[-2])
        allowed = c if allowed is None else (allowed & c)
    s = scores(q, k, scale, allowed)
    lse = row_logsumexp(s)
    lse_col = lse[..., None]
    with np.errstate(invalid="ignore"):
        p = np.where(np.isfinite(lse_col), np.exp(s - np.where(np.isfinite(lse_col), lse_col, 0.0)), 0.0)
    o = p @ v
    return o, lse


# ----------------------------------------------------------------------------
# Backward (Mathematical Formulation; Appendix B)
# ----------------------------------------------------------------------------
def bwd_preprocess(o, do) -> np.ndarray:
    """D = rowsum(dO o O): one softmax correction term per query row."""
    o = np.asarray(o, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    return np.sum(do * o, axis=-1)


def softmax_backward(p: np.ndarray, dp: np.ndarray, D: np.ndarray) -> np.ndarray:
    """dS = P o (dP - D 1^T), the stacked form of ds = p o (dp - (p^T dp) 1)."""
    return p * (dp - D[..., None])


def attention_backward(q, k, v, do, scale: float, causal: bool = False, allowed=None,
                       o_for_D=None):
    """Backward pass.  Returns a dict with dq, dk, dv, D and the recomputed o,
    lse, all float64.

    S and P are recomputed from Q and K with a plain softmax; then
    dV = P^T dO, dP = dO V^T, D = rowsum(dO o O), dS = P o (dP - D),
    dQ = scale * dS K, dK = scale * dS^T Q.

    ``o_for_D``: the O that the backward is given.  The preprocess of the
    attention-backward page ("Precomputing D") forms D from the O the forward
    stored, before the main loop; pass that stored O here (e.g. the forward's O
    rounded to the storage format) to follow that data flow.  By default D uses
    the exact O recomputed here."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    if causal:
        c = causal_allowed(q.shape[-2], k.shape[-2])
        allowed = c if allowed is None else (allowed & c)
    s = scores(q, k, scale, allowed)
    p = softmax_rows(s)
    lse = row_logsumexp(s)
    del s
    o = p @ v
    dv = np.swapaxes(p, -1, -2) @ do
    dp = do @ np.swapaxes(v, -1, -2)
    D = bwd_preprocess(o if o_for_D is None else o_for_D, do)
    ds = softmax_backward(p, dp, D)
    del p, dp
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    return {"dq": dq, "dk": dk, "dv": dv, "D": D, "o": o, "lse": lse}


def attention_backward_sampled(q, k, v, do, scale: float, causal: bool, rows, keys,
                               chunk: int = 1024):
    """The definitions of ``attention_backward`` for one (batch, head), kept to
    selected outputs: O, L, D and dQ of the query rows ``rows``, dK and dV of
    the keys ``keys``.  q, k, v, do: [N, d].  S and P are formed in blocks of
    ``chunk`` query rows (each row's softmax is complete inside its block), so
    no N x N matrix is held; the arithmetic per element is the same as in
    ``attention_backward``: P by plain softmax of S, D from the exact O,
    dS = P o (dP - D), dQ = scale * dS K, dK = scale * dS^T Q, dV = P^T dO.
    Returns a dict of float64 arrays: o, lse, D, dq [len(rows), ...] and
    dk, dv [len(keys), d]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n = q.shape[0]
    rows = np.asarray(rows, dtype=np.int64)
    keys = np.asarray(keys, dtype=np.int64)
    D = np.empty(n)
    o_rows = np.zeros((rows.size, v.shape[1]))
    lse_rows = np.empty(rows.size)
    dq_rows = np.zeros((rows.size, k.shape[1]))
    dk = np.zeros((keys.size, q.shape[1]))
    dv = np.zeros((keys.size, do.shape[1]))

    def block(r0, r1):
        allowed = causal_allowed(r1 - r0, n, row0=r0) if causal else None
        s = scores(q[r0:r1], k, scale, allowed)
        return s, softmax_rows(s)

    # every row's O (for D); the selected rows' O and L
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        s, p = block(r0, r1)
        o = p @ v
        D[r0:r1] = bwd_preprocess(o, do[r0:r1])
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        o_rows[sel] = o[rows[sel] - r0]
        lse_rows[sel] = row_logsumexp(s[rows[sel] - r0])
    # dS block by block: the selected keys' dK, dV and the selected rows' dQ
    for r0 in range(0, n, chunk):
        r1 = min(n, r0 + chunk)
        _, p = block(r0, r1)
        dp = do[r0:r1] @ v.T
        ds = softmax_backward(p, dp, D[r0:r1])
        dv += p[:, keys].T @ do[r0:r1]
        dk += scale * (ds[:, keys].T @ q[r0:r1])
        sel = np.nonzero((rows >= r0) & (rows < r1))[0]
        dq_rows[sel] = scale * (ds[rows[sel] - r0] @ k)
    return {"o": o_rows, "lse": lse_rows, "D": D[rows], "dq": dq_rows, "dk": dk, "dv": dv}


# ----------------------------------------------------------------------------
# Sparse top-k variant (cudnn-frontend PR #684)
# ----------------------------------------------------------------------------
def _valid_keys(idx_row: np.ndarray, count) -> np.ndarray:
    row = np.asarray(idx_row)
    if count is not None:
        row = row[: int(count)]
    return row[row >= 0].astype(np.int64)


def topk_allowed(idx, topk_len, n_kv: int) -> np.ndarray:
    """Dense boolean [Nq, Nkv] mask equivalent to the index lists (for
    duplicate-free lists)."""
    idx = np.asarray(idx)
    out = np.zeros((idx.shape[0], n_kv), dtype=bool)
    for i in range(idx.shape[0]):
        j = _valid_keys(idx[i], None if topk_len is None else topk_len[i])
        out[i, j] = True
    return out


def sparse_forward(q, k, v, idx, topk_len, scale: float):
    """q [Hq, Nq, dqk]; k [Nkv, dqk]; v [Nkv, dv]; idx [Nq, topk] int.

    For each query row i, gather the K and V rows its index list names (the
    same list for every head) and apply the dense forward to that set.
    Returns (O [Hq, Nq, dv], L [Hq, Nq])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, nq, _ = q.shape
    o = np.zeros((hq, nq, v.shape[-1]))
    lse = np.full((hq, nq), -np.inf)
    for i in range(nq):
        j = _valid_keys(idx[i], None if topk_len is None else topk_len[i])
        if j.size == 0:
            continue
        s = scale * (q[:, i, :] @ k[j].T)            # [Hq, t]
        lse_i = row_logsumexp(s)
        p = np.exp(s - lse_i[:, None])
        o[:, i, :] = p @ v[j]
        lse[:, i] = lse_i
    return o, lse


def sparse_backward(q, k, v, do, idx, topk_len, scale: float):
    """Backward of ``sparse_forward``.  Returns dict with dq [Hq, Nq, dqk],
    dk [Nkv, dqk], dv [Nkv, dv] (summed over heads and query rows), D [Hq, Nq],
    o, lse."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    hq, nq, _ = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    o = np.zeros((hq, nq, v.shape[-1]))
    lse = np.full((hq, nq), -np.inf)
    D = np.zeros((hq, nq))
    for i in range(nq):
        j = _valid_keys(idx[i], None if topk_len is None else topk_len[i])
        if j.size == 0:
            continue
        kg, vg = k[j], v[j]
        s = scale * (q[:, i, :] @ kg.T)              # [Hq, t]
        p = softmax_rows(s)
        lse[:, i] = row_logsumexp(s)
        o_i = p @ vg                                 # [Hq, dv]
        do_i = do[:, i, :]
        o[:, i, :] = o_i
        dp = do_i @ vg.T                             # [Hq, t]
        D_i = bwd_preprocess(o_i, do_i)              # [Hq]
        ds = softmax_backward(p, dp, D_i)            # [Hq, t]
        D[:, i] = D_i
        dq[:, i, :] = scale * (ds @ kg)
        np.add.at(dk, j, scale * (ds.T @ q[:, i, :]))
        np.add.at(dv, j, p.T @ do_i)
    return {"dq": dq, "dk": dk, "dv": dv, "D": D, "o": o, "lse": lse}


# ----------------------------------------------------------------------------
# Grouped-query attention: several query heads share one K/V head, as all the
# query heads of the sparse variant share its single K/V head (cudnn-frontend
# PR #684, DSA); the K/V gradients are then sums over the sharing heads.
# ----------------------------------------------------------------------------
def _expand_kv(x, h: int):
    """[..., Hkv, N, d] -> [..., H, N, d]: query head c * (H / Hkv) + r uses
    K/V head c."""
    x = np.asarray(x, dtype=np.float64)
    hkv = x.shape[-3]
    if h % hkv != 0:
        raise ValueError("Hkv must divide H")
    return np.repeat(x, h // hkv, axis=-3)


def gqa_forward(q, k, v, scale: float, causal: bool = False):
    """q [..., H, N, d]; k, v [..., Hkv, N, d].  Dense attention per query head
    with K/V head h / (H / Hkv).  Returns (O [..., H, N, dv], L [..., H, N])."""
    h = np.asarray(q).shape[-3]
    return attention_forward(q, _expand_kv(k, h), _expand_kv(v, h), scale, causal=causal)


def gqa_backward(q, k, v, do, scale: float, causal: bool = False, o_for_D=None):
    """Backward of ``gqa_forward``: per query head as ``attention_backward``,
    then dK and dV of each K/V head summed over the query heads that read it.
    Returns dict with dq [..., H, N, d], dk / dv [..., Hkv, N, d], D, o, lse."""
    h = np.asarray(q).shape[-3]
    hkv = np.asarray(k).shape[-3]
    g = attention_backward(q, _expand_kv(k, h), _expand_kv(v, h), do, scale, causal=causal,
                           o_for_D=o_for_D)
    group = lambda x: x.reshape(x.shape[:-3] + (hkv, h // hkv) + x.shape[-2:]).sum(axis=-3)  # noqa: E731
    g["dk"] = group(g["dk"])
    g["dv"] = group(g["dv"])
    return g

