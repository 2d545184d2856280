"""Pins for the fp64 oracle, each against something other than the oracle itself.

* central finite differences of the scalar loss  sum(dO o O)  (pins dQ, dK, dV
  of the backward against the forward, with no formula retyped);
* PyTorch's CPU float64 attention with autograd, a separate library
  implementation (pins O, L, dQ, dK, dV, scale and the causal convention);
* closed forms and exact identities that follow from the definitions
  (softmax rows sum to one, rowsum(dS) = 0, masked P is exactly 0, ...);
* planted mistakes: a wrong oracle must fail at least one of the pins above.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as oa


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _loss(q, k, v, do, scale, causal, allowed=None):
    o, _ = oracle.attention_forward(q, k, v, scale, causal=causal, allowed=allowed)
    return float(np.sum(do * o))


def _fd_grad(f, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ----------------------------------------------------------------------------
# finite differences
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("n,d", [(5, 3), (7, 4)])
def test_backward_matches_finite_differences(causal, n, d):
    rng = np.random.default_rng(1234 + n + 10 * d + causal)
    q, k, v, do = (_rand(rng, 1, 2, n, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    g = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _fd_grad(lambda: _loss(q, k, v, do, scale, causal), x)
        assert _rel(g[name], fd) < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_backward_matches_finite_differences(causal):
    """Pins the head sums of dK / dV: 4 query heads on 2 K/V heads."""
    rng = np.random.default_rng(99 + causal)
    n, d = 5, 3
    q, do = (_rand(rng, 1, 4, n, d) for _ in range(2))
    k, v = (_rand(rng, 1, 2, n, d) for _ in range(2))
    scale = 1.0 / math.sqrt(d)
    g = oracle.gqa_backward(q, k, v, do, scale, causal=causal)
    loss = lambda: float(np.sum(do * oracle.gqa_forward(q, k, v, scale, causal=causal)[0]))  # noqa: E731
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        assert g[name].shape == x.shape, name
        assert _rel(g[name], _fd_grad(loss, x)) < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_mqa_equals_sparse_with_full_index_lists(causal):
    """One K/V head for every query head is the sparse variant with every key
    (or every key up to the row) in each row's list: two separately written
    head-sum paths must agree."""
    rng = np.random.default_rng(5 + causal)
    h, n, d = 3, 6, 4
    q, do = _rand(rng, h, n, d), _rand(rng, h, n, d)
    k, v = _rand(rng, n, d), _rand(rng, n, d)
    idx = np.tile(np.arange(n), (n, 1))
    tl = np.arange(1, n + 1) if causal else None
    sp = oracle.sparse_backward(q, k, v, do, idx, tl, 0.5)
    gq = oracle.gqa_backward(q[None], k[None, None], v[None, None], do[None], 0.5, causal=causal)
    for name in ("dq", "o", "lse", "D"):
        np.testing.assert_allclose(gq[name][0], sp[name], rtol=1e-12, atol=1e-12, err_msg=name)
    for name in ("dk", "dv"):
        np.testing.assert_allclose(gq[name][0, 0], sp[name], rtol=1e-12, atol=1e-12, err_msg=name)


def test_sparse_backward_matches_finite_differences():
    rng = np.random.default_rng(7)
    hq, nq, nkv, dqk, dv, topk = 2, 6, 6, 4, 3, 3
    q = _rand(rng, hq, nq, dqk)
    k = _rand(rng, nkv, dqk)
    v = _rand(rng, nkv, dv)
    do = _rand(rng, hq, nq, dv)
    from attn_inputs import make_topk_indices
    idx, cnt = make_topk_indices(rng, nq, nkv, topk)
    scale = 1.0 / math.sqrt(dqk)
    g = oracle.sparse_backward(q, k, v, do, idx, cnt, scale)

    def loss():
        o, _ = oracle.sparse_forward(q, k, v, idx, cnt, scale)
        return float(np.sum(do * o))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        assert _rel(g[name], _fd_grad(loss, x)) < 1e-7, name


def test_sparse_unsorted_repeated_lists():
    """Index lists in any order and with a repeated key: the backward still
    matches finite differences of the forward, and the forward weighs a key
    named twice by two (a gather over slots), as the closed form says."""
    rng = np.random.default_rng(17)
    hq, nq, nkv, dqk, dv = 2, 4, 5, 4, 3
    q, k, v, do = _rand(rng, hq, nq, dqk), _rand(rng, nkv, dqk), _rand(rng, nkv, dv), _rand(rng, hq, nq, dv)
    idx = np.array([[3, 0, 3, -1], [4, 1, 2, 1], [2, 2, 2, 0], [0, 4, 1, 3]], dtype=np.int32)
    cnt = np.array([3, 4, 4, 2], dtype=np.int32)
    scale = 0.7
    g = oracle.sparse_backward(q, k, v, do, idx, cnt, scale)

    def loss():
        o, _ = oracle.sparse_forward(q, k, v, idx, cnt, scale)
        return float(np.sum(do * o))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        assert _rel(g[name], _fd_grad(loss, x)) < 1e-7, name
    o, lse = oracle.sparse_forward(q, k, v, idx, cnt, scale)
    for h in range(hq):                          # row 0 names key 3 twice and key 0 once
        e3, e0 = np.exp(scale * q[h, 0] @ k[3]), np.exp(scale * q[h, 0] @ k[0])
        assert _rel(o[h, 0], (2 * e3 * v[3] + e0 * v[0]) / (2 * e3 + e0)) < 1e-13
        assert abs(lse[h, 0] - np.log(2 * e3 + e0)) < 1e-13


# ----------------------------------------------------------------------------
# library routine: PyTorch CPU float64 attention + autograd
# ----------------------------------------------------------------------------
def _torch_ref(q, k, v, do, scale, causal, attn_mask=None):
    import torch
    import torch.nn.functional as F
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=attn_mask, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float64))
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("causal,n,d", [(True, 128, 64), (False, 70, 64), (True, 70, 128), (False, 33, 16)])
def test_against_torch_cpu_fp64(causal, n, d):
    import torch
    rng = np.random.default_rng(99 + n)
    q, k, v, do = (_rand(rng, 1, 2, n, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o_t, dq_t, dk_t, dv_t = _torch_ref(q, k, v, do, scale, causal)
    o, lse = oracle.attention_forward(q, k, v, scale, causal=causal)
    g = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    assert _rel(o, o_t) < 1e-12
    assert _rel(g["o"], o_t) < 1e-12
    assert _rel(g["dq"], dq_t) < 1e-10
    assert _rel(g["dk"], dk_t) < 1e-10
    assert _rel(g["dv"], dv_t) < 1e-10
    # log-sum-exp from torch's own CPU attention kernel
    _, lse_t = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        *(torch.tensor(x) for x in (q, k, v)), 0.0, causal, scale=scale)[:2]
    assert np.max(np.abs(lse - lse_t.numpy())) < 1e-10
    assert np.max(np.abs(g["lse"] - lse_t.numpy())) < 1e-10


@pytest.mark.parametrize("causal", [True, False])
def test_sampled_outputs_against_torch_cpu_fp64(causal):
    """The blockwise, selected-output form of the backward (used where a full
    N x N oracle is too large) against PyTorch's fp64 attention with autograd,
    with blocks smaller than N and selected rows and keys on block edges."""
    rng = np.random.default_rng(4242 + causal)
    n, d, chunk = 150, 32, 64
    q, k, v, do = (_rand(rng, n, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    rows = np.array([0, 1, 63, 64, 65, 127, 128, 149])
    keys = np.array([0, 5, 63, 64, 100, 148, 149])
    g = oracle.attention_backward_sampled(q, k, v, do, scale, causal, rows, keys, chunk=chunk)
    o_t, dq_t, dk_t, dv_t = _torch_ref(q[None], k[None], v[None], do[None], scale, causal)
    o_t, dq_t, dk_t, dv_t = o_t[0], dq_t[0], dk_t[0], dv_t[0]
    assert _rel(g["o"], o_t[rows]) < 1e-12
    assert _rel(g["dq"], dq_t[rows]) < 1e-10
    assert _rel(g["dk"], dk_t[keys]) < 1e-10
    assert _rel(g["dv"], dv_t[keys]) < 1e-10
    assert _rel(g["D"], np.sum(do * o_t, -1)[rows]) < 1e-12
    full = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    assert np.max(np.abs(g["lse"] - full["lse"][rows])) < 1e-12


def test_sparse_against_torch_masked():
    import torch
    rng = np.random.default_rng(5)
    hq, nq, nkv, dqk, dv, topk = 3, 40, 40, 24, 16, 9
    q = _rand(rng, hq, nq, dqk)
    k = _rand(rng, nkv, dqk)
    v = _rand(rng, nkv, dv)
    do = _rand(rng, hq, nq, dv)
    from attn_inputs import make_topk_indices
    idx, cnt = make_topk_indices(rng, nq, nkv, topk)
    scale = 1.0 / math.sqrt(dqk)
    mask = torch.tensor(oracle.topk_allowed(idx, cnt, nkv))
    kk = np.broadcast_to(k, (hq, nkv, dqk)).copy()
    vv = np.broadcast_to(v, (hq, nkv, dv)).copy()
    o_t, dq_t, dk_t, dv_t = _torch_ref(q, kk, vv, do, scale, False, attn_mask=mask)
    o, lse = oracle.sparse_forward(q, k, v, idx, cnt, scale)
    g = oracle.sparse_backward(q, k, v, do, idx, cnt, scale)
    assert _rel(o, o_t) < 1e-12
    assert _rel(g["dq"], dq_t) < 1e-10
    assert _rel(g["dk"], dk_t.sum(0)) < 1e-10      # one K/V head shared by all query heads
    assert _rel(g["dv"], dv_t.sum(0)) < 1e-10


def test_sparse_equals_dense_masked():
    rng = np.random.default_rng(11)
    hq, n, dqk, dv, topk = 2, 50, 8, 8, 12
    q = _rand(rng, hq, n, dqk)
    k = _rand(rng, n, dqk)
    v = _rand(rng, n, dv)
    do = _rand(rng, hq, n, dv)
    from attn_inputs import make_topk_indices
    idx, cnt = make_topk_indices(rng, n, n, topk)
    scale = 0.3
    allowed = oracle.topk_allowed(idx, cnt, n)
    gs = oracle.sparse_backward(q, k, v, do, idx, cnt, scale)
    kk = np.broadcast_to(k, (hq, n, dqk))
    vv = np.broadcast_to(v, (hq, n, dv))
    gd = oracle.attention_backward(q, kk, vv, do, scale, allowed=allowed)
    assert _rel(gs["o"], gd["o"]) < 1e-12
    assert np.max(np.abs(gs["lse"] - gd["lse"])) < 1e-12
    assert _rel(gs["dq"], gd["dq"]) < 1e-12
    assert _rel(gs["dk"], gd["dk"].sum(0)) < 1e-12
    assert _rel(gs["dv"], gd["dv"].sum(0)) < 1e-12


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------
def test_single_key_closed_form():
    rng = np.random.default_rng(3)
    q, k, v, do = (_rand(rng, 2, 3, 1, 8) for _ in range(4))
    o, lse = oracle.attention_forward(q, k, v, 0.35)
    g = oracle.attention_backward(q, k, v, do, 0.35)
    assert np.array_equal(o, v)                     # one key: P = 1 exactly
    assert np.allclose(lse, 0.35 * np.sum(q * k, -1), atol=0, rtol=1e-15)
    assert np.allclose(g["dv"], do, rtol=0, atol=1e-15)
    assert np.max(np.abs(g["dq"])) < 1e-15 and np.max(np.abs(g["dk"])) < 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_equal_keys_give_uniform_average(causal):
    rng = np.random.default_rng(4)
    n, d = 9, 5
    q = _rand(rng, 1, 1, n, d)
    k = np.broadcast_to(_rand(rng, 1, 1, 1, d), (1, 1, n, d)).copy()
    v = _rand(rng, 1, 1, n, d)
    o, lse = oracle.attention_forward(q, k, v, 0.5, causal=causal)
    s0 = 0.5 * np.sum(q[0, 0] * k[0, 0, 0], -1)
    for i in range(n):
        cnt = i + 1 if causal else n
        assert np.allclose(o[0, 0, i], v[0, 0, :cnt].mean(0), rtol=1e-13, atol=1e-14)
        assert abs(lse[0, 0, i] - (s0[i] + math.log(cnt))) < 1e-13


def test_causal_special_rows():
    rng = np.random.default_rng(8)
    n, d = 12, 6
    q, k, v, do = (_rand(rng, 1, 1, n, d) for _ in range(4))
    g = oracle.attention_backward(q, k, v, do, 0.4, causal=True)
    # query 0 sees only key 0: P = 1, dS = dP - D = 0, so dQ_0 = 0
    assert np.max(np.abs(g["dq"][0, 0, 0])) < 1e-14
    # the last key is seen only by the last query
    p_last = math.exp(0.4 * float(q[0, 0, -1] @ k[0, 0, -1]) - g["lse"][0, 0, -1])
    dp_last = float(do[0, 0, -1] @ v[0, 0, -1])
    ds_last = p_last * (dp_last - g["D"][0, 0, -1])
    assert np.allclose(g["dk"][0, 0, -1], 0.4 * ds_last * q[0, 0, -1], rtol=1e-12, atol=1e-14)
    assert np.allclose(g["dv"][0, 0, -1], p_last * do[0, 0, -1], rtol=1e-12, atol=1e-14)


def test_lse_bounds_and_convex_hull():
    rng = np.random.default_rng(9)
    n, d = 20, 7
    q, k, v = (_rand(rng, 1, 2, n, d) for _ in range(3))
    for causal in (False, True):
        o, lse = oracle.attention_forward(q, k, v, 0.6, causal=causal)
        s = 0.6 * np.einsum("bhid,bhjd->bhij", q, k)
        for i in range(n):
            cnt = i + 1 if causal else n
            m = s[..., i, :cnt].max(-1)
            assert np.all(lse[..., i] >= m - 1e-12)
            assert np.all(lse[..., i] <= m + math.log(cnt) + 1e-12)
            lo = v[..., :cnt, :].min(-2)
            hi = v[..., :cnt, :].max(-2)
            assert np.all(o[..., i, :] >= lo - 1e-12) and np.all(o[..., i, :] <= hi + 1e-12)


# ----------------------------------------------------------------------------
# identities of the backward
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [False, True])
def test_backward_identities(causal):
    rng = np.random.default_rng(21 + causal)
    n, d, scale = 48, 16, 0.25
    q, k, v, do = (_rand(rng, 2, 2, n, d) for _ in range(4))
    allowed = oracle.causal_allowed(n, n) if causal else None
    s = oracle.scores(q, k, scale, allowed)
    p = oracle.softmax_rows(s)
    assert np.allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    if causal:
        assert np.all(p[..., ~oracle.causal_allowed(n, n)] == 0.0)
    g = oracle.attention_backward(q, k, v, do, scale, causal=causal)
    dp = do @ np.swapaxes(v, -1, -2)
    ds = p * (dp - g["D"][..., None])
    assert np.max(np.abs(ds.sum(-1))) < 1e-12
    # D = rowsum(P o dP) = rowsum(dO o O)
    assert np.allclose((p * dp).sum(-1), g["D"], rtol=1e-12, atol=1e-12)
    # sum_j dK_j = 0 and sum_j dV_j = sum_i dO_i
    assert np.max(np.abs(g["dk"].sum(-2))) < 1e-11
    assert np.allclose(g["dv"].sum(-2), do.sum(-2), rtol=1e-12, atol=1e-11)
    # sum Q o dQ = sum K o dK = sum dS o S (per head), sum V o dV = sum D
    sq = (q * g["dq"]).sum((-1, -2))
    sk = (k * g["dk"]).sum((-1, -2))
    sfin = np.where(np.isfinite(s), s, 0.0)
    assert np.allclose(sq, sk, rtol=1e-10, atol=1e-10)
    assert np.allclose(sq, (ds * sfin).sum((-1, -2)), rtol=1e-10, atol=1e-10)
    assert np.allclose((v * g["dv"]).sum((-1, -2)), g["D"].sum(-1), rtol=1e-10, atol=1e-10)


def test_stored_o_changes_only_D_path():
    """D taken from a given O: with the exact O nothing changes; with another O
    only D, dS, dQ and dK move, and dQ/dK move by exactly -scale*(dD)(P K) /
    -scale*P^T(dD Q)."""
    rng = np.random.default_rng(31)
    n, d, scale = 10, 4, 0.5
    q, k, v, do = (_rand(rng, 1, 1, n, d) for _ in range(4))
    g0 = oracle.attention_backward(q, k, v, do, scale, causal=True)
    g1 = oracle.attention_backward(q, k, v, do, scale, causal=True, o_for_D=g0["o"])
    for name in ("dq", "dk", "dv", "D"):
        assert np.array_equal(g0[name], g1[name])
    o2 = g0["o"] + 0.01 * _rand(rng, 1, 1, n, d)
    g2 = oracle.attention_backward(q, k, v, do, scale, causal=True, o_for_D=o2)
    assert np.array_equal(g0["dv"], g2["dv"])
    dD = np.sum(do * (o2 - g0["o"]), -1)                       # change of D per row
    p = oracle.softmax_rows(oracle.scores(q, k, scale, oracle.causal_allowed(n, n)))
    assert np.allclose(g2["dq"] - g0["dq"], -scale * dD[..., None] * (p @ k), atol=1e-13)
    assert np.allclose(g2["dk"] - g0["dk"], -scale * np.swapaxes(p, -1, -2) @ (dD[..., None] * q), atol=1e-13)


def test_empty_sparse_row_gives_zero():
    rng = np.random.default_rng(2)
    q = _rand(rng, 2, 3, 4)
    k = _rand(rng, 3, 4)
    v = _rand(rng, 3, 5)
    do = _rand(rng, 2, 3, 5)
    idx = np.array([[0, -1], [-1, -1], [0, 2]], dtype=np.int32)
    o, lse = oracle.sparse_forward(q, k, v, idx, None, 0.5)
    assert np.all(o[:, 1] == 0) and np.all(np.isneginf(lse[:, 1]))
    g = oracle.sparse_backward(q, k, v, do, idx, None, 0.5)
    assert np.all(g["dq"][:, 1] == 0)
    assert np.all(np.isfinite(g["dk"])) and np.all(np.isfinite(g["dv"]))
    assert np.all(g["dk"][1] == 0) and np.all(g["dv"][1] == 0)   # key 1 is never named


# ----------------------------------------------------------------------------
# planted mistakes must be caught by the pins above
# ----------------------------------------------------------------------------
def _fd_pin_passes():
    rng = np.random.default_rng(77)
    n, d = 5, 3
    q, k, v, do = (_rand(rng, 1, 1, n, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    g = oracle.attention_backward(q, k, v, do, scale, causal=True)
    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        fd = _fd_grad(lambda: _loss(q, k, v, do, scale, True), x)
        if not _rel(g[name], fd) < 1e-7:
            return False
    return True


def _torch_pin_passes():
    rng = np.random.default_rng(78)
    n, d = 16, 8
    q, k, v, do = (_rand(rng, 1, 1, n, d) for _ in range(4))
    scale = 1.0 / math.sqrt(d)
    o_t, dq_t, dk_t, dv_t = _torch_ref(q, k, v, do, scale, True)
    o, _ = oracle.attention_forward(q, k, v, scale, causal=True)
    g = oracle.attention_backward(q, k, v, do, scale, causal=True)
    return (_rel(o, o_t) < 1e-12 and _rel(g["dq"], dq_t) < 1e-10
            and _rel(g["dk"], dk_t) < 1e-10 and _rel(g["dv"], dv_t) < 1e-10)


_MUTANTS = {
    "softmax_grad_without_D": ("softmax_backward", lambda p, dp, D: p * dp),
    "softmax_grad_sign": ("softmax_backward", lambda p, dp, D: p * (dp + D[..., None])),
    "preprocess_wrong_operand": ("bwd_preprocess", lambda o, do: np.sum(np.asarray(do) * np.asarray(do), -1)),
    "causal_mask_off_by_one": ("causal_allowed", lambda nq, nk: np.arange(nk)[None, :] < np.arange(nq)[:, None] + 2),
    "scores_transposed_mask": ("causal_allowed", lambda nq, nk: np.arange(nk)[None, :] >= np.arange(nq)[:, None]),
    "scores_unscaled": ("scores", None),
    "lse_without_max": ("row_logsumexp", None),
}


@pytest.mark.parametrize("mutant", sorted(_MUTANTS))
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    name, fn = _MUTANTS[mutant]
    if mutant == "scores_unscaled":
        real = oa.scores
        fn = lambda q, k, scale, allowed=None: real(q, k, 1.0, allowed)  # noqa: E731
    if mutant == "lse_without_max":
        fn = lambda s: np.log(np.sum(np.exp(s), -1)) + 0.01  # noqa: E731
    assert _fd_pin_passes() and _torch_pin_passes()
    monkeypatch.setattr(oa, name, fn)
    assert not (_fd_pin_passes() and _torch_pin_passes()), f"mutant {mutant} survived"
