"""Helpers shared by the GPU parity tests: moving bf16 bit patterns between
numpy and device tensors, and the parity metrics with their tolerances.

Tolerances (per output tensor, bf16 inputs):
  max |gpu - ref|            <= 2e-2 * max |ref|
  sum |gpu - ref| / sum |ref| <= 5e-3            (mean-abs relative error)
  log-sum-exp: max |gpu - ref| <= 1e-3 (absolute)
A reference that is exactly zero everywhere (dQ, dK when N = 1) is checked
absolutely: max |gpu| <= 1e-5.
Adversarial input regimes (wide_logits, late_spike) may pass a `floor`: the
same metrics of PyTorch's CPU bf16 attention on the same inputs against the
same oracle; the bound is then max(bar, 1.5 * floor), the noise-floor practice
of the flash_attention_cuda README's validation.
"""
import sys

import numpy as np

from attn_inputs import bf16_bits_to_f64, f32_to_bf16_bits

MAX_REL = 2e-2
MEAN_REL = 5e-3
LSE_ABS = 1e-3
ZERO_ABS = 1e-5
FLOOR_FACTOR = 1.5


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f64_to_dev_bf16(x: np.ndarray):
    return to_dev(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def from_dev(t) -> np.ndarray:
    """bf16 device tensor -> float64 numpy (exact)."""
    import torch
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
    return t.detach().cpu().numpy().astype(np.float64)


def metrics(gpu: np.ndarray, ref: np.ndarray):
    err = np.abs(gpu - ref)
    mx = float(np.max(np.abs(ref))) if ref.size else 0.0
    return {
        "max_err": float(np.max(err)) if err.size else 0.0,
        "max_ref": mx,
        "max_rel": float(np.max(err)) / mx if mx > 0 else float(np.max(err)) if err.size else 0.0,
        "mean_rel": float(np.sum(err)) / max(float(np.sum(np.abs(ref))), 1e-300),
    }


def assert_close(name, gpu, ref, floor=None):
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    if ref.size and float(np.max(np.abs(ref))) == 0.0:
        mx = float(np.max(np.abs(gpu)))
        say(f"  {name}: reference is exactly 0, max|gpu|={mx:.3e}")
        assert mx <= ZERO_ABS, (name, mx)
        return None
    m = metrics(gpu, ref)
    max_bar, mean_bar = MAX_REL, MEAN_REL
    if floor is not None:
        max_bar = max(max_bar, FLOOR_FACTOR * floor["max_rel"])
        mean_bar = max(mean_bar, FLOOR_FACTOR * floor["mean_rel"])
    say(f"  {name}: max_rel={m['max_rel']:.3e} (<= {max_bar:.2e}) mean_rel={m['mean_rel']:.3e} (<= {mean_bar:.2e})")
    assert m["max_rel"] <= max_bar, (name, m)
    assert m["mean_rel"] <= mean_bar, (name, m)
    return m


def torch_bf16_floor(q, k, v, do, scale, causal, ref):
    """Metrics of PyTorch's CPU bf16 attention (forward + autograd backward) on
    the same bf16 inputs against the oracle results `ref` (dict of float64)."""
    import torch
    import torch.nn.functional as F
    t = lambda x: torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).requires_grad_(True)  # noqa: E731
    tq, tk, tv = t(q), t(k), t(v)
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do, dtype=torch.float32).to(torch.bfloat16))
    got = {"o": o.detach().double().numpy(), "dq": tq.grad.double().numpy(),
           "dk": tk.grad.double().numpy(), "dv": tv.grad.double().numpy()}
    return {n: metrics(got[n], ref[n]) for n in got}


def assert_lse(gpu, ref):
    assert np.all(np.isfinite(gpu))
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    say(f"  lse: max_abs={err:.3e}")
    assert err <= LSE_ABS, err


class Accum:
    """The parity metrics of one output tensor accumulated piece by piece
    (e.g. head by head), so that a full-size tensor is never held twice."""

    def __init__(self, name):
        self.name = name
        self.err_sum = 0.0
        self.ref_sum = 0.0
        self.err_max = 0.0
        self.ref_max = 0.0
        self.n = 0

    def add(self, gpu, ref):
        assert gpu.shape == ref.shape, (self.name, gpu.shape, ref.shape)
        assert np.all(np.isfinite(gpu)), f"{self.name}: non-finite values"
        err = np.abs(gpu - ref)
        self.err_sum += float(np.sum(err))
        self.ref_sum += float(np.sum(np.abs(ref)))
        if err.size:
            self.err_max = max(self.err_max, float(np.max(err)))
            self.ref_max = max(self.ref_max, float(np.max(np.abs(ref))))
        self.n += gpu.size

    def check(self):
        if self.ref_max == 0.0:
            say(f"  {self.name}: reference is exactly 0, max|gpu|={self.err_max:.3e}")
            assert self.err_max <= ZERO_ABS, (self.name, self.err_max)
            return
        max_rel = self.err_max / self.ref_max
        mean_rel = self.err_sum / max(self.ref_sum, 1e-300)
        say(f"  {self.name}: {self.n} elements, max_rel={max_rel:.3e} (<= {MAX_REL:.0e}) "
            f"mean_rel={mean_rel:.3e} (<= {MEAN_REL:.0e})")
        assert max_rel <= MAX_REL, (self.name, max_rel)
        assert mean_rel <= MEAN_REL, (self.name, mean_rel)


class LseAccum:
    def __init__(self):
        self.err = 0.0

    def add(self, gpu, ref):
        assert np.all(np.isfinite(gpu))
        if ref.size:
            self.err = max(self.err, float(np.max(np.abs(gpu - ref))))

    def check(self):
        say(f"  lse: max_abs={self.err:.3e}")
        assert self.err <= LSE_ABS, self.err


# Exact identities of the backward (the attention-backward page, Appendix B,
# "Softmax Backward Derivation": rows of dS sum to zero, and D = rowsum(P o dP)
# = rowsum(dO o O)), over one head:
#   sum_j dK_j = 0,  sum_j dV_j = sum_i dO_i,  sum Q o dQ = sum K o dK,
#   sum V o dV = sum_i D_i.
# Each residual is divided by the random-walk size of its summands,
# sqrt(sum of their squares): per-element errors of relative size rho with
# no common sign move a sum by about rho times that, so the residuals of
# results within the parity bar (rho = 5e-3) stay below 5 rho = 2.5e-2 (the
# column identities are averaged over the head-dim columns, as an RMS).  A
# missing or zero tile of dQ, dK or dV, or a wrong mask, gives 0.1 to 1; a
# 2 % scale error in dQ or dK about 2e-2.
INV_BARS = {"sum_dk": 2.5e-2, "sum_dv": 2.5e-2, "qdq_kdk": 2.5e-2, "vdv_D": 2.5e-2}


def head_invariants(q, k, v, do, dq, dk, dv, D):
    """Residuals of the four identities for one head (float64 [N, d] arrays, D [N])."""
    def cols(s, ss):                            # RMS over columns of |sum| / sqrt(sum of squares)
        return float(np.sqrt(np.mean(s * s / np.maximum(ss, 1e-300))))

    def scalar(a, b):                           # sum a = sum b
        return abs(float(np.sum(a)) - float(np.sum(b))) / max(
            float(np.sqrt(np.sum(a * a) + np.sum(b * b))), 1e-300)

    return {
        "sum_dk": cols(dk.sum(0), (dk * dk).sum(0)),
        "sum_dv": cols(dv.sum(0) - do.sum(0), (dv * dv).sum(0) + (do * do).sum(0)),
        "qdq_kdk": scalar(q * dq, k * dk),
        "vdv_D": scalar(v * dv, D),
    }
