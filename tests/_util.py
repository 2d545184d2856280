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
