"""Helpers shared by the GPU parity tests: moving bf16 bit patterns between
numpy and device tensors, and the parity metrics with their tolerances.

Tolerances (per output tensor, bf16 inputs):
  max |gpu - ref|            <= 2e-2 * max |ref|
  sum |gpu - ref| / sum |ref| <= 5e-3            (mean-abs relative error)
  log-sum-exp: max |gpu - ref| <= 1e-3 (absolute)
"""
import sys

import numpy as np

from attn_inputs import bf16_bits_to_f64, f32_to_bf16_bits

MAX_REL = 2e-2
MEAN_REL = 5e-3
LSE_ABS = 1e-3


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


def assert_close(name, gpu, ref):
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite values"
    m = metrics(gpu, ref)
    say(f"  {name}: max_rel={m['max_rel']:.3e} mean_rel={m['mean_rel']:.3e}")
    assert m["max_rel"] <= MAX_REL, (name, m)
    assert m["mean_rel"] <= MEAN_REL, (name, m)
    return m


def assert_lse(gpu, ref):
    assert np.all(np.isfinite(gpu))
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    say(f"  lse: max_abs={err:.3e}")
    assert err <= LSE_ABS, err
