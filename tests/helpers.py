"""Shared helpers of the test-suite: tolerances, error metrics, bf16 plumbing."""
from __future__ import annotations

import numpy as np

from block_sparse_masked_opr_amd import inputs as I

# Acceptance bar for floating-point results against the fp64 oracle:
# max |x - ref| <= 2e-2 and sum|x - ref| / sum|ref| <= 5e-3.
MAX_ABS = 2e-2
MEAN_REL = 5e-3


def errors(x: np.ndarray, ref: np.ndarray):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.abs(x - ref)
    max_abs = float(d.max()) if d.size else 0.0
    denom = float(np.abs(ref).sum())
    mean_rel = float(d.sum() / denom) if denom > 0 else float(d.sum())
    return max_abs, mean_rel


def assert_close(name: str, x, ref, max_abs=MAX_ABS, mean_rel=MEAN_REL):
    ma, mr = errors(x, ref)
    print(f"  {name}: max_abs={ma:.3e} mean_rel={mr:.3e}", flush=True)
    assert ma <= max_abs and mr <= mean_rel, f"{name}: max_abs={ma:.3e} mean_rel={mr:.3e}"


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return I.bf16_bits_to_f32(bits).astype(np.float64)


def to_device_bf16(bits: np.ndarray, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_device_bf16(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
