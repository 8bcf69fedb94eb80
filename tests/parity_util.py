"""Shared helpers for the GPU parity tests (no GPU code here)."""
import sys

import numpy as np
import torch

# Bars from the workload definitions: max |x - x_ref| / RMS(x_ref), per tensor.
TOL_F32 = 1e-4
TOL_BF16 = 3e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_max_err(x, ref):
    """max |x - ref| / sqrt(mean(ref^2)) in fp64; inf when x has a non-finite value."""
    x = np.asarray(x.detach().cpu().to(torch.float64) if isinstance(x, torch.Tensor) else x,
                   dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    if not np.isfinite(x).all():
        return float("inf")
    rms = np.sqrt(np.mean(ref * ref))
    if rms == 0.0:
        return float(np.abs(x - ref).max())
    return float(np.abs(x - ref).max() / rms)


def tol_for(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def take_sequences(inp, pairs):
    """Gather (b, h) sequences into a [n, T, 1, d] batch (CPU tensors)."""
    out = {}
    for name in ("q", "k", "v", "log_alpha", "b", "w"):
        x = inp[name]
        out[name] = torch.stack([x[b, :, h] for b, h in pairs])[:, :, None].contiguous()
    s0 = inp.get("s0")
    out["s0"] = None if s0 is None else torch.stack([s0[b, h] for b, h in pairs])[:, None].contiguous()
    return out


def to_dev(inp, dev="cuda"):
    return {n: (None if x is None else x.to(dev).contiguous()) for n, x in inp.items()}


class ErrAccum:
    """The whole-tensor parity metric built up over pieces of a tensor: max |x - x_ref| over
    every piece, divided by the RMS of x_ref over every piece (fp64); inf once any piece holds
    a non-finite value."""

    def __init__(self):
        self.maxabs = 0.0
        self.sumsq = 0.0
        self.n = 0
        self.finite = True

    def add(self, x, ref):
        x = np.asarray(x.detach().cpu().to(torch.float64) if isinstance(x, torch.Tensor) else x,
                       dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert x.shape == ref.shape, (x.shape, ref.shape)
        if not np.isfinite(x).all():
            self.finite = False
            return
        self.maxabs = max(self.maxabs, float(np.abs(x - ref).max()) if x.size else 0.0)
        self.sumsq += float(np.sum(ref * ref))
        self.n += ref.size

    def value(self):
        if not self.finite:
            return float("inf")
        rms = np.sqrt(self.sumsq / max(self.n, 1))
        return self.maxabs / rms if rms > 0 else self.maxabs
