"""Shared helpers for the GPU-vs-oracle parity tests.

Tolerance rule: max |gpu - oracle| <= tol * RMS(oracle) over the compared
tensor, with tol = 2e-2 for bf16 q/k/v (fp32 state) and 1e-4 for fp32 inputs;
any non-finite value fails.  The final state is held to the same rule with
its own RMS.
"""
import sys

import numpy as np
import torch

TOL = {torch.bfloat16: 2e-2, torch.float32: 1e-4}


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_np(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().to("cpu")
        if x.dtype != torch.float64:
            x = x.to(torch.float32)
        return x.numpy().astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def rel_err(got, ref):
    got, ref = to_np(got), to_np(ref)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / rms)


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    say(f"  {name}: max|err|/rms = {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{name}: max|err|/rms = {e:.3e} > {tol:.0e}"
    return e


def assert_close_rounded(name, got, ref, tol):
    """bf16 outputs: each element may also carry its own bf16 rounding,
    |got - ref| <= tol * RMS(ref) + 2^-8 |ref|."""
    g, r = to_np(got), to_np(ref)
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    rms = float(np.sqrt(np.mean(r * r)))
    excess = np.abs(g - r) - 2.0 ** -8 * np.abs(r)
    e = float(excess.max() / rms)
    say(f"  {name}: max(|err| - 2^-8|ref|)/rms = {e:.3e} (tol {tol:.0e})")
    assert e <= tol, f"{name}: {e:.3e} > {tol:.0e}"
    return e


def gpu_available():
    return torch.cuda.is_available()
