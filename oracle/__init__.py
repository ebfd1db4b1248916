"""fp64 CPU oracle for the gated delta-rule recurrence -- TEST INFRASTRUCTURE.

Only the test-suite, the package smoke check and the benchmark's CPU-baseline
leg import this module.  It wraps ``gdr_oracle.c`` (plain C, fp64, one token at
a time) through ctypes and shares nothing with the HIP library.

The recurrence follows page "How the New Flash Models Work: Inside
GLM-5.3-Flash and Qwen3.8-Flash-Next", section "Linear attention: a fixed-size
memory in place of the cache" (the Gated DeltaNet and Kimi Delta Attention
equations); see the C file's header for the step order.

Every input is converted to fp64 exactly (bf16 and fp32 values are exactly
representable), so the oracle sees the same numbers as the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "libgdr_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.gdr_oracle_recurrence.argtypes = [
            i64, p, i64, i64, i64, ctypes.c_int, p, p, p, p, p, p, ctypes.c_double, p, p, ctypes.c_int,
        ]
        lib.gdr_oracle_recurrence.restype = ctypes.c_int
        lib.gdr_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().gdr_oracle_max_threads())


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: go through float32 (exact for bf16/fp32), then fp64
        import torch

        a = a.detach().to("cpu")
        if a.dtype != torch.float64:
            a = a.to(torch.float32)
        a = a.numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(q, k, v, beta, log_alpha, *, initial_state=None, seq_bounds=None,
               scale: float = 1.0, num_threads: int = 0):
    """Run the sequential fp64 recurrence.

    Dense form:  q, k [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
                 log_alpha [B, T, H] (per-head decay) or [B, T, H, dk] (per-channel).
    Packed form: same with B == 1 and ``seq_bounds`` = the N+1 token offsets.
    initial_state [N, H, dv, dk] or None (zeros).

    Returns (out [B, T, H, dv], final_state [N, H, dv, dk]) as fp64 numpy arrays.
    """
    q, k, v, beta, log_alpha = (_f64(x) for x in (q, k, v, beta, log_alpha))
    initial_state = _f64(initial_state)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape[:3] != (B, T, H) or beta.shape != (B, T, H):
        raise ValueError("shape mismatch among q/k/v/beta")
    if log_alpha.shape == (B, T, H):
        per_channel = 0
    elif log_alpha.shape == (B, T, H, dk):
        per_channel = 1
    else:
        raise ValueError(f"log_alpha shape {log_alpha.shape} fits neither gate form")
    if seq_bounds is None:
        bounds = np.arange(B + 1, dtype=np.int64) * T
    else:
        if B != 1:
            raise ValueError("packed sequences need B == 1")
        bounds = np.ascontiguousarray(np.asarray(seq_bounds, dtype=np.int64))
        if bounds[0] != 0 or bounds[-1] != T or np.any(np.diff(bounds) < 0):
            raise ValueError("seq_bounds must rise from 0 to T")
    N = len(bounds) - 1
    if initial_state is not None and initial_state.shape != (N, H, dv, dk):
        raise ValueError(f"initial_state shape {initial_state.shape} != {(N, H, dv, dk)}")
    out = np.zeros((B, T, H, dv), dtype=np.float64)
    final = np.zeros((N, H, dv, dk), dtype=np.float64)
    rc = _load().gdr_oracle_recurrence(
        N, _ptr(bounds), H, dk, dv, per_channel, _ptr(q), _ptr(k), _ptr(v), _ptr(beta),
        _ptr(log_alpha), _ptr(initial_state), float(scale), _ptr(out), _ptr(final),
        int(num_threads),
    )
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    return out, final


def decode(q, k, v, beta, log_alpha, state, *, scale: float = 1.0, num_threads: int = 0):
    """One token per sequence: q, k [N, H, dk]; v [N, H, dv]; beta [N, H];
    log_alpha [N, H] or [N, H, dk]; state [N, H, dv, dk].
    Returns (out [N, H, dv], new_state) -- the oracle recurrence with T = 1."""
    q, k, v, beta, log_alpha = (_f64(x) for x in (q, k, v, beta, log_alpha))
    N = q.shape[0]
    out, final = recurrence(
        q.reshape(N, 1, *q.shape[1:]), k.reshape(N, 1, *k.shape[1:]),
        v.reshape(N, 1, *v.shape[1:]), beta.reshape(N, 1, *beta.shape[1:]),
        log_alpha.reshape(N, 1, *log_alpha.shape[1:]), initial_state=state,
        scale=scale, num_threads=num_threads,
    )
    return out[:, 0], final
