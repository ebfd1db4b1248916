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

Grouped value heads (page "How the New Flash Models Work...", section "The two
stacks, layer by layer": 16 key heads and 48 value heads in the Gated DeltaNet
layers; the state-size table of section "Linear attention..." counts one state
per value head): q and k may carry Hk heads while v, the gates and the states
carry H, a multiple of Hk.  Value head h uses q/k head h // (H // Hk), i.e.
each q/k head is repeated for its group of consecutive value heads before the
recurrence runs -- which is all that grouping means.
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


def build_sanitized(out: str) -> str:
    """The oracle with host AddressSanitizer + UndefinedBehaviorSanitizer
    (ROCm's clang, whose ASan runtime also serves the HIP library's sanitized
    build; serial: the OpenMP pragmas are left out).  For the sanitizer test."""
    clang = "/opt/rocm/llvm/bin/clang"
    tmp = out + ".tmp"
    subprocess.run([clang, "-std=c99", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-Wno-unknown-pragmas", _SRC,
                    "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


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
        lib.gdr_oracle_recurrence_backward.argtypes = [
            i64, p, i64, i64, i64, ctypes.c_int, p, p, p, p, p, p, ctypes.c_double, p, p,
            p, p, p, p, p, p, ctypes.c_int,
        ]
        lib.gdr_oracle_recurrence_backward.restype = ctypes.c_int
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


def _expand_groups(q, k, H):
    """q/k with Hk heads on axis -2 -> H heads, value head h taking q/k head
    h // (H // Hk)."""
    Hk = q.shape[-2]
    if Hk == H:
        return q, k
    if Hk < 1 or H % Hk:
        raise ValueError(f"{Hk} q/k heads do not divide {H} value heads")
    return np.repeat(q, H // Hk, axis=-2), np.repeat(k, H // Hk, axis=-2)


def recurrence(q, k, v, beta, log_alpha, *, initial_state=None, seq_bounds=None,
               scale: float = 1.0, num_threads: int = 0):
    """Run the sequential fp64 recurrence.

    Dense form:  q, k [B, T, Hk, dk]; v [B, T, H, dv]; beta [B, T, H];
                 log_alpha [B, T, H] (per-head decay) or [B, T, H, dk] (per-channel);
                 Hk divides H (Hk < H: grouped value heads, see the module text).
    Packed form: same with B == 1 and ``seq_bounds`` = the N+1 token offsets.
    initial_state [N, H, dv, dk] or None (zeros).

    Returns (out [B, T, H, dv], final_state [N, H, dv, dk]) as fp64 numpy arrays.
    """
    q, k, v, beta, log_alpha = (_f64(x) for x in (q, k, v, beta, log_alpha))
    initial_state = _f64(initial_state)
    if k.shape != q.shape or q.ndim != 4 or v.ndim != 4:
        raise ValueError("q and k must be [B, T, Hk, dk], v [B, T, H, dv]")
    q, k = _expand_groups(q, k, v.shape[2])
    bounds, per_channel = _check_prefill(q, k, v, beta, log_alpha, initial_state, seq_bounds)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = len(bounds) - 1
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


def _check_prefill(q, k, v, beta, log_alpha, initial_state, seq_bounds):
    """Shapes, gate form and sequence bounds shared by the forward and the
    backward entry; returns (bounds, per_channel)."""
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
    return bounds, per_channel


def recurrence_backward(q, k, v, beta, log_alpha, d_out, *, initial_state=None,
                        d_final_state=None, seq_bounds=None, scale: float = 1.0,
                        num_threads: int = 0):
    """Gradients of a scalar loss through :func:`recurrence`, given its
    gradients with respect to the outputs (``d_out`` [B, T, H, dv]) and to the
    final states (``d_final_state`` [N, H, dv, dk], None = zeros).

    The pages train these layers but print no backward pass; this is the
    chain rule applied to the recurrence's steps in reverse (the step list is
    in ``gdr_oracle.c``).  Grouped q/k heads: each value head's gradient with
    respect to its (repeated) q/k head is summed over the heads of the group,
    the adjoint of the repetition.

    Returns a dict of fp64 arrays: dq, dk (q's shape), dv (v's), dbeta
    (beta's), dlog_alpha (log_alpha's) and d_initial_state [N, H, dv, dk]
    (the gradient with respect to the initial state, whether or not one was
    passed: a missing initial state is a zero one).
    """
    q, k, v, beta, log_alpha, d_out = (_f64(x) for x in (q, k, v, beta, log_alpha, d_out))
    initial_state = _f64(initial_state)
    d_final_state = _f64(d_final_state)
    if k.shape != q.shape or q.ndim != 4 or v.ndim != 4:
        raise ValueError("q and k must be [B, T, Hk, dk], v [B, T, H, dv]")
    Hk = q.shape[2]
    qe, ke = _expand_groups(q, k, v.shape[2])
    bounds, per_channel = _check_prefill(qe, ke, v, beta, log_alpha, initial_state, seq_bounds)
    B, T, H, dk = qe.shape
    dv = v.shape[-1]
    N = len(bounds) - 1
    if d_out.shape != v.shape:
        raise ValueError(f"d_out shape {d_out.shape} != {v.shape}")
    if d_final_state is not None and d_final_state.shape != (N, H, dv, dk):
        raise ValueError(f"d_final_state shape {d_final_state.shape} != {(N, H, dv, dk)}")
    g = {
        "dq": np.zeros(qe.shape), "dk": np.zeros(qe.shape), "dv": np.zeros(v.shape),
        "dbeta": np.zeros(beta.shape), "dlog_alpha": np.zeros(log_alpha.shape),
        "d_initial_state": np.zeros((N, H, dv, dk)),
    }
    rc = _load().gdr_oracle_recurrence_backward(
        N, _ptr(bounds), H, dk, dv, per_channel, _ptr(qe), _ptr(ke), _ptr(v), _ptr(beta),
        _ptr(log_alpha), _ptr(initial_state), float(scale), _ptr(d_out), _ptr(d_final_state),
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dbeta"]), _ptr(g["dlog_alpha"]),
        _ptr(g["d_initial_state"]), int(num_threads),
    )
    if rc != 0:
        raise RuntimeError(f"oracle failed with code {rc}")
    if Hk != H:
        for name in ("dq", "dk"):
            g[name] = g[name].reshape(B, T, Hk, H // Hk, dk).sum(axis=3)
    return g


def decode(q, k, v, beta, log_alpha, state, *, scale: float = 1.0, num_threads: int = 0):
    """One token per sequence: q, k [N, Hk, dk]; v [N, H, dv]; beta [N, H];
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


def decode_tokens(q, k, v, beta, log_alpha, state_pool, *, num_tokens=None, num_commit=None,
                  state_slots=None, scale: float = 1.0, num_threads: int = 0):
    """Several tokens per sequence from a pool of state slots (speculative
    verify with replay of the accepted tokens: page "How the New Flash Models
    Work...", section "Decoding several tokens per pass"; page "Qwen3.8-Flash-
    Next and GLM-5.3-Flash share a 3:1 long-context pattern", section "GLM's
    serving design is explicitly disaggregated", which names ReplaySSM).

    q, k [N, K, Hk, dk]; v [N, K, H, dv]; beta [N, K, H]; log_alpha [N, K, H]
    or [N, K, H, dk]; state_pool [P, H, dv, dk]; num_tokens, num_commit,
    state_slots: length-N integer arrays or None (K; T_n; n).

    For each sequence n whose slot s = state_slots[n] lies in [0, P): with
    T = clamp(num_tokens[n], 0, K) and C = clamp(num_commit[n], 0, T), run the
    recurrence over its tokens 0..C-1 from state_pool[s], then over tokens
    C..T-1 from the state so reached; the outputs of all T tokens are written
    and state_pool[s] becomes the state after token C-1 (unchanged if C = 0).
    Sequences with a slot outside [0, P) are skipped.

    Returns (out [N, K, H, dv], written [N, K] bool, new_pool [P, H, dv, dk]);
    rows that are not written hold 0 in ``out``.
    """
    q, k, v, beta, log_alpha, pool = (_f64(x) for x in (q, k, v, beta, log_alpha, state_pool))
    N, K = q.shape[:2]
    H, dv = v.shape[2], v.shape[3]
    P = pool.shape[0]

    def ints(a, default):
        if a is None:
            return np.asarray(default, dtype=np.int64)
        if hasattr(a, "detach"):
            a = a.detach().cpu().numpy()
        return np.asarray(a, dtype=np.int64)

    slots = ints(state_slots, np.arange(N))
    T = np.clip(ints(num_tokens, np.full(N, K)), 0, K)
    C = np.clip(ints(num_commit, T), 0, T)
    out = np.zeros((N, K, H, dv))
    written = np.zeros((N, K), dtype=bool)
    new_pool = pool.copy()
    for n in range(N):
        s = int(slots[n])
        if s < 0 or s >= P or T[n] == 0:
            continue
        c, t = int(C[n]), int(T[n])
        tok = lambda a, lo, hi: a[n:n + 1, lo:hi]
        args = lambda lo, hi: [tok(a, lo, hi) for a in (q, k, v, beta, log_alpha)]
        S = pool[s:s + 1]
        if c > 0:
            o1, S = recurrence(*args(0, c), initial_state=S, scale=scale, num_threads=num_threads)
            out[n, :c] = o1[0]
            new_pool[s] = S[0]
        if t > c:
            o2, _ = recurrence(*args(c, t), initial_state=S, scale=scale, num_threads=num_threads)
            out[n, c:t] = o2[0]
        written[n, :t] = True
    return out, written, new_pool


def layer_prologue(x, conv_weight, a_logit, b_logit, *, num_qk_heads, head_dim_k, head_dim_v,
                   conv_state=None, seq_bounds=None, silu=False, qk_norm=True):
    """The layer prologue in fp64, written from its definition: for each
    sequence, the three inputs before its first token (its convolution state,
    or zeros) are put in front of its inputs and each channel is convolved
    causally with its four taps (page "Qwen3.8-Flash-Next and GLM-5.3-Flash
    share a 3:1 long-context pattern", section "Kimi Delta Attention extends
    recurrent memory control": a short convolution of kernel four; page "How
    the New Flash Models Work...", section "Serving: prefill and decode are
    different problems": the convolution state goes with the recurrent state):

        y_t[c] = sum_j w[c, j] x_{t-3+j}[c];  optionally y <- y * sigmoid(y);
        q, k, v = the channel groups of y; optionally q, k <- q/|q|, k/|k| per head;
        beta = sigmoid(b);  log alpha = -softplus(a) = -log(1 + e^a).

    The new state of a sequence is the last three rows of its padded inputs.
    x [B, T, C]; conv_weight [C, 4]; a_logit [B, T, H(, dk)]; b_logit [B, T, H];
    conv_state [N, 3, C] or None; seq_bounds (packed, B == 1) or None.
    Returns (q, k, v, beta, log_alpha, new_state) as fp64 arrays.
    """
    x, w, a, b = (_f64(t) for t in (x, conv_weight, a_logit, b_logit))
    st = _f64(conv_state)
    B, T, C = x.shape
    Hk, dk, dv = num_qk_heads, head_dim_k, head_dim_v
    H = b.shape[-1]
    if C != 2 * Hk * dk + H * dv:
        raise ValueError("channel count does not match the head sizes")
    bounds = np.arange(B + 1) * T if seq_bounds is None else np.asarray(seq_bounds, dtype=np.int64)
    N = len(bounds) - 1
    rows = x.reshape(B * T, C)
    y = np.zeros_like(rows)
    new_state = np.zeros((N, 3, C))
    for n in range(N):
        lo, hi = int(bounds[n]), int(bounds[n + 1])
        prev = st[n] if st is not None else np.zeros((3, C))
        padded = np.concatenate([prev, rows[lo:hi]], axis=0)     # padded[i] = input at position lo - 3 + i
        for t in range(hi - lo):
            y[lo + t] = sum(w[:, j] * padded[t + j] for j in range(4))
        new_state[n] = padded[-3:]
    if silu:
        y = y / (1.0 + np.exp(-y))
    y = y.reshape(B, T, C)
    q = y[..., :Hk * dk].reshape(B, T, Hk, dk)
    k = y[..., Hk * dk:2 * Hk * dk].reshape(B, T, Hk, dk)
    v = y[..., 2 * Hk * dk:].reshape(B, T, H, dv)
    if qk_norm:
        def unit(z):
            nrm = np.sqrt((z * z).sum(-1, keepdims=True))
            return np.where(nrm > 0, z / np.where(nrm > 0, nrm, 1.0), 0.0)
        q, k = unit(q), unit(k)
    beta = 1.0 / (1.0 + np.exp(-b))
    log_alpha = -np.logaddexp(0.0, a)
    return q, k, v, beta, log_alpha, new_state
