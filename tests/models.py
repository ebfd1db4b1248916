"""Independent fp64 numpy models used only to pin the oracle (test code).

None of these shares code with the oracle (C, token-by-token, row by row) or
with the HIP path.  Each one reaches the recurrence's result by a different
route:

* ``product_form`` -- the equation written as a product of dense d_k x d_k
  transition matrices, page "How the New Flash Models Work: Inside
  GLM-5.3-Flash and Qwen3.8-Flash-Next", section "Linear attention: a
  fixed-size memory in place of the cache", KDA equation:
  S_t = S_{t-1} A_t + beta_t v_t k_t^T with A_t = Diag(alpha_t)(I - beta_t k_t k_t^T),
  unrolled into S_T = S_0 A_1...A_T + sum_t beta_t v_t k_t^T A_{t+1}...A_T.
* ``gdn_equation`` -- the Gated DeltaNet equation of the same section taken
  literally: S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
* ``chunked`` -- the chunk-parallel (UT / WY) form the GPU kernels implement:
  inside a chunk, U = (I + A)^-1 diag(beta) (V - X) with
  A = strict_tril(diag(beta) (K*e^g)(K*e^-g)^T), then
  O = (Q*e^g) S0^T + tril((Q*e^g)(K*e^-g)^T) U and
  S_C = S0 Diag(e^{g_C}) + U^T (K*e^{g_C - g}).  This is algebra derived from
  the KDA equation, not printed on the pages; it is pinned here against the
  oracle so the kernels' algorithm is checked before any kernel exists.
"""
from __future__ import annotations

import numpy as np


def _alpha_vec(log_alpha_t, dk):
    la = np.asarray(log_alpha_t, dtype=np.float64)
    return np.exp(la) * np.ones(dk) if la.ndim == 0 else np.exp(la)


def product_form(q, k, v, beta, log_alpha, S0=None):
    """Single sequence, single head: q, k [T, dk]; v [T, dv]; beta [T];
    log_alpha [T] or [T, dk].  Returns (O [T, dv], S_T [dv, dk])."""
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dv, dk)) if S0 is None else np.asarray(S0, dtype=np.float64)
    A = []
    for t in range(T):
        a = _alpha_vec(log_alpha[t], dk)
        A.append(np.diag(a) @ (np.eye(dk) - beta[t] * np.outer(k[t], k[t])))

    def chain(lo, hi):  # A_lo ... A_{hi-1}
        M = np.eye(dk)
        for t in range(lo, hi):
            M = M @ A[t]
        return M

    O = np.zeros((T, dv))
    S = None
    for t_end in range(1, T + 1):
        S = S0 @ chain(0, t_end)
        for t in range(t_end):
            S = S + beta[t] * np.outer(v[t], k[t]) @ chain(t + 1, t_end)
        O[t_end - 1] = S @ q[t_end - 1]
    if S is None:
        S = S0.copy()
    return O, S


def gdn_equation(q, k, v, beta, log_alpha, S0=None):
    """Scalar-decay equation taken literally; log_alpha [T]."""
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for t in range(T):
        alpha = np.exp(log_alpha[t])
        S = alpha * S @ (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) + beta[t] * np.outer(v[t], k[t])
        O[t] = S @ q[t]
    return O, S


def chunked(q, k, v, beta, log_alpha, S0=None, chunk=16):
    """Chunked UT-transform form; single sequence and head.  A partial last
    chunk is simply shorter.  log_alpha [T] (per head) or [T, dk]."""
    T, dk = k.shape
    dv = v.shape[1]
    la = np.asarray(log_alpha, dtype=np.float64)
    if la.ndim == 1:
        la = np.repeat(la[:, None], dk, axis=1)
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        K, Q, V, b = k[c0:c1], q[c0:c1], v[c0:c1], beta[c0:c1]
        g = np.cumsum(la[c0:c1], axis=0)  # inclusive, per channel
        Kt, Kh, Qt = K * np.exp(g), K * np.exp(-g), Q * np.exp(g)
        Kend = K * np.exp(g[-1] - g)
        n = c1 - c0
        A = np.tril(b[:, None] * (Kt @ Kh.T), -1)
        M = np.tril(Qt @ Kh.T)
        X = Kt @ S.T
        U = np.linalg.solve(np.eye(n) + A, b[:, None] * (V - X))
        O[c0:c1] = Qt @ S.T + M @ U
        S = S * np.exp(g[-1])[None, :] + U.T @ Kend
    return O, S
