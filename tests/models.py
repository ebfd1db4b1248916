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
* ``chunked_backward`` -- the gradients of that chunked form, in the
  arrangement the backward kernels use: a forward pass over chunks keeping
  each chunk's incoming state, a reverse pass over chunks carrying the state
  gradient (its recurrence, dS_prev = dS_C Diag(e^{g_C}) + dO^T (Q*e^g) +
  dU^T W with dU = M^T dO + K_end dS_C^T and W = -(I + A)^-1 diag(beta)(K*e^g),
  needs no forward state), then every chunk's input gradients from its two
  states alone, with the Gram-like products taken against operands shifted by
  a per-channel reference exponent m.  Pinned against the oracle's backward.
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


def chunked_backward(q, k, v, beta, log_alpha, d_out, S0=None, d_final=None, chunk=16, scale=1.0):
    """Gradients of ``scale``-scaled :func:`chunked` for one sequence and head.

    Returns dict dq, dk [T, dk]; dv [T, dv]; dbeta [T]; dlog_alpha like
    log_alpha; d_initial_state [dv, dk].
    """
    T, dk = k.shape
    dv = v.shape[1]
    la_in = np.asarray(log_alpha, dtype=np.float64)
    la = np.repeat(la_in[:, None], dk, axis=1) if la_in.ndim == 1 else la_in
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    bounds = [(c0, min(T, c0 + chunk)) for c0 in range(0, T, chunk)]

    def operands(c0, c1):
        K, Q, b = k[c0:c1], q[c0:c1], beta[c0:c1]
        g = np.cumsum(la[c0:c1], axis=0)
        n = c1 - c0
        m = 0.5 * (g[0] + g[-1])                        # per-channel reference
        Kts, Khs, Qts = K * np.exp(g - m), K * np.exp(m - g), Q * np.exp(g - m)
        Tm = np.linalg.inv(np.eye(n) + np.tril(b[:, None] * (Kts @ Khs.T), -1))
        M = np.tril(Qts @ Khs.T)
        Kta, Qt, Kend = K * np.exp(g), Q * np.exp(g), K * np.exp(g[-1] - g)
        W = -(Tm * b[None, :]) @ Kta                    # Wn = -T diag(beta) K e^g
        return dict(K=K, Q=Q, b=b, g=g, m=m, Kts=Kts, Khs=Khs, Qts=Qts, T=Tm, M=M,
                    Kta=Kta, Qt=Qt, Kend=Kend, Wn=W, D=np.exp(g[-1]))

    # forward over chunks: each chunk's incoming state
    starts = []
    for c0, c1 in bounds:
        op = operands(c0, c1)
        starts.append(S.copy())
        U = op["T"] @ (op["b"][:, None] * v[c0:c1]) + op["Wn"] @ S.T
        S = S * op["D"][None, :] + U.T @ op["Kend"]

    # reverse over chunks: state gradient at each chunk's end
    dS = np.zeros((dv, dk)) if d_final is None else np.array(d_final, dtype=np.float64)
    ends = [None] * len(bounds)
    for ci in range(len(bounds) - 1, -1, -1):
        c0, c1 = bounds[ci]
        op = operands(c0, c1)
        ends[ci] = dS.copy()
        dO = scale * d_out[c0:c1]
        dU = op["M"].T @ dO + op["Kend"] @ dS.T
        dS = dS * op["D"][None, :] + dO.T @ op["Qt"] + dU.T @ op["Wn"]
    d_initial = dS

    # every chunk from its two states
    g_out = dict(dq=np.zeros((T, dk)), dk=np.zeros((T, dk)), dv=np.zeros((T, dv)),
                 dbeta=np.zeros(T), dla=np.zeros((T, dk)))
    for ci, (c0, c1) in enumerate(bounds):
        op = operands(c0, c1)
        S0c, dSC = starts[ci], ends[ci]
        b, g, m, Tm, M = op["b"], op["g"], op["m"], op["T"], op["M"]
        dO = scale * d_out[c0:c1]
        Y = v[c0:c1] - op["Kta"] @ S0c.T
        U = Tm @ (b[:, None] * Y)
        dU = M.T @ dO + op["Kend"] @ dSC.T
        Z = Tm.T @ dU
        dY = b[:, None] * Z
        dbeta = (Z * Y).sum(axis=1)
        dT = dU @ (b[:, None] * Y).T
        dA = np.tril(-(Tm.T @ dT @ Tm.T), -1)
        gram = op["Kts"] @ op["Khs"].T
        dbeta = dbeta + (dA * gram).sum(axis=1)
        dAb = b[:, None] * dA
        dM = np.tril(dO @ U.T)
        eg, egm, emg = np.exp(g), np.exp(g - m), np.exp(m - g)
        dQ = (dO @ S0c) * eg + (dM @ op["Khs"]) * egm
        gK1 = -(dY @ S0c) * eg + (dAb @ op["Khs"]) * egm
        gK2 = (dM.T @ op["Qts"] + dAb.T @ op["Kts"]) * emg
        gK3 = (U @ dSC) * np.exp(g[-1] - g)
        K, Q = op["K"], op["Q"]
        dg = K * (gK1 - gK2 - gK3) + Q * dQ
        dg[-1] += (gK3 * K).sum(axis=0) + (dSC * S0c).sum(axis=0) * op["D"]
        g_out["dq"][c0:c1] = dQ
        g_out["dk"][c0:c1] = gK1 + gK2 + gK3
        g_out["dv"][c0:c1] = dY
        g_out["dbeta"][c0:c1] = dbeta
        g_out["dla"][c0:c1] = np.cumsum(dg[::-1], axis=0)[::-1]   # reverse cumulative sum
    dla = g_out.pop("dla")
    g_out["dlog_alpha"] = dla.sum(axis=1) if la_in.ndim == 1 else dla
    g_out["d_initial_state"] = d_initial
    return g_out
