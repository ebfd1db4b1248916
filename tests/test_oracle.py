"""Pins for the fp64 oracle (CPU only).

The pages print no numerical example for the recurrence, so the oracle is
pinned by hand-worked cases derived from the printed equations
(tests/golden/), by special cases with closed forms or textbook equivalents,
by an independent brute-force product form, and by structural invariants the
pages state (erase-then-write; KDA generalises Gated DeltaNet).
"""
import json
import os

import numpy as np
import pytest

import oracle
import models

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
rng0 = np.random.default_rng(1234)


def _rand_case(T, dk, dv, H=1, B=1, per_channel=False, seed=0, unit_keys=True, s0=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal((B, T, H))))
    shape = (B, T, H, dk) if per_channel else (B, T, H)
    log_alpha = -np.log1p(np.exp(r.standard_normal(shape)))
    S0 = 0.5 * r.standard_normal((B, H, dv, dk)) if s0 else None
    return q, k, v, beta, log_alpha, S0


# ---------------------------------------------------------------- golden ----
@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_worked_2x2.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_worked_examples(case):
    k = np.array(case["k"])[None, :, None, :]
    q = np.array(case["q"])[None, :, None, :]
    v = np.array(case["v"])[None, :, None, :]
    beta = np.array(case["beta"])[None, :, None]
    la = np.log(np.array(case["alpha"]))[None, :, None, :]
    S0 = np.array(case["S0"])[None, None]
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    np.testing.assert_allclose(out[0, :, 0], np.array(case["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(fin[0, 0], np.array(case["final_state"]), rtol=0, atol=1e-14)
    # the same case through the per-head gate form when all channels share alpha
    alpha = np.array(case["alpha"])
    if np.all(alpha[:, :1] == alpha):
        out2, fin2 = oracle.recurrence(q, k, v, beta, la[..., 0], initial_state=S0)
        np.testing.assert_allclose(out2[0, :, 0], np.array(case["out"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(fin2[0, 0], np.array(case["final_state"]), rtol=0, atol=1e-14)


# ------------------------------------------------------ special cases ----
@pytest.mark.parametrize("per_channel", [False, True])
def test_p1_no_write_no_decay_keeps_state(per_channel):
    q, k, v, beta, la, S0 = _rand_case(9, 8, 6, H=2, per_channel=per_channel, seed=1)
    beta[:] = 0.0
    la[:] = 0.0
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    assert np.array_equal(fin, S0)
    expect = np.einsum("hij,bthj->bthi", S0[0], q)
    np.testing.assert_allclose(out, expect, rtol=0, atol=1e-15)


@pytest.mark.parametrize("per_channel", [False, True])
def test_p2_erase_then_write_recalls_value(per_channel):
    """Unit-norm key and beta = 1: the written key recalls exactly its value
    (the erase factor removes the old association first)."""
    q, k, v, beta, la, S0 = _rand_case(12, 16, 8, H=3, per_channel=per_channel, seed=2)
    beta[:] = 1.0
    state = S0
    for t in range(k.shape[1]):
        _, state = oracle.recurrence(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], beta[:, t:t + 1],
                                     la[:, t:t + 1], initial_state=state)
        recalled = np.einsum("hij,hj->hi", state[0], k[0, t])
        np.testing.assert_allclose(recalled, v[0, t], rtol=0, atol=1e-13)


def test_p3_equal_channel_kda_is_gdn_equation():
    q, k, v, beta, la, S0 = _rand_case(10, 8, 5, H=2, per_channel=False, seed=3)
    la_kda = np.repeat(la[..., None], 8, axis=-1)
    out_kda, fin_kda = oracle.recurrence(q, k, v, beta, la_kda, initial_state=S0)
    out_gdn, fin_gdn = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    for h in range(2):
        O, S = models.gdn_equation(q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], la[0, :, h], S0[0, h])
        np.testing.assert_allclose(out_kda[0, :, h], O, rtol=0, atol=1e-13)
        np.testing.assert_allclose(fin_kda[0, h], S, rtol=0, atol=1e-13)
        np.testing.assert_allclose(out_gdn[0, :, h], O, rtol=0, atol=1e-13)
        np.testing.assert_allclose(fin_gdn[0, h], S, rtol=0, atol=1e-13)


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_p4_brute_force_product_form(per_channel, T):
    q, k, v, beta, la, S0 = _rand_case(T, 6, 4, H=2, per_channel=per_channel, seed=10 + T,
                                       unit_keys=False)
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    for h in range(2):
        O, S = models.product_form(q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], la[0, :, h], S0[0, h])
        np.testing.assert_allclose(out[0, :, h], O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], S, rtol=0, atol=1e-12)


def test_p5_reduces_to_causal_linear_attention():
    """alpha = 1, beta = 1, orthonormal keys, zero state: each key is written
    once and never disturbed, so o_t = sum_{i<=t} (q_t . k_i) v_i and
    S_T = V^T K -- plain (additive) causal linear attention."""
    T, dk, dv = 7, 12, 5
    r = np.random.default_rng(5)
    Kq, _ = np.linalg.qr(r.standard_normal((dk, T)))
    K = Kq.T                      # T orthonormal rows
    Q = r.standard_normal((T, dk))
    V = r.standard_normal((T, dv))
    out, fin = oracle.recurrence(Q[None, :, None], K[None, :, None], V[None, :, None],
                                 np.ones((1, T, 1)), np.zeros((1, T, 1)))
    np.testing.assert_allclose(out[0, :, 0], np.tril(Q @ K.T) @ V, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fin[0, 0], V.T @ K, rtol=0, atol=1e-13)


@pytest.mark.parametrize("per_channel", [False, True])
def test_p6_pure_decay_closed_form(per_channel):
    q, k, v, beta, la, S0 = _rand_case(11, 8, 4, H=2, per_channel=per_channel, seed=6)
    beta[:] = 0.0
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    g = np.cumsum(la, axis=1)  # [1, T, H(, dk)]
    for h in range(2):
        for t in range(11):
            dec = np.exp(g[0, t, h]) * np.ones(8)
            np.testing.assert_allclose(out[0, t, h], S0[0, h] @ (dec * q[0, t, h]), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(fin[0, h], S0[0, h] * (np.exp(g[0, -1, h]) * np.ones(8))[None, :],
                                   rtol=1e-14, atol=1e-16)


def test_p7_structure_linear_affine_row_independent():
    q, k, v, beta, la, S0 = _rand_case(9, 8, 6, H=2, per_channel=True, seed=7)
    # linear in V when S0 = 0
    o1, s1 = oracle.recurrence(q, k, v, beta, la)
    o2, s2 = oracle.recurrence(q, k, 2.5 * v, beta, la)
    np.testing.assert_allclose(o2, 2.5 * o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s2, 2.5 * s1, rtol=1e-13, atol=1e-14)
    # affine in S0: f(S0) = f(0) + (f(S0, v=0))
    oa, sa = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    ob, sb = oracle.recurrence(q, k, np.zeros_like(v), beta, la, initial_state=S0)
    np.testing.assert_allclose(oa, o1 + ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sa, s1 + sb, rtol=0, atol=1e-13)
    # value channels (rows of S) evolve independently: permuting v permutes rows
    perm = np.array([3, 0, 5, 1, 4, 2])
    op, sp = oracle.recurrence(q, k, v[..., perm], beta, la, initial_state=S0[:, :, perm])
    np.testing.assert_allclose(op, oa[..., perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sp, sa[:, :, perm], rtol=0, atol=1e-14)


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 16, 64])
def test_p8_chunked_algebra_matches_oracle(per_channel, chunk):
    T = 37 if chunk <= 16 else 150
    q, k, v, beta, la, S0 = _rand_case(T, 16, 12, H=1, per_channel=per_channel, seed=8 + chunk)
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    O, S = models.chunked(q[0, :, 0], k[0, :, 0], v[0, :, 0], beta[0, :, 0], la[0, :, 0], S0[0, 0], chunk=chunk)
    np.testing.assert_allclose(O, out[0, :, 0], rtol=0, atol=1e-11)
    np.testing.assert_allclose(S, fin[0, 0], rtol=0, atol=1e-11)


@pytest.mark.parametrize("per_channel", [False, True])
def test_p9_continuation(per_channel):
    q, k, v, beta, la, S0 = _rand_case(23, 8, 8, H=2, per_channel=per_channel, seed=9)
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    T1 = 10
    o_a, s_a = oracle.recurrence(q[:, :T1], k[:, :T1], v[:, :T1], beta[:, :T1], la[:, :T1], initial_state=S0)
    o_b, s_b = oracle.recurrence(q[:, T1:], k[:, T1:], v[:, T1:], beta[:, T1:], la[:, T1:], initial_state=s_a)
    np.testing.assert_allclose(np.concatenate([o_a, o_b], axis=1), out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(s_b, fin, rtol=0, atol=1e-13)
    # token-by-token decode equals the prefill
    state = S0
    for t in range(23):
        o_t, state = oracle.decode(q[:, t], k[:, t], v[:, t], beta[:, t], la[:, t], state)
        np.testing.assert_allclose(o_t, out[:, t], rtol=0, atol=1e-13)
    np.testing.assert_allclose(state, fin, rtol=0, atol=1e-13)


def test_p10_packed_equals_separate_runs():
    lens = [5, 0, 13, 1, 9]
    T = sum(lens)
    q, k, v, beta, la, _ = _rand_case(T, 8, 4, H=3, per_channel=True, seed=10)
    r = np.random.default_rng(11)
    S0 = r.standard_normal((len(lens), 3, 4, 8))
    bounds = np.concatenate([[0], np.cumsum(lens)])
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0, seq_bounds=bounds)
    for n, (a, b) in enumerate(zip(bounds[:-1], bounds[1:])):
        o_n, s_n = oracle.recurrence(q[:, a:b], k[:, a:b], v[:, a:b], beta[:, a:b], la[:, a:b],
                                     initial_state=S0[n:n + 1])
        assert np.array_equal(out[:, a:b], o_n)
        assert np.array_equal(fin[n:n + 1], s_n)
    assert np.array_equal(fin[1], S0[1])  # empty sequence: final = initial


def test_p12_bounded_growth():
    """||k|| = 1, beta in [0, 2], alpha in (0, 1]: the transition is
    non-expansive, so ||S_t||_F <= ||S_{t-1}||_F + |beta_t| ||v_t||."""
    q, k, v, beta, la, S0 = _rand_case(200, 16, 8, per_channel=True, seed=12)
    beta = 2.0 * np.random.default_rng(13).random(beta.shape)
    state = S0
    for t in range(200):
        prev = np.linalg.norm(state)
        _, state = oracle.recurrence(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], beta[:, t:t + 1],
                                     la[:, t:t + 1], initial_state=state)
        assert np.linalg.norm(state) <= prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12


def test_scale_multiplies_readout_only():
    q, k, v, beta, la, S0 = _rand_case(9, 8, 8, per_channel=False, seed=14)
    o1, s1 = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    o2, s2 = oracle.recurrence(q, k, v, beta, la, initial_state=S0, scale=0.125)
    np.testing.assert_allclose(o2, 0.125 * o1, rtol=1e-15, atol=0)
    assert np.array_equal(s1, s2)


def test_planted_mistake_is_caught():
    """Sanity check of the pins themselves: a copy of the recurrence with the
    decay applied after the erase (a plausible mistake) fails the
    erase-then-write pin for per-channel decay, while the oracle passes it."""
    q, k, v, beta, la, S0 = _rand_case(6, 8, 4, per_channel=True, seed=15)
    beta[:] = 1.0
    S = S0[0, 0].copy()
    worst = 0.0
    for t in range(6):
        a = np.exp(la[0, t, 0])
        kt = k[0, t, 0]
        S = (S - np.outer(S @ kt, kt)) * a[None, :] + np.outer(v[0, t, 0], kt)  # wrong order
        worst = max(worst, np.abs(S @ kt - v[0, t, 0]).max())
    assert worst > 1e-3


# ------------------------------------------------- grouped value heads ----
@pytest.mark.parametrize("per_channel", [False, True])
def test_grouped_value_heads_against_product_form(per_channel):
    """Hk = 2 q/k heads shared by H = 6 value heads (groups of 3 consecutive
    value heads): every value head equals the brute-force product form run
    with its own v, gates and state and the q/k of head h // 3.  Distinct q/k
    per head, so a wrong head map (h % Hk, say) fails."""
    T, dk, dv, Hk, H = 6, 5, 3, 2, 6
    r = np.random.default_rng(40)
    q = r.standard_normal((1, T, Hk, dk))
    k = r.standard_normal((1, T, Hk, dk)) / np.sqrt(dk)
    v = r.standard_normal((1, T, H, dv))
    beta = r.random((1, T, H))
    la = -r.random((1, T, H, dk) if per_channel else (1, T, H))
    S0 = r.standard_normal((1, H, dv, dk))
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0)
    for h in range(H):
        O, S = models.product_form(q[0, :, h // 3], k[0, :, h // 3], v[0, :, h], beta[0, :, h], la[0, :, h], S0[0, h])
        np.testing.assert_allclose(out[0, :, h], O, rtol=0, atol=1e-12)
        np.testing.assert_allclose(fin[0, h], S, rtol=0, atol=1e-12)
    # decode takes the same grouping
    o1, s1 = oracle.decode(q[:, 0], k[:, 0], v[:, 0], beta[:, 0], la[:, 0], S0)
    for h in range(H):
        O, S = models.product_form(q[0, :1, h // 3], k[0, :1, h // 3], v[0, :1, h], beta[0, :1, h], la[0, :1, h],
                                   S0[0, h])
        np.testing.assert_allclose(o1[0, h], O[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(s1[0, h], S, rtol=0, atol=1e-12)


def test_grouped_heads_reject_non_divisor():
    q = np.zeros((1, 2, 4, 8))
    v = np.zeros((1, 2, 6, 8))
    with pytest.raises(ValueError):
        oracle.recurrence(q, q, v, np.zeros((1, 2, 6)), np.zeros((1, 2, 6)))


# ------------------------------------------------- multi-token decode ----
def _tokens_case(N, K, Hk, H, dk, dv, P, per_channel, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((N, K, Hk, dk))
    k = r.standard_normal((N, K, Hk, dk)) / np.sqrt(dk)
    v = r.standard_normal((N, K, H, dv))
    beta = r.random((N, K, H))
    la = -r.random((N, K, H, dk) if per_channel else (N, K, H))
    pool = r.standard_normal((P, H, dv, dk))
    return q, k, v, beta, la, pool


@pytest.mark.parametrize("per_channel", [False, True])
def test_decode_tokens_against_product_form(per_channel):
    """Each sequence's outputs are the brute-force product form's readouts of
    its first T tokens from its slot; its slot ends at the product form's
    state after C tokens; other slots, padding entries (slot -1 or >= P) and
    rows past T are untouched.  Values past the limits are clamped."""
    N, K, Hk, H, dk, dv, P = 6, 5, 1, 2, 4, 3, 9
    q, k, v, beta, la, pool = _tokens_case(N, K, Hk, H, dk, dv, P, per_channel, 41)
    slots = np.array([7, 2, -1, 0, 9, 4])
    ntok = np.array([5, 3, 5, 0, 2, 9])       # 9 > K: clamped to 5
    ncom = np.array([5, 0, 2, 0, 1, 2])
    out, written, new_pool = oracle.decode_tokens(q, k, v, beta, la, pool, num_tokens=ntok, num_commit=ncom,
                                                  state_slots=slots)
    touched = set()
    for n in range(N):
        s, T = slots[n], min(ntok[n], K)
        C = min(ncom[n], T)
        if s < 0 or s >= P or T == 0:
            assert not written[n].any() and not out[n].any()
            continue
        assert written[n, :T].all() and not written[n, T:].any() and not out[n, T:].any()
        for h in range(H):
            O, _ = models.product_form(q[n, :T, h // (H // Hk)], k[n, :T, h // (H // Hk)], v[n, :T, h],
                                       beta[n, :T, h], la[n, :T, h], pool[s, h])
            np.testing.assert_allclose(out[n, :T, h], O, rtol=0, atol=1e-12)
            _, Sc = models.product_form(q[n, :C, 0], k[n, :C, 0], v[n, :C, h], beta[n, :C, h], la[n, :C, h],
                                        pool[s, h])
            np.testing.assert_allclose(new_pool[s, h], Sc, rtol=0, atol=1e-12)
        if C > 0:
            touched.add(s)
    for s in range(P):
        if s not in touched:
            assert np.array_equal(new_pool[s], pool[s])
    assert touched == {7, 4}


def test_decode_tokens_verify_then_replay_equals_decoding_the_accepted_tokens():
    """The speculative flow: verify a K-token draft without committing, then
    replay the j accepted tokens (committing them) fused with the next draft;
    the slot then holds the state after the accepted tokens, the draft's
    outputs equal a plain K-token decode's, and one-token decode steps give
    the same numbers."""
    N, K, H, dk, dv = 3, 4, 2, 6, 5
    q, k, v, beta, la, pool = _tokens_case(N, K, H, H, dk, dv, N, True, 42)
    o_verify, _, p1 = oracle.decode_tokens(q, k, v, beta, la, pool, num_commit=np.zeros(N))
    assert np.array_equal(p1, pool)
    o_plain, _, p_all = oracle.decode_tokens(q, k, v, beta, la, pool)
    np.testing.assert_array_equal(o_verify, o_plain)
    state = pool.copy()
    for t in range(K):
        o_t, state = oracle.decode(q[:, t], k[:, t], v[:, t], beta[:, t], la[:, t], state)
        np.testing.assert_allclose(o_plain[:, t], o_t, rtol=0, atol=1e-13)
    np.testing.assert_allclose(p_all, state, rtol=0, atol=1e-13)
    acc = np.array([1, 3, 0])
    _, _, p2 = oracle.decode_tokens(q, k, v, beta, la, pool, num_tokens=np.full(N, K), num_commit=acc)
    for n in range(N):
        j = acc[n]
        _, s_j = oracle.recurrence(q[n:n + 1, :j], k[n:n + 1, :j], v[n:n + 1, :j], beta[n:n + 1, :j],
                                   la[n:n + 1, :j], initial_state=pool[n:n + 1])
        np.testing.assert_allclose(p2[n], s_j[0], rtol=0, atol=1e-13)


# ------------------------------------------------------- layer prologue ----
def _pro_case(T, Hk=1, H=2, dk=4, dv=2, seed=0, per_channel=False, state=True):
    r = np.random.default_rng(seed)
    C = 2 * Hk * dk + H * dv
    x = r.standard_normal((1, T, C))
    w = r.standard_normal((C, 4))
    a = r.standard_normal((1, T, H, dk) if per_channel else (1, T, H))
    b = r.standard_normal((1, T, H))
    st = r.standard_normal((1, 3, C)) if state else None
    return x, w, a, b, st, dict(num_qk_heads=Hk, head_dim_k=dk, head_dim_v=dv)


def _split(y, Hk, dk, H, dv):
    return (y[..., :Hk * dk].reshape(*y.shape[:-1], Hk, dk), y[..., Hk * dk:2 * Hk * dk].reshape(*y.shape[:-1], Hk, dk),
            y[..., 2 * Hk * dk:].reshape(*y.shape[:-1], H, dv))


def test_prologue_single_taps_are_shifts():
    """Tap 3 alone passes x_t through; tap 0 alone gives x_{t-3}, whose first
    three values are the state rows in order (row r: the input 3 - r tokens
    before the first); the taps of a channel act on that channel only."""
    x, w, a, b, st, kw = _pro_case(7, seed=50)
    C = x.shape[-1]
    for tap, expect in ((3, x[0]), (0, np.concatenate([st[0], x[0, :-3]])), (2, np.concatenate([st[0, 2:], x[0, :-1]]))):
        wt = np.zeros((C, 4))
        wt[:, tap] = 1.0
        q, k, v, *_ = oracle.layer_prologue(x, wt, a, b, conv_state=st, qk_norm=False, **kw)
        eq, ek, ev = _split(expect[None], 1, 4, 2, 2)
        np.testing.assert_array_equal(q, eq)
        np.testing.assert_array_equal(k, ek)
        np.testing.assert_array_equal(v, ev)


def test_prologue_constant_input_closed_form():
    """x_t = c for all t with a zero state: y_t = c * (w_3 + ... + w_{3-t})
    (the taps that reach a token inside the sequence)."""
    T = 6
    x, w, a, b, _, kw = _pro_case(T, seed=51, state=False)
    c = np.linspace(-1.0, 2.0, x.shape[-1])
    xc = np.broadcast_to(c, x.shape).copy()
    q, k, v, *_ = oracle.layer_prologue(xc, w, a, b, qk_norm=False, **kw)
    y = np.concatenate([q.reshape(1, T, -1), k.reshape(1, T, -1), v.reshape(1, T, -1)], axis=-1)
    for t in range(T):
        np.testing.assert_allclose(y[0, t], c * w[:, max(0, 3 - t):].sum(1), rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("split_at", [1, 2, 3, 5])
def test_prologue_continuation_through_the_state(split_at):
    """Running the first tokens, then the rest from the returned state, gives
    the single run's outputs and final state (also when the first part is
    shorter than the convolution)."""
    x, w, a, b, st, kw = _pro_case(9, seed=52, per_channel=True)
    full = oracle.layer_prologue(x, w, a, b, conv_state=st, silu=True, **kw)
    p1 = oracle.layer_prologue(x[:, :split_at], w, a[:, :split_at], b[:, :split_at], conv_state=st, silu=True, **kw)
    p2 = oracle.layer_prologue(x[:, split_at:], w, a[:, split_at:], b[:, split_at:], conv_state=p1[5], silu=True, **kw)
    for i in range(5):
        np.testing.assert_allclose(np.concatenate([p1[i], p2[i]], axis=1), full[i], rtol=0, atol=1e-14)
    np.testing.assert_array_equal(p2[5], full[5])
    np.testing.assert_array_equal(full[5][0], x[0, -3:])


def test_prologue_short_sequence_state_keeps_older_rows():
    x, w, a, b, st, kw = _pro_case(2, seed=53)
    *_, new = oracle.layer_prologue(x, w, a, b, conv_state=st, **kw)
    np.testing.assert_array_equal(new[0], np.concatenate([st[0, 2:], x[0]]))
    *_, same = oracle.layer_prologue(x[:, :0], w, a[:, :0], b[:, :0], conv_state=st, **kw)
    np.testing.assert_array_equal(same, st)


def test_prologue_norm_silu_and_gates():
    x, w, a, b, st, kw = _pro_case(5, Hk=2, H=3, dk=4, dv=2, seed=54, per_channel=True)
    q0, k0, v0, *_ = oracle.layer_prologue(x, w, a, b, conv_state=st, qk_norm=False, **kw)
    q, k, v, beta, la, _ = oracle.layer_prologue(x, w, a, b, conv_state=st, qk_norm=True, **kw)
    np.testing.assert_allclose(np.linalg.norm(q, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(q * np.linalg.norm(q0, axis=-1, keepdims=True), q0, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(v, v0)
    # a zero head stays zero
    xz = x.copy()
    xz[..., :4] = 0.0
    stz = st.copy()
    stz[..., :4] = 0.0
    qz, *_ = oracle.layer_prologue(xz, w, a, b, conv_state=stz, **kw)
    assert not qz[..., 0, :].any()
    # silu(y) = y / (1 + e^-y), applied before the norm
    qs, ks, vs, *_ = oracle.layer_prologue(x, w, a, b, conv_state=st, silu=True, qk_norm=False, **kw)
    np.testing.assert_allclose(vs, v0 / (1 + np.exp(-v0)), rtol=1e-14)
    # gates: closed forms and values at 0
    np.testing.assert_allclose(beta, 1 / (1 + np.exp(-b)), rtol=1e-15)
    np.testing.assert_allclose(la, np.log(1 / (1 + np.exp(a))), rtol=1e-13)
    z = np.zeros((1, 1, 3))
    *_, bz, lz, _ = oracle.layer_prologue(x[:, :1], w, z, z, conv_state=st, **kw)
    assert np.all(bz == 0.5) and np.allclose(lz, -np.log(2.0), rtol=1e-15)


def test_prologue_packed_equals_separate_runs():
    lens = [4, 0, 1, 6]
    T = sum(lens)
    x, w, a, b, _, kw = _pro_case(T, seed=55)
    st = np.random.default_rng(56).standard_normal((len(lens), 3, x.shape[-1]))
    bounds = np.concatenate([[0], np.cumsum(lens)])
    full = oracle.layer_prologue(x, w, a, b, conv_state=st, seq_bounds=bounds, **kw)
    for n in range(len(lens)):
        lo, hi = bounds[n], bounds[n + 1]
        part = oracle.layer_prologue(x[:, lo:hi], w, a[:, lo:hi], b[:, lo:hi], conv_state=st[n:n + 1], **kw)
        for i in range(5):
            np.testing.assert_array_equal(full[i][:, lo:hi], part[i])
        np.testing.assert_array_equal(full[5][n], part[5][0])


# ------------------------------------------------------------ backward ----
# The pages train these layers but print no backward pass.  The oracle's
# gradients are pinned by (1) a closed form of the one-token scalar case,
# (2) central finite differences of the (already pinned) forward oracle over
# every input element, (3) exact identities that follow from the recurrence
# being linear in q (readout) and jointly linear in (v, S0), and (4) a special
# case (beta = 0 cuts k and v out of the recurrence).

def _loss_weights(shape_out, shape_state, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal(shape_out), r.standard_normal(shape_state)


def test_backward_scalar_closed_form():
    """d_k = d_v = 1, one token: s1 = a s0 (1 - b k^2) + b v k, o = c s1 q,
    loss = w_o o + w_s s1; every derivative written out by hand."""
    q, k, v, b, a, s0, c, w_o, w_s = 0.8, -1.3, 0.45, 0.6, 0.7, 1.7, 0.9, -0.35, 1.25
    s1 = a * s0 * (1 - b * k * k) + b * v * k
    G = w_s + c * w_o * q                      # d loss / d s1
    want = {
        "dq": c * w_o * s1,
        "dv": G * b * k,
        "dbeta": G * k * (v - a * s0 * k),
        "dk": G * (b * v - 2 * a * s0 * b * k),
        "dlog_alpha": G * a * s0 * (1 - b * k * k),
        "d_initial_state": G * a * (1 - b * k * k),
    }
    arr = lambda x: np.full((1, 1, 1, 1), x)
    for la in (np.full((1, 1, 1), np.log(a)), np.full((1, 1, 1, 1), np.log(a))):
        g = oracle.recurrence_backward(arr(q), arr(k), arr(v), np.full((1, 1, 1), b), la,
                                       arr(w_o), initial_state=arr(s0), d_final_state=arr(w_s),
                                       scale=c)
        for name, val in want.items():
            assert abs(float(g[name].ravel()[0]) - val) < 1e-14, name


def _fd_case(layout, per_channel, T=5, dk=3, dv=2, seed=0):
    r = np.random.default_rng(seed)
    B, H, Hk, bounds = 1, 1, 1, None
    if layout == "dense":
        B = 2
    elif layout == "packed":
        bounds = [0, 2, 2, T]                  # the middle sequence is empty
    elif layout == "grouped":
        H, Hk = 2, 1
    N = B if bounds is None else len(bounds) - 1
    q = r.standard_normal((B, T, Hk, dk))
    k = r.standard_normal((B, T, Hk, dk)) / np.sqrt(dk)
    v = r.standard_normal((B, T, H, dv))
    beta = r.random((B, T, H))
    la = -r.random((B, T, H, dk) if per_channel else (B, T, H))
    S0 = r.standard_normal((N, H, dv, dk))
    return [q, k, v, beta, la, S0], bounds


def _finite_difference_check(args, bounds, scale, seed, eps=1e-6, backward=None):
    q, k, v, beta, la, S0 = args
    W_o, W_s = _loss_weights(v.shape, S0.shape, seed)

    def loss(*a):
        o, f = oracle.recurrence(*a[:5], initial_state=a[5], seq_bounds=bounds, scale=scale)
        return float((o * W_o).sum() + (f * W_s).sum())

    backward = backward or oracle.recurrence_backward
    g = backward(q, k, v, beta, la, W_o, initial_state=S0, d_final_state=W_s,
                 seq_bounds=bounds, scale=scale)
    worst = 0.0
    for ai, name in enumerate(["dq", "dk", "dv", "dbeta", "dlog_alpha", "d_initial_state"]):
        x = args[ai]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            a2 = list(args)
            xp = x.copy(); xp[idx] += eps; a2[ai] = xp; lp = loss(*a2)
            xm = x.copy(); xm[idx] -= eps; a2[ai] = xm; lm = loss(*a2)
            num[idx] = (lp - lm) / (2 * eps)
        worst = max(worst, np.abs(num - g[name]).max() / max(1.0, np.abs(num).max()))
    return worst


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("layout", ["dense", "packed", "grouped"])
def test_backward_matches_finite_differences(layout, per_channel):
    args, bounds = _fd_case(layout, per_channel, seed=3)
    assert _finite_difference_check(args, bounds, scale=0.7, seed=4) < 1e-8


def test_backward_finite_differences_across_checkpoint_segments():
    """150 tokens: three of the oracle's recomputation segments (64 tokens)."""
    args, bounds = _fd_case("single", True, T=150, dk=2, dv=2, seed=5)
    assert _finite_difference_check(args, bounds, scale=1.0, seed=6) < 1e-8


@pytest.mark.parametrize("per_channel", [False, True])
def test_backward_homogeneity_identities(per_channel):
    """o_t is linear in q_t and S_t does not depend on q, so
    sum <dq, q> = <d_out, out>.  With k, beta and the gates fixed, (out, S_T)
    is linear in (v, S0) jointly, so <dv, v> + <dS0, S0> = <d_out, out> +
    <d_final, S_T> (Euler's identity for degree-one homogeneous maps)."""
    r = np.random.default_rng(7)
    T, H, dk, dv = 300, 2, 16, 12
    bounds = [0, 37, 201, 300]
    q = r.standard_normal((1, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.standard_normal((1, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((1, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((1, T, H))))
    la = -np.log1p(np.exp(r.standard_normal((1, T, H, dk) if per_channel else (1, T, H))))
    S0 = r.standard_normal((3, H, dv, dk))
    W_o, W_s = _loss_weights(v.shape, S0.shape, 8)
    out, fin = oracle.recurrence(q, k, v, beta, la, initial_state=S0, seq_bounds=bounds, scale=0.5)
    g = oracle.recurrence_backward(q, k, v, beta, la, W_o, initial_state=S0, d_final_state=W_s,
                                   seq_bounds=bounds, scale=0.5)
    lo, ls = float((W_o * out).sum()), float((W_s * fin).sum())
    assert abs(float((g["dq"] * q).sum()) - lo) < 1e-10 * max(1.0, abs(lo))
    rhs = float((g["dv"] * v).sum() + (g["d_initial_state"] * S0).sum())
    assert abs(rhs - (lo + ls)) < 1e-10 * max(1.0, abs(lo + ls))


@pytest.mark.parametrize("per_channel", [False, True])
def test_backward_zero_beta_cuts_keys_and_values(per_channel):
    """beta = 0 leaves only decay and readout: k and v have no influence."""
    q, k, v, beta, la, S0 = _rand_case(20, 8, 6, per_channel=per_channel, seed=9)
    beta[:] = 0.0
    W_o, W_s = _loss_weights(v.shape, S0.shape, 10)
    g = oracle.recurrence_backward(q, k, v, beta, la, W_o, initial_state=S0, d_final_state=W_s)
    assert np.all(g["dk"] == 0.0) and np.all(g["dv"] == 0.0)
    assert np.abs(g["dbeta"]).max() > 1e-3 and np.abs(g["dq"]).max() > 1e-3


def test_backward_planted_mistake_is_caught():
    """Sanity check of the finite-difference pin: a token-by-token backward
    with one term dropped (the key's path through what the state recalls,
    S'^T dx) fails it by a wide margin."""
    def wrong_backward(q, k, v, beta, la, d_out, *, initial_state, d_final_state, seq_bounds, scale):
        right = oracle.recurrence_backward(q, k, v, beta, la, d_out, initial_state=initial_state,
                                           d_final_state=d_final_state, seq_bounds=seq_bounds,
                                           scale=scale)
        T, dk = q.shape[1], q.shape[3]
        S = initial_state[0, 0].copy()
        wrong_dk = right["dk"].copy()
        # recompute the dropped term and take it out of token 0's key gradient:
        # only token 0's S' is the decayed initial state, so the term is exact there
        a0 = np.exp(la[0, 0, 0]) * np.ones(dk)
        Sp = S * a0[None, :]
        dx = -beta[0, 0, 0] * (right["dv"][0, 0, 0] / beta[0, 0, 0])
        wrong_dk[0, 0, 0] -= Sp.T @ dx
        out = dict(right)
        out["dk"] = wrong_dk
        return out

    args, bounds = _fd_case("single", True, seed=11)
    assert _finite_difference_check(args, bounds, scale=1.0, seed=12) < 1e-8
    assert _finite_difference_check(args, bounds, scale=1.0, seed=12, backward=wrong_backward) > 1e-3


@pytest.mark.parametrize("per_channel", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 3, 5, 16, 32])
def test_backward_chunked_algebra_matches_oracle(per_channel, chunk):
    """The chunk-level gradient algebra (forward pass keeping chunk states,
    reverse pass carrying the state gradient, per-chunk gradients from the
    two states with shifted Gram operands) equals the oracle's token-by-token
    chain rule; 37 tokens leave a ragged last chunk."""
    r = np.random.default_rng(100 + chunk)
    T, dk, dv = 37, 8, 6
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    b = r.random(T)
    la = -np.log1p(np.exp(r.standard_normal((T, dk) if per_channel else T)))
    S0, dF = r.standard_normal((dv, dk)), r.standard_normal((dv, dk))
    dO = r.standard_normal((T, dv))
    got = models.chunked_backward(q, k, v, b, la, dO, S0, dF, chunk=chunk, scale=0.6)
    e = lambda x: x[None, :, None]
    want = oracle.recurrence_backward(e(q), e(k), e(v), e(b), e(la), e(dO), initial_state=S0[None, None],
                                      d_final_state=dF[None, None], scale=0.6)
    for name, val in got.items():
        np.testing.assert_allclose(val, want[name].reshape(val.shape), rtol=0, atol=1e-12, err_msg=name)
