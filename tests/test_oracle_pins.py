"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every test here runs on the CPU.  Each one checks the oracle against a value,
closed form, invariant or special case that does not come from the oracle
itself, so that a plausible slip in it (readout before the update, gate after
the correction, a transposed state, a dropped sign or beta) fails at least one
of them.  Sources are the "Complex KDA" paper (Eqs. (1)-(3), Prop. 2/7,
Thm. 1, Thm. 8, Lemma 24, App. B.2), its discussion slides, the KDA course
lesson's worked trace and the state-reduction slides.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def run(oracle_lib, q, k, v, a, b, h0=None):
    """Oracle on fp64 arrays; shapes [T,dk] etc. for a single head."""
    e = lambda x: np.asarray(x, np.float64)[None, None]
    h = None if h0 is None else np.asarray(h0, np.float64)[None, None]
    o, hT = oracle_lib.fwd(e(q), e(k), e(v), e(a), np.asarray(b, np.float64)[None, None], h0=h)
    return o[0, 0], hT[0, 0]


def states(oracle_lib, q, k, v, a, b, h0):
    """H_1..H_T by resuming the oracle one token at a time."""
    out, H = [], np.asarray(h0, np.float64)
    for t in range(len(b)):
        _, H = run(oracle_lib, q[t:t + 1], k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1], H)
        out.append(H)
    return out


def transition(oracle_lib, a, k, beta):
    """The n x n transition matrix A = (I - beta k k^T) Diag(a), read off the
    oracle by pushing the identity through one step with v = 0."""
    n = len(a)
    z = np.zeros((1, n))
    _, H1 = run(oracle_lib, z, np.asarray(k)[None], np.zeros((1, n)), np.asarray(a)[None], [beta], np.eye(n))
    return H1


def unit(rng, n):
    x = rng.standard_normal(n)
    return x / np.linalg.norm(x)


# --------------------------------------------------------------------------
# KDA course, worked case (full trace), parts A and B


def test_worked_trace_decay(oracle_lib):
    g = json.load(open(os.path.join(GOLD, "kda_course_worked_trace.json")))
    S0, a = np.array(g["S0"]), np.array(g["gate"])
    T = 3
    z = np.zeros((T, 2))
    Hs = states(oracle_lib, z, z, z, np.tile(a, (T, 1)), np.zeros(T), S0)
    for t in range(T):
        np.testing.assert_allclose(Hs[t], np.array(g["part_A_decay_no_write"][f"t{t+1}"]), rtol=0, atol=1e-12)


def test_worked_trace_of_one(oracle_lib):
    g = json.load(open(os.path.join(GOLD, "kda_course_worked_trace.json")))
    a = np.array(g["gate"])
    T = 4
    z = np.zeros((T, 2))
    Hs = [np.eye(2)] + states(oracle_lib, z, z, z, np.tile(a, (T, 1)), np.zeros(T), np.eye(2))
    tr = g["trace_of_one"]
    for t in range(T + 1):
        for ch, key in ((0, "channel1"), (1, "channel2")):
            printed = tr[key][t]
            # printed to 3 decimals, except 0.0016 which is exact
            assert abs(Hs[t][ch, ch] - printed) <= 5e-4 + 1e-12, (t, ch, Hs[t][ch, ch], printed)
    assert abs(Hs[4][1, 1] - 0.0016) < 1e-15


def test_worked_trace_write(oracle_lib):
    g = json.load(open(os.path.join(GOLD, "kda_course_worked_trace.json")))
    S0, a = np.array(g["S0"]), np.array(g["gate"])
    B = g["part_B_write_at_step2"]
    T = 4
    k = np.zeros((T, 2)); v = np.zeros((T, 2)); b = np.zeros(T)
    k[1], v[1], b[1] = B["k"], B["v"], B["beta"]
    # q = k_2 at step 2 reads the state's prediction for the written key
    q = np.zeros((T, 2)); q[1] = [0.0, 1.0]
    o, _ = run(oracle_lib, q, k, v, np.tile(a, (T, 1)), b, S0)
    Hs = states(oracle_lib, q, k, v, np.tile(a, (T, 1)), b, S0)
    # gated state of step 2, and the prediction it makes for k = [0, 1]
    S_prime = np.diag(a) @ Hs[0]
    np.testing.assert_allclose(S_prime.T @ k[1], B["v_hat"], atol=1e-12)
    np.testing.assert_allclose(v[1] - S_prime.T @ k[1], B["error"], atol=1e-12)
    np.testing.assert_allclose(Hs[1], B["S_after_write"], atol=1e-12)
    # exact correction: the read-out of the written key returns v
    np.testing.assert_allclose(o[1], B["v"], atol=1e-12)
    np.testing.assert_allclose(Hs[3][1], [B["channel2_two_steps_later"]] * 2, atol=1e-12)
    # the same write on channel 1
    k1 = k.copy(); k1[1] = [1.0, 0.0]
    H = states(oracle_lib, q, k1, v, np.tile(a, (T, 1)), b, S0)[3]
    np.testing.assert_allclose(H[0], [B["same_write_on_channel1_two_steps_later"]] * 2, atol=1e-12)
    # half-lives printed on the same page
    hl = g["half_lives_tokens"]
    assert round(math.log(0.5) / math.log(a[0]), 2) == hl["channel1"]
    assert round(math.log(0.5) / math.log(a[1]), 2) == hl["channel2"]


# --------------------------------------------------------------------------
# Closed forms


def test_two_reflections_make_rotation(oracle_lib):
    """Discussion slides, 'Two reflections make a rotation in one update':
    k=(1,1)/sqrt2, beta=2, alpha=(-1,1) gives R_{pi/2}; four steps give I."""
    k = np.array([1.0, 1.0]) / math.sqrt(2.0)
    A = transition(oracle_lib, [-1.0, 1.0], k, 2.0)
    np.testing.assert_allclose(A, [[0.0, -1.0], [1.0, 0.0]], atol=1e-15)
    T = 4
    z = np.zeros((T, 2))
    _, H4 = run(oracle_lib, z, np.tile(k, (T, 1)), z, np.tile([-1.0, 1.0], (T, 1)), 2.0 * np.ones(T), np.eye(2))
    np.testing.assert_allclose(H4, np.eye(2), atol=1e-14)


@pytest.mark.parametrize("m", [1, 2, 3, 5, 7])
def test_one_step_modular_counter(oracle_lib, m):
    """Paper Lemma 24: beta=2, alpha=(1,-1), k=(-sin phi/2, cos phi/2) rotates by
    phi = pi/m; from c_0 = e1 the orbit has period 2m with 2m distinct points."""
    phi = math.pi / m
    k = np.array([-math.sin(phi / 2), math.cos(phi / 2)])
    T = 2 * m
    z = np.zeros((T, 2))
    q = np.tile([0.3, 0.7], (T, 1))
    Hs = states(oracle_lib, q, np.tile(k, (T, 1)), z, np.tile([1.0, -1.0], (T, 1)), 2.0 * np.ones(T), np.eye(2))
    for i, H in enumerate(Hs, start=1):
        R = np.array([[math.cos(i * phi), -math.sin(i * phi)], [math.sin(i * phi), math.cos(i * phi)]])
        np.testing.assert_allclose(H, R, atol=1e-13)
    pts = [np.array([1.0, 0.0])] + [H[:, 0] for H in Hs[:-1]]
    assert len({(round(p[0], 9), round(p[1], 9)) for p in pts}) == 2 * m
    np.testing.assert_allclose(Hs[-1], np.eye(2), atol=1e-13)


@pytest.mark.parametrize("alpha", [-1.0, -0.7, -0.3, 0.0, 0.4, 1.0])
@pytest.mark.parametrize("theta", [0.0, 0.3, math.pi / 4, 1.1, math.pi / 2])
def test_eq2_planar_transition(oracle_lib, alpha, theta):
    """Paper Eq. (2): (I-2kk^T)Diag(alpha,1) with k=(cos t, sin t) equals
    [[-a cos2t, -sin2t], [-a sin2t, cos2t]]; trace (1-a)cos2t, det -a,
    discriminant (1-a)^2 cos^2 2t + 4a; a non-real pair has |lambda| = sqrt(-a)."""
    k = np.array([math.cos(theta), math.sin(theta)])
    A = transition(oracle_lib, [alpha, 1.0], k, 2.0)
    c2, s2 = math.cos(2 * theta), math.sin(2 * theta)
    np.testing.assert_allclose(A, [[-alpha * c2, -s2], [-alpha * s2, c2]], atol=1e-14)
    assert abs(np.trace(A) - (1 - alpha) * c2) < 1e-14
    assert abs(np.linalg.det(A) + alpha) < 1e-14
    disc = (1 - alpha) ** 2 * c2 ** 2 + 4 * alpha
    lam = np.linalg.eigvals(A)
    if disc < -1e-12:
        assert np.all(np.abs(lam.imag) > 0)
        np.testing.assert_allclose(np.abs(lam), math.sqrt(-alpha), atol=1e-12)
    elif disc > 1e-12:
        assert np.all(np.abs(lam.imag) < 1e-12)


def test_eq3_diagonal_as_axis_householders(oracle_lib):
    """Paper Eq. (3): Diag(alpha) = prod_i (I - (1 - alpha_i) e_i e_i^T).  A gate
    step (beta=0) equals n delta steps with k=e_i, beta=1-alpha_i, alpha=1, v=0."""
    rng = np.random.default_rng(3)
    n, dv = 5, 3
    a = rng.uniform(-1, 1, n)
    H0 = rng.standard_normal((n, dv))
    _, Hg = run(oracle_lib, np.zeros((1, n)), np.zeros((1, n)), np.zeros((1, dv)), a[None], [0.0], H0)
    K = np.eye(n)
    _, Hh = run(oracle_lib, np.zeros((n, n)), K, np.zeros((n, dv)), np.ones((n, n)), 1.0 - a, H0)
    np.testing.assert_allclose(Hh, Hg, atol=1e-14)
    np.testing.assert_allclose(Hg, np.diag(a) @ H0, atol=1e-15)


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0, 1.5, 2.0])
@pytest.mark.parametrize("theta", [0.2, 0.7, 1.3])
def test_prop2_sign_magnitude_block(oracle_lib, beta, theta):
    """Paper Prop. 2 / Prop. 7: with S = Diag(sign alpha), (I - beta k k^T) S
    restricted to span{k-, k+} is B(beta,theta) = [[b cos^2 - 1, -b sin cos],
    [b sin cos, 1 - b sin^2]]; it acts as S on the complement; non-real pair iff
    beta^2 cos^2(2 theta) < 4 (beta - 1); at beta=2 it is a rotation by 2 theta."""
    rng = np.random.default_rng(int(beta * 10 + theta * 100))
    n = 6
    sgn = np.array([-1, -1, -1, 1, 1, 1], float)
    em = np.zeros(n); em[:3] = unit(rng, 3)
    ep = np.zeros(n); ep[3:] = unit(rng, 3)
    k = math.cos(theta) * em + math.sin(theta) * ep
    A = transition(oracle_lib, sgn, k, beta)
    Bm = np.array([[beta * math.cos(theta) ** 2 - 1, -beta * math.sin(theta) * math.cos(theta)],
                   [beta * math.sin(theta) * math.cos(theta), 1 - beta * math.sin(theta) ** 2]])
    Q = np.stack([em, ep], axis=1)
    np.testing.assert_allclose(Q.T @ A @ Q, Bm, atol=1e-14)
    x = np.zeros(n); x[:3] = np.cross(em[:3], unit(rng, 3)); x /= np.linalg.norm(x)
    np.testing.assert_allclose(A @ x, -x, atol=1e-14)
    lam = np.linalg.eigvals(Bm)
    nonreal = beta ** 2 * math.cos(2 * theta) ** 2 < 4 * (beta - 1)
    assert (np.max(np.abs(lam.imag)) > 1e-12) == nonreal
    if beta == 2.0:
        R = np.array([[math.cos(2 * theta), -math.sin(2 * theta)], [math.sin(2 * theta), math.cos(2 * theta)]])
        np.testing.assert_allclose(Bm, R, atol=1e-14)


# --------------------------------------------------------------------------
# Invariants


def test_transitions_non_expansive_and_spectrum(oracle_lib):
    """Discussion slides 'The transition remains non-expansive': ||A||_2 <= 1
    for alpha in [-1,1]^n, beta in [0,2], unit k.  Paper Thm. 8: at most one
    non-real pair, and only if beta > 1 and some alpha_i < 0."""
    rng = np.random.default_rng(8)
    for trial in range(300):
        n = int(rng.integers(2, 9))
        a = rng.uniform(-1, 1, n)
        if trial % 3 == 0:
            a = np.abs(a)
        beta = float(rng.uniform(0, 2)) if trial % 5 else float(rng.choice([0.0, 1.0, 2.0]))
        k = unit(rng, n)
        A = transition(oracle_lib, a, k, beta)
        np.testing.assert_allclose(A, (np.eye(n) - beta * np.outer(k, k)) @ np.diag(a), atol=1e-14)
        assert np.linalg.norm(A, 2) <= 1 + 1e-12
        lam = np.linalg.eigvals(A)
        n_nonreal = int(np.sum(np.abs(lam.imag) > 1e-9))
        assert n_nonreal <= 2
        if beta <= 1 or np.all(a >= 0):
            assert n_nonreal == 0


def test_orthogonal_special_case_preserves_norm(oracle_lib):
    """Paper Thm. 1: beta = 2, alpha in {+-1}^n gives orthogonal transitions,
    so with v = 0 the Frobenius norm of the state never changes."""
    rng = np.random.default_rng(11)
    n, dv, T = 8, 5, 400
    k = np.stack([unit(rng, n) for _ in range(T)])
    a = np.where(rng.integers(0, 2, (T, n)) == 0, -1.0, 1.0)
    H0 = rng.standard_normal((n, dv))
    _, HT = run(oracle_lib, np.zeros((T, n)), k, np.zeros((T, dv)), a, 2.0 * np.ones(T), H0)
    assert abs(np.linalg.norm(HT) - np.linalg.norm(H0)) < 1e-12 * np.linalg.norm(H0)
    A = transition(oracle_lib, a[0], k[0], 2.0)
    np.testing.assert_allclose(A.T @ A, np.eye(n), atol=1e-14)


def test_homogeneous_propagation_non_expansive(oracle_lib):
    """With v = 0 (no additive write) ||H_t||_2 <= ||H_{t-1}||_2 in CKDA ranges."""
    rng = np.random.default_rng(12)
    n, dv, T = 6, 4, 60
    k = np.stack([unit(rng, n) for _ in range(T)])
    Hs = states(oracle_lib, np.zeros((T, n)), k, np.zeros((T, dv)), rng.uniform(-1, 1, (T, n)),
                rng.uniform(0, 2, T), rng.standard_normal((n, dv)))
    norms = [np.linalg.norm(H, 2) for H in Hs]
    assert all(b <= a + 1e-12 for a, b in zip(norms, norms[1:]))


def brute_force(q, k, v, a, b, H0):
    """Closed-form solution of the affine recurrence H_t = A_t H_{t-1} + B_t:
    H_t = Phi_{t,0} H_0 + sum_{s<=t} Phi_{t,s} B_s with Phi_{t,s} = A_t ... A_{s+1},
    A_t = (I - b_t k_t k_t^T) Diag(a_t), B_t = b_t k_t v_t^T (paper App. B.2 Eq. (9)),
    and o_t = H_t^T q_t.  Built from explicit dense matrix products."""
    T, n = k.shape
    A = [(np.eye(n) - b[t] * np.outer(k[t], k[t])) @ np.diag(a[t]) for t in range(T)]
    Bw = [b[t] * np.outer(k[t], v[t]) for t in range(T)]
    o = np.zeros((T, v.shape[1]))
    Ht = None
    for t in range(T):
        Phi = np.eye(n)
        acc = np.zeros_like(H0)
        for s in range(t, -1, -1):       # s = t, t-1, ..., 0 ; Phi = A_t ... A_{s+1}
            acc += Phi @ Bw[s]
            Phi = Phi @ A[s]
        Ht = Phi @ H0 + acc              # Phi = A_t ... A_0 here
        o[t] = Ht.T @ q[t]
    return o, Ht


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(oracle_lib, seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.integers(1, 17))
    n = int(rng.integers(1, 9))
    dv = int(rng.integers(1, 9))
    q = rng.standard_normal((T, n))
    k = np.stack([unit(rng, n) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, n))
    b = rng.uniform(0, 2, T)
    H0 = rng.standard_normal((n, dv)) if seed % 2 else np.zeros((n, dv))
    o, HT = run(oracle_lib, q, k, v, a, b, H0)
    ob, Hb = brute_force(q, k, v, a, b, H0)
    np.testing.assert_allclose(o, ob, atol=1e-13)
    np.testing.assert_allclose(HT, Hb, atol=1e-13)


def test_exact_retrieval_at_beta_one(oracle_lib):
    """KDA course 'Delta correction': with beta = 1 and a unit key the write is
    an exact correction, H_t^T k_t = v_t, whatever the gate and the old state."""
    rng = np.random.default_rng(13)
    n, dv, T = 7, 5, 20
    k = np.stack([unit(rng, n) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    Hs = states(oracle_lib, np.zeros((T, n)), k, v, rng.uniform(-1, 1, (T, n)), np.ones(T),
                rng.standard_normal((n, dv)))
    for t in range(T):
        np.testing.assert_allclose(Hs[t].T @ k[t], v[t], atol=1e-13)


def test_pure_decay_at_beta_zero(oracle_lib):
    """beta = 0: only the per-channel decay acts, H_T = Diag(prod_t alpha_t) H_0."""
    rng = np.random.default_rng(14)
    n, dv, T = 6, 3, 30
    a = rng.uniform(-1, 1, (T, n))
    H0 = rng.standard_normal((n, dv))
    o, HT = run(oracle_lib, rng.standard_normal((T, n)), rng.standard_normal((T, n)),
                rng.standard_normal((T, dv)), a, np.zeros(T), H0)
    np.testing.assert_allclose(HT, np.diag(np.prod(a, axis=0)) @ H0, atol=1e-15)


def test_rank_bound_from_zero_state(oracle_lib):
    """State-reduction slides: from S_0 = 0, rank(S_t) <= t (DeltaNet rank bound;
    the diagonal gate cannot raise the rank)."""
    rng = np.random.default_rng(15)
    n, dv, T = 8, 8, 6
    k = np.stack([unit(rng, n) for _ in range(T)])
    Hs = states(oracle_lib, np.zeros((T, n)), k, rng.standard_normal((T, dv)), rng.uniform(-1, 1, (T, n)),
                rng.uniform(0.1, 2, T), np.zeros((n, dv)))
    for t, H in enumerate(Hs, start=1):
        assert np.linalg.matrix_rank(H, tol=1e-10) <= t


def test_gauge_sign_absorption(oracle_lib):
    """Discussion slides 'Absorb cumulative signs into keys and queries' (paper
    Lemma 27): with P_t = S_1...S_t, running the positive-magnitude recurrence on
    (P_t k_t, P_t q_t, |alpha_t|) gives the same outputs and H_T = P_T H~_T."""
    rng = np.random.default_rng(16)
    n, dv, T = 6, 4, 25
    q = rng.standard_normal((T, n))
    k = np.stack([unit(rng, n) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, n))
    a[3, 2] = 0.0          # sign(0) = +1
    b = rng.uniform(0, 2, T)
    H0 = rng.standard_normal((n, dv))
    o, HT = run(oracle_lib, q, k, v, a, b, H0)
    S = np.where(a < 0, -1.0, 1.0)
    P = np.cumprod(S, axis=0)
    o2, HT2 = run(oracle_lib, P * q, P * k, v, np.abs(a), b, H0)
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(P[-1][:, None] * HT2, HT, atol=1e-12)


def test_channel_permutation_and_sign_flip(oracle_lib):
    """State-reduction slides, joint orthogonal change of key/query coordinates,
    restricted to transforms that commute with Diag(alpha): permuting channels
    (with alpha and the rows of h0) or flipping a channel's sign in k, q and h0
    leaves o unchanged and moves hT's rows the same way."""
    rng = np.random.default_rng(17)
    n, dv, T = 7, 3, 18
    q = rng.standard_normal((T, n))
    k = np.stack([unit(rng, n) for _ in range(T)])
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, n))
    b = rng.uniform(0, 2, T)
    H0 = rng.standard_normal((n, dv))
    o, HT = run(oracle_lib, q, k, v, a, b, H0)
    p = rng.permutation(n)
    o2, HT2 = run(oracle_lib, q[:, p], k[:, p], v, a[:, p], b, H0[p])
    np.testing.assert_allclose(o2, o, atol=1e-12)
    np.testing.assert_allclose(HT2, HT[p], atol=1e-12)
    f = np.ones(n); f[[1, 4]] = -1
    o3, HT3 = run(oracle_lib, q * f, k * f, v, a, b, H0 * f[:, None])
    np.testing.assert_allclose(o3, o, atol=1e-12)
    np.testing.assert_allclose(HT3, HT * f[:, None], atol=1e-12)


def test_resume_and_decode_continue_forward(oracle_lib):
    """The state is the checkpoint: fwd(T1) -> hT -> fwd(T2, h0=hT) equals
    fwd(T1+T2), and decode steps continue a forward exactly."""
    rng = np.random.default_rng(18)
    B, H, T, n, dv = 2, 3, 40, 5, 4
    q = rng.standard_normal((B, H, T, n))
    k = rng.standard_normal((B, H, T, n)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    a = rng.uniform(-1, 1, (B, H, T, n))
    b = rng.uniform(0, 2, (B, H, T))
    h0 = rng.standard_normal((B, H, n, dv))
    o, hT = oracle_lib.fwd(q, k, v, a, b, h0=h0)
    T1 = 23
    o1, h1 = oracle_lib.fwd(q[:, :, :T1], k[:, :, :T1], v[:, :, :T1], a[:, :, :T1], b[:, :, :T1], h0=h0)
    o2, h2 = oracle_lib.fwd(q[:, :, T1:], k[:, :, T1:], v[:, :, T1:], a[:, :, T1:], b[:, :, T1:], h0=h1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=2), o)
    np.testing.assert_array_equal(h2, hT)
    S = h1.copy()
    for t in range(T1, T):
        ot = oracle_lib.decode(q[:, :, t], k[:, :, t], v[:, :, t], a[:, :, t], b[:, :, t], S)
        np.testing.assert_array_equal(ot, o[:, :, t])
    np.testing.assert_array_equal(S, hT)


def test_bf16_reader_widens_exactly(oracle_lib):
    """The oracle reads bf16 bit patterns; pushing them through a beta = 0,
    identity-state step returns each widened value exactly (checked against
    torch's own bf16 -> fp64 conversion)."""
    from gated_delta_rule_ckda_amd.inputs import raw
    rng = np.random.default_rng(19)
    n = 16
    x = torch.from_numpy(rng.standard_normal((1, 1, 5, n)).astype(np.float32) * 7).to(torch.bfloat16)
    a = torch.ones_like(x)
    b = torch.zeros((1, 1, 5), dtype=torch.bfloat16)
    h0 = np.eye(n, dtype=np.float32)[None, None]
    o, _ = oracle_lib.fwd(raw(x), raw(x), raw(x[..., :n]), raw(a), raw(b), h0=h0)
    np.testing.assert_array_equal(o, x.to(torch.float64).numpy())
    # negative zero, subnormal and extreme bf16 patterns
    bits = np.array([0x8000, 0x0001, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80, 0x0080, 0x1234,
                     0x4049, 0xC049, 0x3C00, 0x5000, 0x2000, 0x7F00, 0x00FF, 0x8001], np.uint16)
    xb = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).reshape(1, 1, 1, n)
    o, _ = oracle_lib.fwd(raw(xb), raw(xb), raw(xb), raw(torch.ones_like(xb)),
                          raw(torch.zeros((1, 1, 1), dtype=torch.bfloat16)), h0=h0)
    np.testing.assert_array_equal(o, xb.to(torch.float64).numpy())


# --------------------------------------------------------------------------
# Per-token prologue: the practical gate parameterisation of the discussion
# slides (frame "Backup: practical gates differ from exact theoretical
# endpoints") and unit-norm keys / queries.  Pinned through identities and
# limits stated on the pages, not by re-deriving the oracle's own formula.

G, NK, NQ = 1, 2, 4


def pro(oracle_lib, a, b, k=None, q=None, flags=G):
    a = np.atleast_2d(np.asarray(a, np.float64))
    b = np.asarray(b, np.float64).reshape(a.shape[:-1])
    k = np.ones_like(a) if k is None else np.atleast_2d(np.asarray(k, np.float64))
    q = np.ones_like(a) if q is None else np.atleast_2d(np.asarray(q, np.float64))
    return oracle_lib.prologue(a, b, k, q, flags)


def test_practical_gate_endpoints_and_zero(oracle_lib):
    """log|alpha| spans [-5, 0]: alpha(0) = +e^-5 (s = +1 at r = 0) and the
    gate tends to +-1 as the logit grows (reached in fp64 at |a| = 80)."""
    al, be, _, _ = pro(oracle_lib, [0.0, 80.0, -80.0], [0.0])
    assert al[0, 0] == math.exp(-5.0)
    assert al[0, 1] == 1.0 and al[0, 2] == -1.0
    assert be[0] == 1.0                      # beta = 2 sigma(0) = 1


def test_practical_gate_matches_sigmoid_form(oracle_lib):
    """tanh(a/2) = 2 sigma(a) - 1 (both forms are given for r): the gate built
    from the sigmoid form agrees, for logits of both signs."""
    rng = np.random.default_rng(7)
    a = rng.normal(0.0, 3.0, 512)
    al, _, _, _ = pro(oracle_lib, a, [0.0])
    r = 2.0 / (1.0 + np.exp(-a)) - 1.0
    eps = math.exp(-5.0)
    want = np.where(r >= 0, 1.0, -1.0) * (eps + (1.0 - eps) * np.abs(r))
    assert np.max(np.abs(al[0] - want)) < 1e-14


def test_practical_gate_sign_symmetry_and_range(oracle_lib):
    """The gate carries the logit's sign, is odd away from zero, and its
    magnitude grows with |a| inside [e^-5, 1]."""
    a = np.linspace(0.01, 20.0, 400)
    al_p, _, _, _ = pro(oracle_lib, a, [0.0])
    al_m, _, _, _ = pro(oracle_lib, -a, [0.0])
    assert np.all(al_p[0] > 0) and np.all(al_m[0] < 0)
    assert np.array_equal(al_m[0], -al_p[0])
    assert np.all(np.diff(al_p[0]) > 0)
    la = np.log(np.abs(al_p[0]))
    assert la.min() >= -5.0 and la.max() <= 0.0


def test_practical_beta(oracle_lib):
    """beta = 2 sigma(b): beta(b) + beta(-b) = 2, range (0, 2), beta(0) = 1."""
    b = np.linspace(-12.0, 12.0, 241)
    _, bp, _, _ = pro(oracle_lib, np.zeros((241, 1)), b)
    _, bm, _, _ = pro(oracle_lib, np.zeros((241, 1)), -b)
    assert np.max(np.abs(bp + bm - 2.0)) < 1e-15
    assert np.all(bp > 0) and np.all(bp < 2) and bp[120] == 1.0


def test_unit_norm_keys_and_queries(oracle_lib):
    """(3, 4) -> (0.6, 0.8) up to the 1e-6 guard; random rows come out with
    unit norm in their own direction; a zero row stays zero; with its flag off
    a vector passes through unchanged."""
    k = np.array([[3.0, 4.0, 0.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    q = np.array([[1.0, 2.0, 2.0, 0.0], [0.0, 0.0, 0.0, 0.0]])
    _, _, kk, qq = pro(oracle_lib, np.zeros((2, 4)), [0.0, 0.0], k, q, NK)
    assert np.max(np.abs(kk[0] - [0.6, 0.8, 0.0, 0.0])) < 1e-7
    assert np.all(kk[1] == 0.0)
    assert np.array_equal(qq, q)                     # NORM_Q off
    _, _, _, qq = pro(oracle_lib, np.zeros((2, 4)), [0.0, 0.0], k, q, NQ)
    assert np.max(np.abs(qq[0] - np.array([1.0, 2.0, 2.0, 0.0]) / 3.0)) < 1e-7
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 128)) * rng.uniform(0.1, 10.0, (64, 1))
    _, _, kk, _ = pro(oracle_lib, np.zeros_like(x), np.zeros(64), x, x, NK)
    n = np.linalg.norm(kk, axis=1)
    assert np.max(np.abs(n - 1.0)) < 1e-6
    cos = np.sum(kk * x, axis=1) / np.linalg.norm(x, axis=1)
    assert np.max(np.abs(cos - 1.0)) < 1e-6


def test_fused_forward_is_the_recurrence_on_prepared_inputs(oracle_lib):
    """fwd_fused = the plain recurrence on gates built by the sigmoid form of
    the slides and keys scaled by numpy's norm (tolerance for the 1e-6 guard)."""
    rng = np.random.default_rng(11)
    T, n, dv = 24, 6, 5
    a = rng.normal(0, 2, (T, n))
    b = rng.normal(0, 1, T)
    k = rng.normal(0, 1, (T, n))
    q = rng.normal(0, 1, (T, n))
    v = rng.normal(0, 1, (T, dv))
    h0 = rng.normal(0, 0.1, (n, dv))
    e = lambda x: x[None, None]
    o_f, h_f = oracle_lib.fwd_fused(e(q), e(k), e(v), e(a), b[None, None], h0=h0[None, None], flags=G | NK | NQ)
    r = 2.0 / (1.0 + np.exp(-a)) - 1.0
    eps = math.exp(-5.0)
    al = np.where(r >= 0, 1.0, -1.0) * (eps + (1.0 - eps) * np.abs(r))
    be = 2.0 / (1.0 + np.exp(-b))
    kn = k / np.linalg.norm(k, axis=1, keepdims=True)
    qn = q / np.linalg.norm(q, axis=1, keepdims=True)
    o_p, h_p = run(oracle_lib, qn, kn, v, al, be, h0)
    assert np.max(np.abs(o_f[0, 0] - o_p)) < 1e-5 * max(1.0, np.max(np.abs(o_p)))
    assert np.max(np.abs(h_f[0, 0] - h_p)) < 1e-5 * max(1.0, np.max(np.abs(h_p)))


# ---------------------------------------------------------------- DeltaProduct_2

def dp2(oracle_lib, q, k, v, a, b, h0=None):
    """DeltaProduct_2 oracle on one head: q [T,dk], k [T,2,dk], v [T,2,dv], b [T,2], a [T] or None."""
    e = lambda x: np.asarray(x, np.float64)[None, None]
    h = None if h0 is None else e(h0)
    o, hT = oracle_lib.deltaproduct2(e(q), e(k), e(v), None if a is None else e(a), e(b), h0=h)
    return o[0, 0], hT[0, 0]


def test_deltaproduct2_tracks_permutations_with_transposition_keys(oracle_lib):
    """Paper App. C ("Consequences for CKDA and Gated DeltaProduct"): with
    keys (e_i - e_j)/sqrt2, beta = 2, gate 1, no additive term and H_0 = I,
    each Householder factor is the transposition (i j) and the state is the
    permutation matrix of the running product -- two transpositions per token
    here, so a token can apply a 3-cycle."""
    n = 5
    rng = np.random.default_rng(21)
    T = 12
    k = np.zeros((T, 2, n))
    P = np.eye(n)
    want = []
    for t in range(T):
        for j in range(2):
            a, c = rng.choice(n, 2, replace=False)
            k[t, j, a], k[t, j, c] = 1 / math.sqrt(2), -1 / math.sqrt(2)
            Tr = np.eye(n)
            Tr[[a, c]] = Tr[[c, a]]
            P = Tr @ P                       # the first sub-step acts first
        want.append(P.copy())
    q = rng.standard_normal((T, n))
    v = np.zeros((T, 2, n))            # no additive term; dv = n so that H_t is n x n
    o, hT = dp2(oracle_lib, q, k, v, np.ones(T), np.full((T, 2), 2.0), np.eye(n))
    assert np.max(np.abs(hT - want[-1])) < 1e-12
    for t in range(T):
        assert np.max(np.abs(o[t] - want[t].T @ q[t])) < 1e-12
    # ungated (alpha = NULL) is the same as gate 1
    o2, h2 = dp2(oracle_lib, q, k, v, None, np.full((T, 2), 2.0), np.eye(n))
    assert np.array_equal(o, o2) and np.array_equal(hT, h2)


def test_deltaproduct2_transition_is_the_gated_householder_product(oracle_lib):
    """Gated DeltaProduct transition alpha_t (I - b2 k2 k2^T)(I - b1 k1 k1^T)
    (paper App. C): with no additive term (v = 0) the state after T tokens is
    the product of these dense matrices applied to H_0 (brute force)."""
    rng = np.random.default_rng(22)
    T, n, dv = 9, 4, 3
    k = rng.standard_normal((T, 2, n))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    b = rng.uniform(0, 2, (T, 2))
    a = rng.uniform(-1, 1, T)
    h0 = rng.standard_normal((n, dv))
    _, hT = dp2(oracle_lib, rng.standard_normal((T, n)), k, np.zeros((T, 2, dv)), a, b, h0)
    H = h0.copy()
    for t in range(T):
        A = a[t] * (np.eye(n) - b[t, 1] * np.outer(k[t, 1], k[t, 1])) @ (np.eye(n) - b[t, 0] * np.outer(k[t, 0], k[t, 0]))
        H = A @ H
    assert np.max(np.abs(hT - H)) < 1e-12


@pytest.mark.parametrize("which", [0, 1])
def test_deltaproduct2_with_one_inactive_substep_is_the_delta_rule(oracle_lib, which):
    """beta = 0 on one sub-step leaves a single delta-rule update per token:
    the plain (pinned) recurrence with the scalar gate on every channel; with
    the first sub-step inactive the gate still acts before the second."""
    rng = np.random.default_rng(23 + which)
    T, n, dv = 11, 5, 4
    q = rng.standard_normal((T, n))
    k = rng.standard_normal((T, 2, n))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 2, dv))
    b = rng.uniform(0, 2, (T, 2))
    b[:, which] = 0.0
    a = rng.uniform(-1, 1, T)
    h0 = rng.standard_normal((n, dv))
    o, hT = dp2(oracle_lib, q, k, v, a, b, h0)
    act = 1 - which
    o_p, h_p = run(oracle_lib, q, k[:, act], v[:, act], np.repeat(a[:, None], n, 1), b[:, act], h0)
    assert np.max(np.abs(o - o_p)) < 1e-12 and np.max(np.abs(hT - h_p)) < 1e-12


def test_deltaproduct2_decode_continues_the_forward(oracle_lib):
    rng = np.random.default_rng(24)
    T, n, dv = 6, 4, 3
    q = rng.standard_normal((T, n))
    k = rng.standard_normal((T, 2, n))
    v = rng.standard_normal((T, 2, dv))
    b = rng.uniform(0, 2, (T, 2))
    a = rng.uniform(-1, 1, T)
    o, hT = dp2(oracle_lib, q, k, v, a, b)
    S = np.zeros((1, 1, n, dv))
    for t in range(T):
        ot = oracle_lib.deltaproduct2_decode(q[t][None, None], k[t][None, None], v[t][None, None],
                                             np.asarray(a[t]).reshape(1, 1), b[t][None, None], S)
        assert np.max(np.abs(ot[0, 0] - o[t])) < 1e-12
    assert np.max(np.abs(S[0, 0] - hT)) < 1e-12
