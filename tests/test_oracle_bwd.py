"""Pins of the oracle's backward (ckda_oracle_bwd) against central finite
differences of the pinned forward, on the CPU.  The loss is
L = sum(o * do) + sum(hT * dhT) with random do, dhT, so dL/dx is exactly
what the backward returns; fp64 central differences agree to ~1e-9."""
import numpy as np
import pytest

RNG = np.random.default_rng


def loss(orc, q, k, v, a, b, h0, do, dhT):
    o, hT = orc.fwd(q, k, v, a, b, h0=h0)
    return float(np.sum(o * do) + np.sum(hT * dhT))


def problem(seed, B=1, H=2, T=13, dk=3, dv=2, law="uniform"):
    r = RNG(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, dv))
    if law == "uniform":
        a = r.uniform(-1, 1, (B, H, T, dk))
    else:   # exact zeros and +-1 mixed in
        a = r.uniform(-1, 1, (B, H, T, dk))
        pick = r.integers(0, 4, a.shape)
        a = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, np.where(pick == 2, -1.0, a)))
    b = r.uniform(0, 2, (B, H, T))
    h0 = 0.3 * r.standard_normal((B, H, dk, dv))
    do = r.standard_normal((B, H, T, dv))
    dhT = r.standard_normal((B, H, dk, dv))
    return q, k, v, a, b, h0, do, dhT


def fd_check(orc, args, grads, names=("q", "k", "v", "a", "b", "h0"), sample=None, eps=1e-6, seed=0):
    q, k, v, a, b, h0, do, dhT = args
    inputs = dict(q=q, k=k, v=v, a=a, b=b, h0=h0)
    worst = 0.0
    r = RNG(seed)
    for name, g in zip(names, grads):
        x = inputs[name]
        idx = list(np.ndindex(x.shape))
        if sample is not None and len(idx) > sample:
            idx = [idx[i] for i in r.choice(len(idx), sample, replace=False)]
        for ix in idx:
            old = x[ix]
            x[ix] = old + eps
            lp = loss(orc, *(inputs[n] for n in ("q", "k", "v", "a", "b", "h0")), do, dhT)
            x[ix] = old - eps
            lm = loss(orc, *(inputs[n] for n in ("q", "k", "v", "a", "b", "h0")), do, dhT)
            x[ix] = old
            fd = (lp - lm) / (2 * eps)
            err = abs(fd - g[ix]) / max(1.0, abs(fd))
            worst = max(worst, err)
            assert err < 1e-6, (name, ix, fd, g[ix])
    return worst


@pytest.mark.parametrize("law", ["uniform", "zeros_and_units"])
def test_backward_matches_finite_differences(oracle_lib, law):
    args = problem(31 if law == "uniform" else 32, law=law)
    q, k, v, a, b, h0, do, dhT = args
    dq, dk, dv, da, db, dh0 = oracle_lib.bwd(q, k, v, a, b, do, dhT=dhT, h0=h0)
    fd_check(oracle_lib, args, (dq, dk, dv, da, db, dh0))


def test_backward_across_checkpoint_segments(oracle_lib):
    """T = 150 spans three 64-token checkpoint segments of the oracle."""
    args = problem(33, B=1, H=1, T=150, dk=2, dv=3)
    q, k, v, a, b, h0, do, dhT = args
    grads = oracle_lib.bwd(q, k, v, a, b, do, dhT=dhT, h0=h0)
    fd_check(oracle_lib, args, grads, sample=40, seed=1)


def test_backward_without_optional_terms(oracle_lib):
    """do only (dhT = None) and a zero initial state (h0 = None)."""
    q, k, v, a, b, h0, do, dhT = problem(34)
    dq, dk, dv, da, db, dh0 = oracle_lib.bwd(q, k, v, a, b, do, dhT=None, h0=None)
    z = np.zeros_like(h0)
    fd_check(oracle_lib, (q, k, v, a, b, z, do, np.zeros_like(dhT)), (dq, dk, dv, da, db, dh0))


def test_backward_of_pure_decay_is_closed_form(oracle_lib):
    """beta = 0: H_T = Diag(prod alpha) H_0 and o_t = (Diag(Gamma_t) H_0)^T q_t
    (the course's pure decay), so dq_t = Diag(Gamma_t) H_0 do_t, dh0 follows
    in closed form, and dk, dv vanish (k and v enter only through beta)."""
    q, k, v, a, b, h0, do, dhT = problem(35, T=6)
    b[:] = 0.0
    dq, dk, dv, da, db, dh0 = oracle_lib.bwd(q, k, v, a, b, do, dhT=dhT, h0=h0)
    gam = np.cumprod(a, axis=2)                       # Gamma_t = alpha_1 ... alpha_t
    want_dq = np.einsum("bhti,bhij,bhtj->bhti", gam, h0, do)
    assert np.max(np.abs(dq - want_dq)) < 1e-12
    assert np.max(np.abs(dv)) == 0.0 and np.max(np.abs(dk)) == 0.0
    want_dh0 = gam[:, :, -1, :, None] * dhT + np.einsum("bhti,bhti,bhtj->bhij", gam, q, do)
    assert np.max(np.abs(dh0 - want_dh0)) < 1e-12
