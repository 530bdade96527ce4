"""Pins of the oracle's prologue backward (ckda_oracle_prologue_bwd), of the
fused backward built from it (oracle.bwd_fused) and of the DeltaProduct_2
backward (oracle.deltaproduct2_bwd), on the CPU.

The prologue of the "Complex KDA" discussion slides (frame "Backup: practical
gates differ from exact theoretical endpoints") makes the gate from a logit,
alpha = s [eps + (1 - eps) |tanh(a / 2)|], s the sign, and beta = 2 sigma(b);
the same frame fixes the backward convention: s is held constant and |r| takes
the zero subgradient at r = 0.  Away from a = 0 the gate is smooth, so central
finite differences of the pinned forward prologue decide the derivative; at
a = 0 the convention decides it (zero), and on either side of 0 the slope is
the one-sided slope of the smooth branch, not the jump of 2 eps."""
import math

import numpy as np
import pytest

RNG = np.random.default_rng
EPS5 = math.exp(-5.0)


def _problem(seed, ntok=5, dk=4, margin=0.05):
    r = RNG(seed)
    a = r.normal(0.0, 2.0, (ntok, dk))
    a = np.where(np.abs(a) < margin, np.sign(a + 1e-300) * margin, a)   # away from the kink at 0
    b = r.normal(0.0, 1.5, ntok)
    k = r.standard_normal((ntok, dk))
    q = r.standard_normal((ntok, dk))
    g = [r.standard_normal((ntok, dk)), r.standard_normal(ntok), r.standard_normal((ntok, dk)),
         r.standard_normal((ntok, dk))]
    return a, b, k, q, g


def _lin(o, a, b, k, q, flags, g):
    al, be, kk, qq = o.prologue(a, b, k, q, flags)
    return float(np.sum(al * g[0]) + np.sum(be * g[1]) + np.sum(kk * g[2]) + np.sum(qq * g[3]))


@pytest.mark.parametrize("flags", [7, 1, 2, 4, 0])
def test_prologue_backward_matches_finite_differences(oracle_lib, flags, seed=3):
    """L = sum(dalpha alpha) + sum(dbeta beta) + sum(dk k^) + sum(dq q^):
    the backward's gradients equal central differences of L in fp64."""
    o = oracle_lib
    a, b, k, q, g = _problem(seed)
    da, db, dk, dq = o.prologue_bwd(a, b, k, q, flags, *g)
    h = 1e-6
    for name, x, grad in (("a", a, da), ("b", b, db), ("k", k, dk), ("q", q, dq)):
        for ix in np.ndindex(x.shape):
            old = x[ix]
            x[ix] = old + h
            lp = _lin(o, a, b, k, q, flags, g)
            x[ix] = old - h
            lm = _lin(o, a, b, k, q, flags, g)
            x[ix] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[ix]) <= 1e-7 * max(1.0, abs(fd)), (flags, name, ix, fd, grad[ix])


def test_gate_slope_closed_form_and_zero_subgradient(oracle_lib):
    """d alpha / d a = (1 - eps) (1 - r^2) / 2 on both sides of zero (the sign
    held constant), exactly 0 at a = 0; beta' = 2 sigma (1 - sigma)."""
    o = oracle_lib
    a0 = 2.0 * math.atanh(0.5)                       # r = 1/2
    a = np.array([[0.0, a0, -a0, 1e-9, -1e-9, 30.0]])
    b = np.array([0.0])
    one = np.ones_like(a)
    da, db, _, _ = o.prologue_bwd(a, b, np.ones_like(a), np.ones_like(a), 1, one, np.ones(1), one, one)
    assert da[0, 0] == 0.0                            # zero subgradient of |r| at r = 0
    assert abs(da[0, 1] - (1 - EPS5) * 0.375) < 1e-15
    assert da[0, 2] == da[0, 1]                        # same slope below zero: the sign is detached
    assert abs(da[0, 3] - (1 - EPS5) * 0.5) < 1e-12    # one-sided slope, not the 2 eps jump
    assert abs(da[0, 4] - (1 - EPS5) * 0.5) < 1e-12
    assert 0.0 < da[0, 5] < 1e-12                      # saturated gate
    assert db[0] == 0.5                                # 2 sigma(0) (1 - sigma(0))


def test_detached_sign_differs_from_differencing_across_zero(oracle_lib):
    """A central difference across a = 0 sees the jump 2 eps of the gate; the
    backward does not (its slope near 0 is (1 - eps) / 2)."""
    o = oracle_lib
    h = 1e-8
    al_p, _, _, _ = o.prologue(np.array([[h]]), np.zeros(1), np.ones((1, 1)), np.ones((1, 1)), 1)
    al_m, _, _, _ = o.prologue(np.array([[-h]]), np.zeros(1), np.ones((1, 1)), np.ones((1, 1)), 1)
    across = (al_p[0, 0] - al_m[0, 0]) / (2 * h)
    assert across > 1e5                                # dominated by 2 eps / (2 h)
    da, _, _, _ = o.prologue_bwd(np.array([[h]]), np.zeros(1), np.ones((1, 1)), np.ones((1, 1)), 1,
                                 np.ones((1, 1)), np.ones(1), np.ones((1, 1)), np.ones((1, 1)))
    assert abs(da[0, 0] - (1 - EPS5) / 2) < 1e-12


def test_normalisation_backward_is_tangent(oracle_lib):
    """The gradient through a unit-norm row is orthogonal to the row (the
    normalisation cannot change with the row's length), and an upstream
    gradient along the row itself maps to ~0."""
    o = oracle_lib
    r = RNG(11)
    k = r.standard_normal((6, 8)) * 3.0
    z = np.zeros((6, 8))
    dy = r.standard_normal((6, 8))
    _, _, dk, _ = o.prologue_bwd(z, np.zeros(6), k, k, 2, z, np.zeros(6), dy, z)
    assert np.max(np.abs(np.sum(dk * k, axis=1))) < 1e-7 * np.max(np.abs(dk))
    _, _, dk2, _ = o.prologue_bwd(z, np.zeros(6), k, k, 2, z, np.zeros(6), k.copy(), z)
    assert np.max(np.abs(dk2)) < 1e-6


def _fused_problem(seed, scalar):
    r = RNG(seed)
    B, H, T, dk, dv = 1, 2, 7, 3, 2
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, dk))
    v = r.standard_normal((B, H, T, dv))
    a = r.normal(0.0, 2.0, (B, H, T) if scalar else (B, H, T, dk))
    a = np.where(np.abs(a) < 0.05, 0.05, a)
    b = r.normal(0.0, 1.0, (B, H, T))
    h0 = 0.3 * r.standard_normal((B, H, dk, dv))
    do = r.standard_normal((B, H, T, dv))
    dhT = r.standard_normal((B, H, dk, dv))
    return q, k, v, a, b, h0, do, dhT


@pytest.mark.parametrize("scalar", [False, True])
def test_fused_backward_matches_finite_differences(oracle_lib, scalar, flags=7):
    """bwd_fused (prologue, recurrence backward, prologue backward) against
    central differences of fwd_fused for L = sum(o do) + sum(hT dhT), with
    respect to every raw input: logits, raw keys and queries, values, h0."""
    o = oracle_lib
    q, k, v, a, b, h0, do, dhT = _fused_problem(5, scalar)
    grads = o.bwd_fused(q, k, v, a, b, do, dhT=dhT, h0=h0, flags=flags, scalar=scalar)

    def loss():
        af = np.broadcast_to(a[..., None], k.shape).copy() if scalar else a
        out, hT = o.fwd_fused(q, k, v, af, b, h0=h0, flags=flags)
        return float(np.sum(out * do) + np.sum(hT * dhT))

    h = 1e-6
    for name, x, g in zip(("q", "k", "v", "a", "b", "h0"), (q, k, v, a, b, h0), grads):
        for ix in np.ndindex(x.shape):
            old = x[ix]
            x[ix] = old + h
            lp = loss()
            x[ix] = old - h
            lm = loss()
            x[ix] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[ix]) <= 1e-6 * max(1.0, abs(fd)), (scalar, name, ix, fd, g[ix])


def dp2_problem(seed, gated, B=1, H=2, T=6, dk=3, dv=2):
    r = RNG(seed)
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, 2, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, 2, dv))
    a = r.uniform(-1, 1, (B, H, T)) if gated else None
    b = r.uniform(0, 2, (B, H, T, 2))
    h0 = 0.3 * r.standard_normal((B, H, dk, dv))
    do = r.standard_normal((B, H, T, dv))
    dhT = r.standard_normal((B, H, dk, dv))
    return q, k, v, a, b, h0, do, dhT


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("T,dk,dv", [(6, 3, 2), (5, 2, 4)])
def test_deltaproduct2_backward_agrees_with_the_substep_route(oracle_lib, gated, T, dk, dv):
    """The adjoint of the token step (deltaproduct2_bwd) and the delta-rule
    backward over the 2 T sub-steps (deltaproduct2_bwd_substeps, through the
    pinned bwd()) are two separate constructions of the same gradients."""
    q, k, v, a, b, h0, do, dhT = dp2_problem(40 + T + gated, gated, T=T, dk=dk, dv=dv)
    g1 = oracle_lib.deltaproduct2_bwd(q, k, v, a, b, do, dhT=dhT, h0=h0)
    import oracle as orc
    g2 = orc.deltaproduct2_bwd_substeps(q, k, v, a, b, do, dhT=dhT, h0=h0)
    for x, y in zip(g1, g2):
        if x is None:
            assert y is None
        else:
            np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-11)


def test_deltaproduct2_backward_across_checkpoints_and_without_optional_terms(oracle_lib):
    """70 tokens (two checkpoint segments), no h0 and no dhT, dk > dv."""
    q, k, v, a, b, _, do, _ = dp2_problem(77, True, T=70, dk=5, dv=2)
    g = oracle_lib.deltaproduct2_bwd(q, k, v, a, b, do)
    import oracle as orc
    g2 = orc.deltaproduct2_bwd_substeps(q, k, v, a, b, do)
    for x, y in zip(g, g2):
        np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-10)
    # a few central differences across the segment boundary
    o = oracle_lib

    def loss():
        out, _ = o.deltaproduct2(q, k, v, a, b)
        return float(np.sum(out * do))

    h = 1e-6
    for name, x, gx, ix in (("a", a, g[3], (0, 1, 63)), ("k", k, g[1], (0, 0, 64, 1, 2)),
                            ("v", v, g[2], (0, 1, 65, 0, 1)), ("b", b, g[4], (0, 0, 62, 1))):
        old = x[ix]
        x[ix] = old + h
        lp = loss()
        x[ix] = old - h
        lm = loss()
        x[ix] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - gx[ix]) <= 1e-6 * max(1.0, abs(fd)), (name, ix, fd, gx[ix])


@pytest.mark.parametrize("gated", [True, False])
def test_deltaproduct2_backward_matches_finite_differences(oracle_lib, gated):
    """deltaproduct2_bwd (the adjoint of the token step) against central
    differences of the separately written DeltaProduct_2 forward
    (ckda_oracle_deltaproduct2: the gate, then two Householder writes per
    token), for L = sum(o do) + sum(hT dhT), with respect to every input."""
    o = oracle_lib
    r = RNG(21 + gated)
    B, H, T, dk, dv = 1, 2, 6, 3, 2
    q = r.standard_normal((B, H, T, dk))
    k = r.standard_normal((B, H, T, 2, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, H, T, 2, dv))
    a = r.uniform(-1, 1, (B, H, T)) if gated else None
    b = r.uniform(0, 2, (B, H, T, 2))
    h0 = 0.3 * r.standard_normal((B, H, dk, dv))
    do = r.standard_normal((B, H, T, dv))
    dhT = r.standard_normal((B, H, dk, dv))
    grads = o.deltaproduct2_bwd(q, k, v, a, b, do, dhT=dhT, h0=h0)

    def loss():
        out, hT = o.deltaproduct2(q, k, v, a, b, h0=h0)
        return float(np.sum(out * do) + np.sum(hT * dhT))

    h = 1e-6
    inputs = (("q", q, grads[0]), ("k", k, grads[1]), ("v", v, grads[2]), ("b", b, grads[4]), ("h0", h0, grads[5]))
    if gated:
        inputs += (("a", a, grads[3]),)
    else:
        assert grads[3] is None
    for name, x, g in inputs:
        for ix in np.ndindex(x.shape):
            old = x[ix]
            x[ix] = old + h
            lp = loss()
            x[ix] = old - h
            lm = loss()
            x[ix] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - g[ix]) <= 1e-6 * max(1.0, abs(fd)), (gated, name, ix, fd, g[ix])
