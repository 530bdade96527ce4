"""The chunked backward model (tests/chunk_bwd_model.py) against the
sequential oracle backward, on the CPU: chunk sizes, ragged tails, zero
and +-1 gates, no division by a gate anywhere."""
import numpy as np
import pytest

import oracle
from chunk_bwd_model import bwd


@pytest.mark.parametrize("C,T,law", [(16, 40, "uniform"), (8, 33, "zeros"), (16, 64, "small"), (4, 9, "uniform"),
                                     (32, 70, "zeros")])
def test_chunk_backward_model_matches_oracle(C, T, law):
    r = np.random.default_rng(C * 100 + T)
    dk, dv = 5, 3
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    a = r.uniform(-1, 1, (T, dk))
    if law == "zeros":
        pick = r.integers(0, 4, a.shape)
        a = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, np.where(pick == 2, -1.0, a)))
    elif law == "small":
        a = np.sign(a) * np.exp(r.uniform(np.log(1e-9), 0, a.shape))
    b = r.uniform(0, 2, T)
    h0 = 0.3 * r.standard_normal((dk, dv))
    do = r.standard_normal((T, dv))
    dhT = r.standard_normal((dk, dv))
    got = bwd(q, k, v, a, b, do, dhT=dhT, h0=h0, C=C)
    e = lambda x: x[None, None]
    want = oracle.bwd(e(q), e(k), e(v), e(a), b[None, None], e(do), dhT=e(dhT), h0=e(h0))
    for g, w, name in zip(got, want, ("dq", "dk", "dv", "dalpha", "dbeta", "dh0")):
        w = w[0, 0]
        err = np.max(np.abs(g - w)) / max(1.0, np.max(np.abs(w)))
        assert err < 1e-10, (name, err)
