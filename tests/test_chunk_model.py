"""The chunkwise (UT/WY) form equals the sequential oracle (KDA course lesson,
'Chunkwise execution': chunking changes cost, never the numbers).  Checks the
derivation the GPU kernels implement, for several chunk sizes, ragged tails,
and stress gates (zeros, +-1, tiny magnitudes, repeated keys)."""
import numpy as np
import pytest

import chunk_model


def draw(rng, T, n, dv, law):
    q = rng.standard_normal((T, n))
    k = rng.standard_normal((T, n))
    if law == "repeated_keys":
        k[:] = k[0]
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    a = rng.uniform(-1, 1, (T, n))
    b = rng.uniform(0, 2, T)
    if law == "zero_and_unit":
        pick = rng.integers(0, 4, (T, n))
        a = np.where(pick == 0, 0.0, np.where(pick == 1, 1.0, np.where(pick == 2, -1.0, a)))
        b = rng.integers(0, 3, T).astype(float)
    elif law == "tiny":
        a = np.exp(rng.uniform(np.log(1e-12), 0, (T, n))) * np.where(rng.integers(0, 2, (T, n)) == 0, -1, 1)
    elif law == "kda":
        a = 1 / (1 + np.exp(-(rng.standard_normal((T, n)) + 2)))
        b = 1 / (1 + np.exp(-rng.standard_normal(T)))
    return q, k, v, a, b


@pytest.mark.parametrize("chunk", [1, 4, 16, 48, 64])
@pytest.mark.parametrize("law", ["ckda", "kda", "zero_and_unit", "tiny", "repeated_keys"])
def test_chunk_form_matches_oracle(oracle_lib, chunk, law):
    rng = np.random.default_rng(chunk * 7 + len(law))
    T, n, dv = 100, 8, 5                      # 100 is ragged for every chunk size > 4
    q, k, v, a, b = draw(rng, T, n, dv, law)
    H0 = rng.standard_normal((n, dv))
    o_ref, h_ref = oracle_lib.fwd(q[None, None], k[None, None], v[None, None], a[None, None],
                                  b[None, None], h0=H0[None, None])
    o, h = chunk_model.forward(q, k, v, a, b, H0, chunk)
    scale = max(1.0, np.abs(o_ref).max())
    assert np.abs(o - o_ref[0, 0]).max() <= 1e-11 * scale
    assert np.abs(h - h_ref[0, 0]).max() <= 1e-11 * max(1.0, np.abs(h_ref).max())
