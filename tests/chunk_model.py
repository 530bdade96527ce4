"""fp64 numpy model of the chunkwise (UT/WY) form of the CKDA recurrence.

Test-only.  It is neither the oracle nor the GPU path: it restates, in plain
numpy, the chunk algebra that the GPU kernels implement, so that the
derivation itself can be checked against the sequential oracle and so that a
kernel's intermediates have something to be compared with.

The pages call chunkwise execution exact (the KDA course lesson, section
"Chunkwise execution": it changes cost, never the numbers) but do not print
the algorithm (the paper defers it to an appendix that is not on the pages).
The form below is derived from the recurrence of the paper's Eq. (1):

  per chunk, with incoming state H0 and local positions t = 1..C,
  sign/magnitude split     s_t = sign(alpha_t) (sign(0) = +1), m_t = |alpha_t|
                           (paper Prop. 2; discussion slides, sign absorption)
  cumulative parity        P_t = s_1 ... s_t          (chunk-local)
  absorbed keys/queries    k~_t = P_t k_t, q~_t = P_t q_t
  decay between positions  r(t, j) = m_{j+1} ... m_t   (per channel, j <= t)
  A[t, j] = beta_t sum_c k~_tc k~_jc r_c(t, j)   for j < t
  M[t, j] =        sum_c q~_tc k~_jc r_c(t, j)   for j <= t
  T = (I + A)^-1                                  (unit lower triangular)
  U = T diag(beta) (V - (K~ . gamma) H0),   gamma_t = r(t, 0)
  O = (Q~ . gamma) H0 + M U
  H_C = P_C . [ gamma_C . H0 + (K~ . r(C, j))^T U ]
"""
from __future__ import annotations

import numpy as np


def decay(mag: np.ndarray, t: int, j: int) -> np.ndarray:
    """prod_{s=j+1..t} mag_s (1-based positions; 1 when t == j)."""
    return np.prod(mag[j:t], axis=0) if t > j else np.ones(mag.shape[1])


def chunk_step(q, k, v, a, b, H0):
    """One chunk.  q, k, a: [C, n]; v: [C, dv]; b: [C]; H0: [n, dv] (fp64).
    Returns (O [C, dv], H_C [n, dv], intermediates dict)."""
    C, n = k.shape
    s = np.where(a < 0, -1.0, 1.0)
    m = np.abs(a)
    P = np.cumprod(s, axis=0)
    kt, qt = P * k, P * q
    R = np.zeros((C + 1, C + 1, n))                   # R[t, j] = r(t, j), 1-based t, j in 0..C
    for t in range(C + 1):
        for j in range(t + 1):
            R[t, j] = decay(m, t, j)
    gamma = np.stack([R[t, 0] for t in range(1, C + 1)])          # [C, n]
    A = np.zeros((C, C))
    M = np.zeros((C, C))
    for t in range(C):
        for j in range(t + 1):
            rr = R[t + 1, j + 1]
            M[t, j] = np.sum(qt[t] * kt[j] * rr)
            if j < t:
                A[t, j] = b[t] * np.sum(kt[t] * kt[j] * rr)
    Tm = np.linalg.inv(np.eye(C) + A)
    Kg, Qg = kt * gamma, qt * gamma
    U = Tm @ (b[:, None] * (v - Kg @ H0))
    O = Qg @ H0 + M @ U
    Kr = kt * np.stack([R[C, j + 1] for j in range(C)])
    HC = P[-1][:, None] * (gamma[-1][:, None] * H0 + Kr.T @ U)
    return O, HC, dict(P=P, gamma=gamma, A=A, M=M, T=Tm, U=U, Kg=Kg, Qg=Qg, Kr=Kr)


def forward(q, k, v, a, b, H0, chunk):
    """Whole sequence for one head, chunk by chunk (last chunk may be short).
    q, k, a: [T, n]; v: [T, dv]; b: [T]; H0: [n, dv].  Returns (o, hT)."""
    T = k.shape[0]
    H = np.array(H0, np.float64)
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, chunk):
        c1 = min(T, c0 + chunk)
        o[c0:c1], H, _ = chunk_step(q[c0:c1], k[c0:c1], v[c0:c1], a[c0:c1], b[c0:c1], H)
    return o, H
