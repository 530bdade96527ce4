"""fp64 numpy model of the chunkwise backward the GPU kernels implement
(test infrastructure, checked against the sequential oracle backward).

Per chunk of C positions with incoming state H (and signed gate products
G(t, j) = alpha_{j+1} ... alpha_t per channel, Gamma_t = G(t, -1)):

  forward:  KG = K . Gamma,  QG = Q . Gamma,  KR_j = k_j . G(C-1, j)
            S[t, j] = sum_c k_tc k_jc G_c(t, j) (j < t),  M[t, j] = sum_c q_tc k_jc G_c(t, j) (j <= t)
            T = (I + Diag(beta) S)^-1,  TB = T Diag(beta)
            X = V - KG H,  U = TB X,  O = QG H + M U,  H' = Gamma_C . H + KR^T U
  backward: dU = M^T dO + KR dH',  dX = TB^T dU (= dV)
            dH = Gamma_C . dH' + QG^T dO - KG^T dX
            dQG = dO H^T,  dKG = -dX H^T,  dKR = U dH'^T,  dGamma_C = rowsum(H . dH')
            dM = tril(dO U^T),  dTB = tril(dU X^T)
            dbeta_t = sum_i T[i, t] dTB[i, t] + sum_j dA[t, j] S[t, j],
            dA = -T^T (dTB Diag(beta)) T^T (strictly lower),  dS = Diag(beta) dA
  then the decayed-Gram backward and every gate derivative by recursive
  halving: for a block split into halves L (positions j) and R (t) at
  m = last of L, G(t, j) = G(t, m) G(m, j) with both factors products of
  gates, so the cross terms are plain products of rescaled operands; the
  derivative for the gate at s collects every pair j < s <= t with
  G(t, s) G(s - 1, j), i.e. the gate's own factor left out -- no division
  by a gate anywhere.
"""
from __future__ import annotations

import numpy as np


def _prod(a, lo, hi):
    """prod of rows lo..hi (inclusive) of a [C, dk]; ones if empty."""
    if hi < lo:
        return np.ones(a.shape[1])
    return np.prod(a[lo:hi + 1], axis=0)


def gram_pairs(x, y, a, lo=0, hi=None, out=None):
    """out[t, j] = sum_c x_tc y_jc G_c(t, j) for lo <= j < t <= hi, by halving."""
    C = x.shape[0]
    hi = C - 1 if hi is None else hi
    if out is None:
        out = np.zeros((C, C))
    if hi <= lo:
        return out
    m = (lo + hi) // 2           # L = lo..m, R = m+1..hi
    xr = np.stack([x[t] * _prod(a, m + 1, t) for t in range(m + 1, hi + 1)])   # x_t G(t, m)
    yl = np.stack([y[j] * _prod(a, j + 1, m) for j in range(lo, m + 1)])       # y_j G(m, j)
    out[m + 1:hi + 1, lo:m + 1] = xr @ yl.T
    gram_pairs(x, y, a, lo, m, out)
    gram_pairs(x, y, a, m + 1, hi, out)
    return out


def gram_bwd(WM, WS, q, k, a, lo=0, hi=None, acc=None):
    """Backward of S (weights WS, x = y = k) and M (weights WM, x = q, y = k)
    off the diagonal: returns (dq, dk, dalpha) contributions."""
    C, dk = q.shape
    hi = C - 1 if hi is None else hi
    if acc is None:
        acc = (np.zeros((C, dk)), np.zeros((C, dk)), np.zeros((C, dk)))
    dq, dkk, da = acc
    if hi <= lo:
        return acc
    m = (lo + hi) // 2
    L, R = range(lo, m + 1), range(m + 1, hi + 1)
    gR = {t: _prod(a, m + 1, t) for t in R}          # G(t, m)
    gL = {j: _prod(a, j + 1, m) for j in L}          # G(m, j)
    WMr, WSr = WM[m + 1:hi + 1, lo:m + 1], WS[m + 1:hi + 1, lo:m + 1]
    ky = np.stack([k[j] * gL[j] for j in L])                   # y_j G(m, j)
    qx = np.stack([q[t] * gR[t] for t in R])                   # x_t G(t, m), M term
    kx = np.stack([k[t] * gR[t] for t in R])                   # x_t G(t, m), S term
    ZM = WMr @ ky                                              # rows t in R
    ZS = WSr @ ky
    ZL = WMr.T @ qx + WSr.T @ kx                               # rows j in L
    for i, t in enumerate(R):
        dq[t] += gR[t] * ZM[i]
        dkk[t] += gR[t] * ZS[i]
    for i, j in enumerate(L):
        dkk[j] += gL[j] * ZL[i]
    # gate s in L: pairs (t in R, j in L, j < s): G(m, s) sum_{j<s} y_j ZL_j G(s-1, j)
    f = np.zeros(dk)
    for i, s in enumerate(L):
        da[s] += _prod(a, s + 1, m) * f
        f = a[s] * f + k[s] * ZL[i]
    # gate s in R: pairs (t in R, t >= s, j in L): G(s-1, m) sum_{t>=s} x_t Z_t G(t, s)
    bsum = np.zeros(dk)
    Rl = list(R)
    for i in range(len(Rl) - 1, -1, -1):
        s = Rl[i]
        bsum = q[s] * ZM[i] + k[s] * ZS[i] + (a[s + 1] * bsum if i + 1 < len(Rl) else 0.0)
        da[s] += _prod(a, m + 1, s - 1) * bsum
    gram_bwd(WM, WS, q, k, a, lo, m, acc)
    gram_bwd(WM, WS, q, k, a, m + 1, hi, acc)
    return acc


def chunk_consts(q, k, a, b):
    C, dk = q.shape
    Gam = np.cumprod(a, axis=0)
    Gend = np.stack([_prod(a, j + 1, C - 1) for j in range(C)])    # G(C-1, j)
    S = gram_pairs(k, k, a)
    M = gram_pairs(q, k, a) + np.diag(np.sum(q * k, axis=1))
    T = np.linalg.inv(np.eye(C) + b[:, None] * S)
    return Gam, Gend, S, M, T, T * b[None, :]


def bwd(q, k, v, a, b, do, dhT=None, h0=None, C=16):
    """Chunked backward for one head: q, k, a [T, dk]; v, do [T, dv]; b [T]."""
    Tn, dk = q.shape
    dv = v.shape[1]
    n = (Tn + C - 1) // C
    pad = n * C - Tn
    P = lambda x, fill: np.concatenate([x, np.full((pad,) + x.shape[1:], fill)]) if pad else x
    q, k, v, do = P(q, 0.0), P(k, 0.0), P(v, 0.0), P(do, 0.0)
    a, b = P(a, 1.0), P(b, 0.0)
    H = np.zeros((dk, dv)) if h0 is None else h0.copy()
    Hs, consts = [], []
    for c in range(n):
        sl = slice(c * C, (c + 1) * C)
        Gam, Gend, S, M, T, TB = cc = chunk_consts(q[sl], k[sl], a[sl], b[sl])
        consts.append(cc)
        Hs.append(H)
        U = TB @ (v[sl] - (k[sl] * Gam) @ H)
        H = Gam[-1][:, None] * H + (k[sl] * Gend).T @ U
    dH = np.zeros((dk, dv)) if dhT is None else dhT.copy()
    out = dict(dq=np.zeros((n * C, dk)), dk=np.zeros((n * C, dk)), dv=np.zeros((n * C, dv)),
               da=np.zeros((n * C, dk)), db=np.zeros(n * C))
    for c in range(n - 1, -1, -1):
        sl = slice(c * C, (c + 1) * C)
        qq, kk, aa, bb, VV, dO = q[sl], k[sl], a[sl], b[sl], v[sl], do[sl]
        Gam, Gend, S, M, T, TB = consts[c]
        H = Hs[c]
        KG, QG, KR = kk * Gam, qq * Gam, kk * Gend
        X = VV - KG @ H
        U = TB @ X
        dU = M.T @ dO + KR @ dH
        dX = TB.T @ dU
        dQG, dKG, dKR = dO @ H.T, -dX @ H.T, U @ dH.T
        dGC = np.sum(H * dH, axis=1)
        dM = np.tril(dO @ U.T)
        dTB = np.tril(dU @ X.T)
        db = np.sum(T * dTB, axis=0)
        dA = np.tril(-T.T @ (dTB * bb[None, :]) @ T.T, -1)
        db += np.sum(dA * S, axis=1)
        dS = bb[:, None] * dA
        dq, dkk, da = gram_bwd(np.tril(dM, -1), dS, qq, kk, aa)
        dq += np.diag(dM)[:, None] * kk           # diagonal of M: G = 1
        dkk += np.diag(dM)[:, None] * qq
        dq += dQG * Gam
        dkk += dKG * Gam + dKR * Gend
        # gate terms of Gamma_t (virtual pair with the chunk start), KR (with
        # the chunk end) and Gamma_C (both)
        Cn = qq.shape[0]
        Rt = dQG * qq + dKG * kk
        bsum = np.zeros(dk)
        for s in range(Cn - 1, -1, -1):
            bsum = Rt[s] + (aa[s + 1] * bsum if s + 1 < Cn else 0.0)
            da[s] += _prod(aa, 0, s - 1) * bsum
        f = np.zeros(dk)
        for s in range(Cn):
            da[s] += _prod(aa, s + 1, Cn - 1) * f
            f = aa[s] * f + dKR[s] * kk[s]
        for s in range(Cn):
            da[s] += dGC * _prod(aa, 0, s - 1) * _prod(aa, s + 1, Cn - 1)
        out["dq"][sl], out["dk"][sl], out["dv"][sl], out["da"][sl], out["db"][sl] = dq, dkk, dX, da, db
        dH = Gam[-1][:, None] * dH + QG.T @ dO - KG.T @ dX
    cut = lambda x: x[:Tn]
    return (cut(out["dq"]), cut(out["dk"]), cut(out["dv"]), cut(out["da"]), cut(out["db"]), dH)
