"""fp64 CPU oracle for the (Complex) Kimi Delta Attention recurrence.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg import this package.  The GPU library never
imports, links or calls it, and the two share no code.

The arithmetic lives in ``ckda_oracle.c`` (plain C, fp64, OpenMP across the
independent (batch, head) recurrences); this module only compiles it with gcc
and marshals numpy arrays into it.  Inputs are handed over as raw element
bytes exactly as the GPU receives them: ``float32``, ``float64``, or
``uint16`` arrays holding bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ckda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libckda_oracle.so")

F32, BF16, F64 = 0, 1, 2
_lib = None


def build(force: bool = True) -> str:
    """Compile ckda_oracle.c into libckda_oracle.so with gcc (-O2, OpenMP)."""
    global _lib
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    _lib = None
    return _LIB_PATH


def _declare(lib):
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.ckda_oracle_fwd.argtypes = [vp, vp, vp, vp, vp, i, vp, i, vp, vp, i, i, i, i, i, i]
    lib.ckda_oracle_fwd.restype = i
    lib.ckda_oracle_decode.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i]
    lib.ckda_oracle_decode.restype = i
    lib.ckda_oracle_num_threads.argtypes = []
    lib.ckda_oracle_num_threads.restype = i
    lib.ckda_oracle_prologue.argtypes = [vp, vp, vp, vp, i, i, ctypes.c_longlong, i, vp, vp, vp, vp]
    lib.ckda_oracle_prologue.restype = i
    lib.ckda_oracle_deltaproduct2.argtypes = [vp, vp, vp, vp, vp, i, vp, i, vp, vp, i, i, i, i, i, i]
    lib.ckda_oracle_deltaproduct2.restype = i
    lib.ckda_oracle_deltaproduct2_decode.argtypes = [vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i]
    lib.ckda_oracle_deltaproduct2_decode.restype = i
    lib.ckda_oracle_bwd.argtypes = [vp] * 5 + [i, vp, i, vp, vp, i] + [vp] * 6 + [i] * 6
    lib.ckda_oracle_bwd.restype = i
    lib.ckda_oracle_prologue_bwd.argtypes = [vp, vp, vp, vp, i, i, ctypes.c_longlong, i] + [vp] * 8
    lib.ckda_oracle_prologue_bwd.restype = i
    lib.ckda_oracle_deltaproduct2_bwd.argtypes = [vp] * 5 + [i, vp, i, vp, vp, i] + [vp] * 6 + [i] * 6
    lib.ckda_oracle_deltaproduct2_bwd.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs must be float32, float64 or uint16(bf16 bits), got {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().ckda_oracle_num_threads()


def fwd(q, k, v, alpha, beta, h0=None, want_o=True, nthreads=0):
    """Sequential fp64 forward.

    q, k, alpha: [B,H,T,dk]; v: [B,H,T,dv]; beta: [B,H,T]; all one dtype.
    h0: [B,H,dk,dv] float32 or float64, or None for a zero state.
    Returns (o [B,H,T,dv] float64 or None, hT [B,H,dk,dv] float64).
    """
    q, k, v, alpha, beta = (np.ascontiguousarray(x) for x in (q, k, v, alpha, beta))
    code = _code(q)
    for x in (k, v, alpha, beta):
        if _code(x) != code:
            raise TypeError("q, k, v, alpha, beta must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (B, H, T, dv) \
            or beta.shape != (B, H, T):
        raise ValueError("inconsistent shapes")
    h0c, h0code = None, F32
    if h0 is not None:
        h0c = np.ascontiguousarray(h0)
        if h0c.shape != (B, H, dk, dv):
            raise ValueError("h0 shape")
        h0code = _code(h0c)
        if h0code == BF16:
            raise TypeError("h0 must be float32 or float64")
    o = np.empty((B, H, T, dv), np.float64) if want_o else None
    hT = np.empty((B, H, dk, dv), np.float64)
    rc = _load().ckda_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), code,
                                 _ptr(h0c), h0code, _ptr(o), _ptr(hT),
                                 B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_fwd failed with code {rc}")
    return o, hT


def decode(q, k, v, alpha, beta, S, nthreads=0):
    """One recurrent step applied in place to the fp64 state S [N,H,dk,dv].

    q, k, alpha: [N,H,dk]; v: [N,H,dv]; beta: [N,H].  Returns o [N,H,dv] float64.
    """
    q, k, v, alpha, beta = (np.ascontiguousarray(x) for x in (q, k, v, alpha, beta))
    code = _code(q)
    for x in (k, v, alpha, beta):
        if _code(x) != code:
            raise TypeError("q, k, v, alpha, beta must share one dtype")
    N, H, dk = q.shape
    dv = v.shape[-1]
    if not (isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous
            and S.shape == (N, H, dk, dv)):
        raise ValueError("S must be a C-contiguous float64 [N,H,dk,dv] array")
    if k.shape != q.shape or alpha.shape != q.shape or v.shape != (N, H, dv) \
            or beta.shape != (N, H):
        raise ValueError("inconsistent shapes")
    o = np.empty((N, H, dv), np.float64)
    rc = _load().ckda_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), code,
                                    _ptr(S), _ptr(o), N, H, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_decode failed with code {rc}")
    return o


# flags of the per-token prologue (ckda_oracle.c)
GATES, NORM_K, NORM_Q = 1, 2, 4


def prologue(a, b, k, q, flags):
    """Practical gates from logits and unit-norm keys / queries, in fp64.

    a, k, q: [..., dk]; b: [...]; one dtype.  With GATES, a and b are the
    logits of alpha and beta; NORM_K / NORM_Q scale k / q to unit norm per
    token.  Returns fp64 (alpha, beta, k, q); a step whose flag is off returns
    its input widened."""
    a, b, k, q = (np.ascontiguousarray(x) for x in (a, b, k, q))
    code = _code(a)
    for x in (b, k, q):
        if _code(x) != code:
            raise TypeError("a, b, k, q must share one dtype")
    if k.shape != a.shape or q.shape != a.shape or b.shape != a.shape[:-1]:
        raise ValueError("inconsistent shapes")
    dk = a.shape[-1]
    ntok = int(np.prod(a.shape[:-1], dtype=np.int64))
    alpha, kk, qq = (np.empty(a.shape, np.float64) for _ in range(3))
    beta = np.empty(b.shape, np.float64)
    rc = _load().ckda_oracle_prologue(_ptr(a), _ptr(b), _ptr(k), _ptr(q), code, int(flags), ntok, dk,
                                      _ptr(alpha), _ptr(beta), _ptr(kk), _ptr(qq))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_prologue failed with code {rc}")
    return alpha, beta, kk, qq


def _widen(x):
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def fwd_fused(q, k, v, a, b, h0=None, flags=GATES | NORM_K, want_o=True, nthreads=0):
    """fwd() after the per-token prologue: the recurrence runs on the fp64
    gates and unit vectors the prologue produces (v widened exactly)."""
    alpha, beta, kk, qq = prologue(a, b, k, q, flags)
    return fwd(qq, kk, _widen(v), alpha, beta, h0=h0, want_o=want_o, nthreads=nthreads)


def decode_fused(q, k, v, a, b, S, flags=GATES | NORM_K, nthreads=0):
    """decode() after the per-token prologue."""
    alpha, beta, kk, qq = prologue(a, b, k, q, flags)
    return decode(qq, kk, _widen(v), alpha, beta, S, nthreads=nthreads)


def bwd(q, k, v, alpha, beta, do, dhT=None, h0=None, nthreads=0):
    """Reverse-mode gradients of fwd() (ckda_oracle_bwd): given do = dL/do
    [B,H,T,dv] and dhT = dL/dH_T [B,H,dk,dv] (None: zero), returns fp64
    (dq, dk, dv, dalpha [B,H,T,dk or dv], dbeta [B,H,T], dh0 [B,H,dk,dv]).
    Inputs as fwd(); do and dhT float32 or float64 (one dtype)."""
    q, k, v, alpha, beta = (np.ascontiguousarray(x) for x in (q, k, v, alpha, beta))
    code = _code(q)
    for x in (k, v, alpha, beta):
        if _code(x) != code:
            raise TypeError("q, k, v, alpha, beta must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    do = np.ascontiguousarray(do)
    gcode = _code(do)
    if do.shape != (B, H, T, dv) or gcode == BF16:
        raise ValueError("do must be float32/float64 [B,H,T,dv]")
    dhTc = None
    if dhT is not None:
        dhTc = np.ascontiguousarray(dhT)
        if dhTc.shape != (B, H, dk, dv) or _code(dhTc) != gcode:
            raise ValueError("dhT must be [B,H,dk,dv] in do's dtype")
    h0c, h0code = None, F32
    if h0 is not None:
        h0c = np.ascontiguousarray(h0)
        h0code = _code(h0c)
    out = [np.empty((B, H, T, dk)), np.empty((B, H, T, dk)), np.empty((B, H, T, dv)), np.empty((B, H, T, dk)),
           np.empty((B, H, T)), np.empty((B, H, dk, dv))]
    rc = _load().ckda_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), code, _ptr(h0c), h0code,
                                 _ptr(do), _ptr(dhTc), gcode, *(_ptr(x) for x in out), B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_bwd failed with code {rc}")
    return tuple(out)


def prologue_bwd(a, b, k, q, flags, dalpha, dbeta, dk, dq):
    """Reverse mode of prologue() (ckda_oracle_prologue_bwd): the gradients
    with respect to a, b, k, q (the logits and raw vectors) from those with
    respect to its outputs alpha, beta, k, q (fp64 arrays of the same shapes).
    The sign of a gate is held constant and |tanh(a / 2)| takes the zero
    subgradient at 0.  Returns fp64 (da, db, dk, dq)."""
    a, b, k, q = (np.ascontiguousarray(x) for x in (a, b, k, q))
    code = _code(a)
    for x in (b, k, q):
        if _code(x) != code:
            raise TypeError("a, b, k, q must share one dtype")
    if k.shape != a.shape or q.shape != a.shape or b.shape != a.shape[:-1]:
        raise ValueError("inconsistent shapes")
    g = [np.ascontiguousarray(x, dtype=np.float64) for x in (dalpha, dbeta, dk, dq)]
    if g[0].shape != a.shape or g[1].shape != b.shape or g[2].shape != a.shape or g[3].shape != a.shape:
        raise ValueError("gradient shapes must match the prologue's outputs")
    dk_ = a.shape[-1]
    ntok = int(np.prod(a.shape[:-1], dtype=np.int64))
    da, dkr, dqr = (np.empty(a.shape, np.float64) for _ in range(3))
    db = np.empty(b.shape, np.float64)
    rc = _load().ckda_oracle_prologue_bwd(_ptr(a), _ptr(b), _ptr(k), _ptr(q), code, int(flags), ntok, dk_,
                                          *(_ptr(x) for x in g), _ptr(da), _ptr(db), _ptr(dkr), _ptr(dqr))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_prologue_bwd failed with code {rc}")
    return da, db, dkr, dqr


def bwd_fused(q, k, v, a, b, do, dhT=None, h0=None, flags=GATES | NORM_K, scalar=False, nthreads=0):
    """Gradients of fwd_fused() with respect to its raw inputs: prologue(),
    bwd() on what it produced, prologue_bwd().  With scalar, a is [B,H,T]
    (one gate logit per token and head, the same on every channel): its
    gradient sums the per-channel ones.  Returns fp64 (dq, dk, dv, da, db,
    dh0) for the raw q, k, v, a, b and h0."""
    a = np.ascontiguousarray(a)
    af = np.ascontiguousarray(np.broadcast_to(a[..., None], np.shape(k))) if scalar else a
    alpha, beta, kk, qq = prologue(af, b, k, q, flags)
    dq_, dk_, dv, dalpha, dbeta, dh0 = bwd(qq, kk, _widen(v), alpha, beta, do, dhT=dhT, h0=h0, nthreads=nthreads)
    da, db, dkr, dqr = prologue_bwd(af, b, k, q, flags, dalpha, dbeta, dk_, dq_)
    if scalar:
        da = da.sum(axis=-1)
    return dqr, dkr, dv, da, db, dh0


def deltaproduct2(q, k, v, alpha, beta, h0=None, nthreads=0):
    """DeltaProduct_2 forward in fp64 (ckda_oracle_deltaproduct2).

    q: [B,H,T,dk]; k: [B,H,T,2,dk]; v: [B,H,T,2,dv]; beta: [B,H,T,2];
    alpha: [B,H,T] scalar gates or None (ungated); one dtype.  h0 as fwd().
    Returns (o [B,H,T,dv], hT [B,H,dk,dv]) float64."""
    q, k, v, beta = (np.ascontiguousarray(x) for x in (q, k, v, beta))
    alpha = None if alpha is None else np.ascontiguousarray(alpha)
    code = _code(q)
    for x in (k, v, beta) + (() if alpha is None else (alpha,)):
        if _code(x) != code:
            raise TypeError("inputs must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, H, T, 2, dk) or v.shape != (B, H, T, 2, dv) or beta.shape != (B, H, T, 2) \
            or (alpha is not None and alpha.shape != (B, H, T)):
        raise ValueError("inconsistent shapes")
    h0c, h0code = None, F32
    if h0 is not None:
        h0c = np.ascontiguousarray(h0)
        if h0c.shape != (B, H, dk, dv):
            raise ValueError("h0 shape")
        h0code = _code(h0c)
    o = np.empty((B, H, T, dv), np.float64)
    hT = np.empty((B, H, dk, dv), np.float64)
    rc = _load().ckda_oracle_deltaproduct2(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), code, _ptr(h0c),
                                           h0code, _ptr(o), _ptr(hT), B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_deltaproduct2 failed with code {rc}")
    return o, hT


def deltaproduct2_bwd(q, k, v, alpha, beta, do, dhT=None, h0=None, nthreads=0):
    """Gradients of deltaproduct2() for L with dL/do = do [B,H,T,dv] and
    dL/dH_T = dhT (ckda_oracle_deltaproduct2_bwd: the adjoint of the token
    step, two Householder writes after the scalar gate, differentiated line
    by line in reverse).  Inputs as deltaproduct2(); do and dhT float32 or
    float64 (one dtype).  Returns fp64 (dq, dk [B,H,T,2,dk], dv [B,H,T,2,dv],
    dalpha [B,H,T] or None, dbeta [B,H,T,2], dh0)."""
    q, k, v, beta = (np.ascontiguousarray(x) for x in (q, k, v, beta))
    alpha = None if alpha is None else np.ascontiguousarray(alpha)
    code = _code(q)
    for x in (k, v, beta) + (() if alpha is None else (alpha,)):
        if _code(x) != code:
            raise TypeError("inputs must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if k.shape != (B, H, T, 2, dk) or v.shape != (B, H, T, 2, dv) or beta.shape != (B, H, T, 2) \
            or (alpha is not None and alpha.shape != (B, H, T)):
        raise ValueError("inconsistent shapes")
    do = np.ascontiguousarray(do)
    gcode = _code(do)
    if do.shape != (B, H, T, dv) or gcode == BF16:
        raise ValueError("do must be float32/float64 [B,H,T,dv]")
    dhTc = None
    if dhT is not None:
        dhTc = np.ascontiguousarray(dhT)
        if dhTc.shape != (B, H, dk, dv) or _code(dhTc) != gcode:
            raise ValueError("dhT must be [B,H,dk,dv] in do's dtype")
    h0c, h0code = None, F32
    if h0 is not None:
        h0c = np.ascontiguousarray(h0)
        h0code = _code(h0c)
    out = [np.empty((B, H, T, dk)), np.empty((B, H, T, 2, dk)), np.empty((B, H, T, 2, dv)),
           np.empty((B, H, T)) if alpha is not None else None, np.empty((B, H, T, 2)), np.empty((B, H, dk, dv))]
    rc = _load().ckda_oracle_deltaproduct2_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), code, _ptr(h0c),
                                               h0code, _ptr(do), _ptr(dhTc), gcode, *(_ptr(x) for x in out), B, H, T,
                                               dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_deltaproduct2_bwd failed with code {rc}")
    return tuple(out)


def deltaproduct2_bwd_substeps(q, k, v, alpha, beta, do, dhT=None, h0=None, nthreads=0):
    """The same gradients by a second route, kept as a cross-check of
    deltaproduct2_bwd(): DeltaProduct_2 is the delta rule over 2 T sub-steps
    (sub-step 2 t with the gate alpha_t on every channel, sub-step 2 t + 1
    ungated, only the odd sub-steps read out, with q_t), so bwd() on that
    sequence (queries repeated, gates [alpha_t, 1], upstream gradient
    [0, do_t]), then dq_t sums its two sub-steps and dalpha_t the channels of
    its gate.  Returns what deltaproduct2_bwd() returns."""
    B, H, T, dk = np.shape(q)
    dv = np.shape(v)[-1]
    q2 = np.repeat(_widen(q), 2, axis=2)
    a2 = np.ones((B, H, 2 * T, dk))
    if alpha is not None:
        a2[:, :, 0::2, :] = _widen(alpha)[..., None]
    do2 = np.zeros((B, H, 2 * T, dv))
    do2[:, :, 1::2, :] = np.asarray(do, np.float64)
    k2 = _widen(k).reshape(B, H, 2 * T, dk)
    v2 = _widen(v).reshape(B, H, 2 * T, dv)
    b2 = _widen(beta).reshape(B, H, 2 * T)
    dhT2 = None if dhT is None else np.asarray(dhT, np.float64)
    dq2, dk2, dv2, da2, db2, dh0 = bwd(q2, k2, v2, a2, b2, do2, dhT=dhT2, h0=h0, nthreads=nthreads)
    dq = dq2[:, :, 0::2, :] + dq2[:, :, 1::2, :]
    da = None if alpha is None else da2[:, :, 0::2, :].sum(axis=-1)
    return (dq, dk2.reshape(B, H, T, 2, dk), dv2.reshape(B, H, T, 2, dv), da, db2.reshape(B, H, T, 2), dh0)


def deltaproduct2_decode(q, k, v, alpha, beta, S):
    """One DeltaProduct_2 token applied in place to the fp64 state S [N,H,dk,dv].
    q [N,H,dk]; k [N,H,2,dk]; v [N,H,2,dv]; beta [N,H,2]; alpha [N,H] or None."""
    q, k, v, beta = (np.ascontiguousarray(x) for x in (q, k, v, beta))
    alpha = None if alpha is None else np.ascontiguousarray(alpha)
    N, H, dk = q.shape
    dv = v.shape[-1]
    if not (isinstance(S, np.ndarray) and S.dtype == np.float64 and S.flags.c_contiguous
            and S.shape == (N, H, dk, dv)):
        raise ValueError("S must be a C-contiguous float64 [N,H,dk,dv] array")
    o = np.empty((N, H, dv), np.float64)
    rc = _load().ckda_oracle_deltaproduct2_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _code(q),
                                                  _ptr(S), _ptr(o), N, H, dk, dv)
    if rc != 0:
        raise RuntimeError(f"ckda_oracle_deltaproduct2_decode failed with code {rc}")
    return o


class Variant:
    """An oracle bound to another build of ckda_oracle.c (same ABI).

    Used only by the mutation tests, which compile deliberately broken copies
    of the source to show that the pins catch each planted mistake."""

    def __init__(self, lib_path: str):
        self._path = lib_path

    def _swap(self, fn, *a, **kw):
        global _lib
        saved = _lib
        _lib = _declare(ctypes.CDLL(self._path))
        try:
            return fn(*a, **kw)
        finally:
            _lib = saved

    def fwd(self, *a, **kw):
        return self._swap(fwd, *a, **kw)

    def decode(self, *a, **kw):
        return self._swap(decode, *a, **kw)

    def prologue(self, *a, **kw):
        return self._swap(prologue, *a, **kw)

    def fwd_fused(self, *a, **kw):
        return self._swap(fwd_fused, *a, **kw)

    def deltaproduct2(self, *a, **kw):
        return self._swap(deltaproduct2, *a, **kw)

    def deltaproduct2_decode(self, *a, **kw):
        return self._swap(deltaproduct2_decode, *a, **kw)

    def bwd(self, *a, **kw):
        return self._swap(bwd, *a, **kw)

    def deltaproduct2_bwd(self, *a, **kw):
        return self._swap(deltaproduct2_bwd, *a, **kw)

    def prologue_bwd(self, *a, **kw):
        return self._swap(prologue_bwd, *a, **kw)

    def bwd_fused(self, *a, **kw):
        return self._swap(bwd_fused, *a, **kw)


def build_variant(source_text: str, out_path: str) -> "Variant":
    """Compile a modified copy of the oracle source (mutation tests only)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", src, "-o", out_path, "-lm"],
                   check=True)
    return Variant(out_path)


def source() -> str:
    with open(_SRC) as f:
        return f.read()
