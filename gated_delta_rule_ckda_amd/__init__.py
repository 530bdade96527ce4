"""MI355X (gfx950) CKDA / KDA kernels: Python binding of the C ABI in include/ckda.h.

Only argument marshalling happens here: torch supplies device memory and the
current HIP stream, and every step of the computation runs in the HIP
kernels of libckda.so.  There is no fallback: if the library is missing or
fails to load, every call raises.

    o, hT = chunk_fwd(q, k, v, alpha, beta, h0=None, chunk=64)
    o = decode_step(q, k, v, alpha, beta, H)          # H updated in place

With fuse=FUSE_GATES | FUSE_NORM_K (| FUSE_NORM_Q) the kernels first apply the
per-token prologue: alpha and beta are logits, keys (queries) are normalised.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libckda.so")

DTYPE_F32, DTYPE_BF16 = 0, 1
STATUS = {0: "CKDA_OK", 1: "CKDA_ERR_NULL", 2: "CKDA_ERR_DIM", 3: "CKDA_ERR_UNSUPPORTED",
          4: "CKDA_ERR_ALIAS", 5: "CKDA_ERR_HIP", 6: "CKDA_ERR_WORKSPACE", 7: "CKDA_ERR_FLAGS"}
(ERR_NULL, ERR_DIM, ERR_UNSUPPORTED, ERR_ALIAS, ERR_HIP, ERR_WORKSPACE, ERR_FLAGS) = range(1, 8)
FUSE_GATES, FUSE_NORM_K, FUSE_NORM_Q = 1, 2, 4       # CKDA_FUSE_*
GATE_SCALAR = 8                                      # CKDA_GATE_SCALAR
EXPORTS = ("ckda_chunk_fwd_workspace_size", "ckda_chunk_fwd", "ckda_chunk_fwd_noalloc", "ckda_chunk_fwd_timed",
           "ckda_chunk_fwd_ex",
           "ckda_chunk_fwd_gather", "ckda_decode_step", "ckda_decode_step_ex", "ckda_decode_step_gather",
           "ckda_deltaproduct2_fwd", "ckda_deltaproduct2_decode_step", "ckda_chunk_bwd",
           "ckda_chunk_bwd_workspace_size", "ckda_chunk_bwd_ex", "ckda_chunk_bwd_ex_workspace_size",
           "ckda_deltaproduct2_bwd", "ckda_deltaproduct2_bwd_workspace_size",
           "ckda_status_string", "ckda_last_error", "ckda_abi_version")

_lib = None


class CkdaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libckda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with gated_delta_rule_ckda_amd/build.py "
                               "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.ckda_chunk_fwd_workspace_size.argtypes = [i] * 7
        L.ckda_chunk_fwd_workspace_size.restype = sz
        L.ckda_chunk_fwd.argtypes = [vp] * 8 + [i] * 7 + [vp, sz, vp]
        L.ckda_chunk_fwd.restype = i
        L.ckda_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i] * 7 + [vp]
        L.ckda_chunk_fwd_noalloc.restype = i
        L.ckda_chunk_fwd_timed.argtypes = [vp] * 8 + [i] * 7 + [vp, sz, vp, vp, vp, vp]
        L.ckda_chunk_fwd_timed.restype = i
        L.ckda_chunk_fwd_ex.argtypes = [vp] * 8 + [i] * 8 + [vp, sz, vp]
        L.ckda_chunk_fwd_ex.restype = i
        L.ckda_chunk_fwd_gather.argtypes = [vp] * 8 + [i] * 4 + [vp] + [i] * 5 + [vp, sz, vp]
        L.ckda_chunk_fwd_gather.restype = i
        L.ckda_decode_step_gather.argtypes = [vp] * 7 + [i] * 3 + [vp] + [i] * 4 + [vp]
        L.ckda_decode_step_gather.restype = i
        L.ckda_deltaproduct2_fwd.argtypes = [vp] * 8 + [i] * 8 + [vp, sz, vp]
        L.ckda_deltaproduct2_fwd.restype = i
        L.ckda_deltaproduct2_decode_step.argtypes = [vp] * 7 + [i] * 6 + [vp]
        L.ckda_deltaproduct2_decode_step.restype = i
        L.ckda_chunk_bwd_workspace_size.argtypes = [i] * 6
        L.ckda_chunk_bwd_workspace_size.restype = sz
        L.ckda_chunk_bwd.argtypes = [vp] * 14 + [i] * 6 + [vp, sz, vp]
        L.ckda_chunk_bwd.restype = i
        L.ckda_chunk_bwd_ex_workspace_size.argtypes = [i] * 7
        L.ckda_chunk_bwd_ex_workspace_size.restype = sz
        L.ckda_chunk_bwd_ex.argtypes = [vp] * 14 + [i] * 7 + [vp, sz, vp]
        L.ckda_chunk_bwd_ex.restype = i
        L.ckda_deltaproduct2_bwd_workspace_size.argtypes = [i] * 6
        L.ckda_deltaproduct2_bwd_workspace_size.restype = sz
        L.ckda_deltaproduct2_bwd.argtypes = [vp] * 14 + [i] * 6 + [vp, sz, vp]
        L.ckda_deltaproduct2_bwd.restype = i
        L.ckda_decode_step.argtypes = [vp] * 7 + [i] * 5 + [vp]
        L.ckda_decode_step.restype = i
        L.ckda_decode_step_ex.argtypes = [vp] * 7 + [i] * 6 + [vp]
        L.ckda_decode_step_ex.restype = i
        L.ckda_status_string.argtypes = [i]
        L.ckda_status_string.restype = ctypes.c_char_p
        L.ckda_last_error.argtypes = []
        L.ckda_last_error.restype = ctypes.c_char_p
        L.ckda_abi_version.argtypes = []
        L.ckda_abi_version.restype = i
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise CkdaError(status, lib().ckda_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _require(ts, dtype):
    for name, t in ts.items():
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def _shapes(expect):
    """Raise ValueError unless every given tensor has exactly its expected
    shape.  The C ABI receives bare pointers and cannot see shapes, so this is
    the only guard against a wrong-shaped tensor turning into out-of-bounds
    device reads or writes; it runs before anything else touches the
    tensors.  `expect` maps a name to (tensor or None, shape tuple)."""
    for name, (t, shape) in expect.items():
        if t is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(t, n, name):
    if t.dim() != n:
        raise ValueError(f"{name} must have {n} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _scratch(nbytes, device, stream):
    """A temporary uint8 workspace for one call.  It is allocated from torch's
    caching allocator; when the kernels run on another stream than the
    current one, the allocation is tied to that stream too, so that it is not
    handed out again before those kernels are done with it."""
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(device):
        ws.record_stream(stream)
    return ws


def workspace_size(B, H, T, dk, dv, chunk, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(lib().ckda_chunk_fwd_workspace_size(B, H, T, dk, dv, chunk, code))


def chunk_fwd(q, k, v, alpha, beta, h0=None, chunk=64, workspace=None, o=None, hT=None,
              want_state=True, stream=None, events=None, fuse=0, idx=None):
    """Chunkwise forward.  q, k, alpha [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T];
    h0 [B,H,dk,dv] fp32 or None.  Returns (o [B,H,T,dv], hT [B,H,dk,dv] fp32 or None).

    `workspace` (uint8 GPU tensor of at least workspace_size() bytes), `o` and
    `hT` may be passed in to avoid allocations (e.g. in timed loops).
    `events`, three recorded-once torch.cuda.Event objects (or None), are
    recorded before the Gram kernel, between the kernels and after the
    state-pass kernel (ckda_chunk_fwd_timed).  `fuse` (FUSE_* bits) applies
    the per-token prologue (ckda_chunk_fwd_ex); it cannot be combined with
    `events`.  `idx` ([H, dk] int32 GPU tensor) gathers each head's retained
    key channels from full-width q, k, alpha rows [B,H,T,dk_in] inside the
    kernels (ckda_chunk_fwd_gather); states then have dk rows."""
    B, H, T, dk = _dims(q, 4, "q")
    dk_in = dk
    if idx is not None:
        if idx.dim() != 2 or idx.shape[0] != H:
            raise ValueError(f"idx must be [H, dk], got {tuple(idx.shape)}")
        dk = idx.shape[1]
    dv = _dims(v, 4, "v")[-1]
    scalar = bool(fuse & GATE_SCALAR)
    _shapes(dict(k=(k, (B, H, T, dk_in)), v=(v, (B, H, T, dv)),
                 alpha=(alpha, (B, H, T) if scalar else (B, H, T, dk_in)), beta=(beta, (B, H, T)),
                 h0=(h0, (B, H, dk, dv)), o=(o, (B, H, T, dv)), hT=(hT, (B, H, dk, dv))))
    _require(dict(q=q, k=k, v=v, alpha=alpha, beta=beta), q.dtype)
    if idx is not None:
        _require(dict(idx=idx), torch.int32)
    code = _dtype_code(q)
    if h0 is not None:
        _require(dict(h0=h0), torch.float32)
    if o is not None:
        _require(dict(o=o), q.dtype)
    if hT is not None:
        _require(dict(hT=hT), torch.float32)
    need = workspace_size(B, H, T, dk, dv, chunk, code)
    if need == 0:
        raise CkdaError(ERR_UNSUPPORTED, f"unsupported sizes dk={dk} dv={dv} chunk={chunk}")
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if hT is None and want_state:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(o), _ptr(hT),
            B, H, T, dk, dv, chunk, code, _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    if idx is not None:
        if events is not None:
            raise ValueError("events are recorded by the plain forward only")
        _check(lib().ckda_chunk_fwd_gather(*args[:11], dk_in, _ptr(idx), *args[11:15], int(fuse), *args[15:]))
    elif fuse:
        if events is not None:
            raise ValueError("events are recorded by the plain forward only (fuse=0)")
        args = args[:15] + (int(fuse),) + args[15:]
        _check(lib().ckda_chunk_fwd_ex(*args))
    elif events is None:
        _check(lib().ckda_chunk_fwd(*args))
    else:
        handles = [None if e is None else ctypes.c_void_p(e.cuda_event) for e in events]
        _check(lib().ckda_chunk_fwd_timed(*args, *handles))
    return o, hT


def chunk_fwd_noalloc(q, k, v, alpha, beta, h0, o, hT=None, chunk=64, stream=None):
    """ckda_chunk_fwd_noalloc: the chunkwise forward with no workspace and no
    allocation (for callers that cannot allocate, e.g. under graph capture).
    The caller passes the outputs o [B,H,T,dv] and hT [B,H,dk,dv] fp32 (or
    None).  Calls that overlap in time on one GPU share its fixed scratch and
    race; calls on one stream are safe.  Returns (o, hT)."""
    B, H, T, dk = _dims(q, 4, "q")
    dv = _dims(v, 4, "v")[-1]
    if o is None:
        raise ValueError("o is required (this entry point allocates nothing)")
    _shapes(dict(k=(k, (B, H, T, dk)), v=(v, (B, H, T, dv)), alpha=(alpha, (B, H, T, dk)), beta=(beta, (B, H, T)),
                 h0=(h0, (B, H, dk, dv)), o=(o, (B, H, T, dv)), hT=(hT, (B, H, dk, dv))))
    _require(dict(q=q, k=k, v=v, alpha=alpha, beta=beta, o=o), q.dtype)
    for name, t in (("h0", h0), ("hT", hT)):
        if t is not None:
            _require({name: t}, torch.float32)
    _check(lib().ckda_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(o),
                                        _ptr(hT), B, H, T, dk, dv, chunk, _dtype_code(q), _stream(stream)))
    return o, hT


def decode_step(q, k, v, alpha, beta, H, o=None, stream=None, fuse=0, idx=None):
    """One decode step.  q, k, alpha [N,Hh,dk]; v [N,Hh,dv]; beta [N,Hh];
    H [N,Hh,dk,dv] fp32 updated in place.  Returns o [N,Hh,dv].  `fuse`
    (FUSE_* bits) applies the per-token prologue first (ckda_decode_step_ex).
    `idx` ([Hh, dk] int32) gathers retained key channels from rows of dk_in
    (ckda_decode_step_gather)."""
    N, Hh, dk = _dims(q, 3, "q")
    dk_in = dk
    if idx is not None:
        if idx.dim() != 2 or idx.shape[0] != Hh:
            raise ValueError(f"idx must be [H, dk], got {tuple(idx.shape)}")
        dk = idx.shape[1]
    dv = _dims(v, 3, "v")[-1]
    scalar = bool(fuse & GATE_SCALAR)
    _shapes(dict(k=(k, (N, Hh, dk_in)), v=(v, (N, Hh, dv)), alpha=(alpha, (N, Hh) if scalar else (N, Hh, dk_in)),
                 beta=(beta, (N, Hh)), H=(H, (N, Hh, dk, dv)), o=(o, (N, Hh, dv))))
    _require(dict(q=q, k=k, v=v, alpha=alpha, beta=beta), q.dtype)
    _require(dict(H=H), torch.float32)
    if idx is not None:
        _require(dict(idx=idx), torch.int32)
    if o is not None:
        _require(dict(o=o), q.dtype)
    code = _dtype_code(q)
    if o is None:
        o = torch.empty((N, Hh, dv), dtype=q.dtype, device=q.device)
    ptrs = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(H), _ptr(o))
    if idx is not None:
        _check(lib().ckda_decode_step_gather(*ptrs, N, Hh, dk_in, _ptr(idx), dk, dv, code, int(fuse), _stream(stream)))
    elif fuse:
        _check(lib().ckda_decode_step_ex(*ptrs, N, Hh, dk, dv, code, int(fuse), _stream(stream)))
    else:
        _check(lib().ckda_decode_step(*ptrs, N, Hh, dk, dv, code, _stream(stream)))
    return o


def deltaproduct2_fwd(q, k, v, beta, alpha=None, h0=None, chunk=64, workspace=None, o=None, hT=None,
                      want_state=True, stream=None, fuse=0):
    """DeltaProduct_2 forward (ckda_deltaproduct2_fwd): q [B,H,T,dk];
    k [B,H,T,2,dk]; v [B,H,T,2,dv]; beta [B,H,T,2]; alpha [B,H,T] scalar
    gates or None (ungated); h0 [B,H,dk,dv] fp32 or None.  Returns (o, hT)."""
    B, H, T, dk = _dims(q, 4, "q")
    dv = _dims(v, 5, "v")[-1]
    _shapes(dict(k=(k, (B, H, T, 2, dk)), v=(v, (B, H, T, 2, dv)), beta=(beta, (B, H, T, 2)),
                 alpha=(alpha, (B, H, T)), h0=(h0, (B, H, dk, dv)), o=(o, (B, H, T, dv)), hT=(hT, (B, H, dk, dv))))
    ts = dict(q=q, k=k, v=v, beta=beta)
    if alpha is not None:
        ts["alpha"] = alpha
    if o is not None:
        ts["o"] = o
    _require(ts, q.dtype)
    code = _dtype_code(q)
    for name, t in (("h0", h0), ("hT", hT)):
        if t is not None:
            _require({name: t}, torch.float32)
    need = workspace_size(B, H, 2 * T, dk, dv, chunk, code)
    if need == 0:
        raise CkdaError(ERR_UNSUPPORTED, f"unsupported sizes dk={dk} dv={dv} chunk={chunk}")
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if hT is None and want_state:
        hT = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    _check(lib().ckda_deltaproduct2_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(o),
                                        _ptr(hT), B, H, T, dk, dv, chunk, code, int(fuse), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return o, hT


def deltaproduct2_decode_step(q, k, v, beta, H, alpha=None, o=None, stream=None, fuse=0):
    """One DeltaProduct_2 decode step: q [N,Hh,dk]; k [N,Hh,2,dk];
    v [N,Hh,2,dv]; beta [N,Hh,2]; alpha [N,Hh] or None; H fp32 in place."""
    N, Hh, dk = _dims(q, 3, "q")
    dv = _dims(v, 4, "v")[-1]
    _shapes(dict(k=(k, (N, Hh, 2, dk)), v=(v, (N, Hh, 2, dv)), beta=(beta, (N, Hh, 2)), alpha=(alpha, (N, Hh)),
                 H=(H, (N, Hh, dk, dv)), o=(o, (N, Hh, dv))))
    ts = dict(q=q, k=k, v=v, beta=beta)
    if alpha is not None:
        ts["alpha"] = alpha
    if o is not None:
        ts["o"] = o
    _require(ts, q.dtype)
    _require(dict(H=H), torch.float32)
    code = _dtype_code(q)
    if o is None:
        o = torch.empty((N, Hh, dv), dtype=q.dtype, device=q.device)
    _check(lib().ckda_deltaproduct2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(H), _ptr(o),
                                                N, Hh, dk, dv, code, int(fuse), _stream(stream)))
    return o


def bwd_workspace_size(B, H, T, dk, dv, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(lib().ckda_chunk_bwd_workspace_size(B, H, T, dk, dv, code))


def bwd_ex_workspace_size(B, H, T, dk, dv, dtype, flags) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(lib().ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, code, int(flags)))


def chunk_bwd(q, k, v, alpha, beta, do, h0=None, dhT=None, want_dh0=True, workspace=None, stream=None, fuse=0):
    """Backward of chunk_fwd (ckda_chunk_bwd): given do = dL/do [B,H,T,dv]
    (input dtype) and dhT = dL/dH_T [B,H,dk,dv] fp32 or None, returns fp32
    (dq, dk, dv, dalpha, dbeta, dh0 or None).  With `fuse` (FUSE_* and
    GATE_SCALAR bits, ckda_chunk_bwd_ex) the inputs are those of the fused
    forward and the gradients are with respect to them: logits, raw keys
    and queries; with GATE_SCALAR alpha and dalpha are [B,H,T]."""
    B, H, T, dk = _dims(q, 4, "q")
    dv = _dims(v, 4, "v")[-1]
    _shapes(dict(k=(k, (B, H, T, dk)), alpha=(alpha, (B, H, T) if fuse & GATE_SCALAR else (B, H, T, dk)),
                 beta=(beta, (B, H, T)), do=(do, (B, H, T, dv)), h0=(h0, (B, H, dk, dv)), dhT=(dhT, (B, H, dk, dv))))
    _require(dict(q=q, k=k, v=v, alpha=alpha, beta=beta, do=do), q.dtype)
    code = _dtype_code(q)
    if h0 is not None:
        _require(dict(h0=h0), torch.float32)
    if dhT is not None:
        _require(dict(dhT=dhT), torch.float32)
    need = bwd_ex_workspace_size(B, H, T, dk, dv, code, fuse) if fuse else bwd_workspace_size(B, H, T, dk, dv, code)
    if need == 0:
        raise CkdaError(ERR_UNSUPPORTED, f"unsupported sizes dk={dk} dv={dv} or flags {fuse}")
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    f32 = dict(dtype=torch.float32, device=q.device)
    gq, gk = (torch.empty((B, H, T, dk), **f32) for _ in range(2))
    galpha = torch.empty((B, H, T) if fuse & GATE_SCALAR else (B, H, T, dk), **f32)
    gv = torch.empty((B, H, T, dv), **f32)
    gbeta = torch.empty((B, H, T), **f32)
    gh0 = torch.empty((B, H, dk, dv), **f32) if want_dh0 else None
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dhT),
            _ptr(gq), _ptr(gk), _ptr(gv), _ptr(galpha), _ptr(gbeta), _ptr(gh0), B, H, T, dk, dv, code)
    tail = (_ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    if fuse:
        _check(lib().ckda_chunk_bwd_ex(*args, int(fuse), *tail))
    else:
        _check(lib().ckda_chunk_bwd(*args, *tail))
    return gq, gk, gv, galpha, gbeta, gh0


def deltaproduct2_bwd(q, k, v, alpha, beta, do, h0=None, dhT=None, want_dh0=True, workspace=None, stream=None):
    """Backward of deltaproduct2_fwd (ckda_deltaproduct2_bwd): q [B,H,T,dk],
    k [B,H,T,2,dk], v [B,H,T,2,dv], beta [B,H,T,2], alpha [B,H,T] or None,
    do [B,H,T,dv] (input dtype), dhT fp32 or None.  Returns fp32 (dq, dk, dv,
    dalpha or None, dbeta, dh0 or None) in the inputs' shapes."""
    B, H, T, dk = _dims(q, 4, "q")
    dv = _dims(v, 5, "v")[-1]
    _shapes(dict(k=(k, (B, H, T, 2, dk)), v=(v, (B, H, T, 2, dv)), beta=(beta, (B, H, T, 2)),
                 alpha=(alpha, (B, H, T)), do=(do, (B, H, T, dv)), h0=(h0, (B, H, dk, dv)),
                 dhT=(dhT, (B, H, dk, dv))))
    ts = dict(q=q, k=k, v=v, beta=beta, do=do)
    if alpha is not None:
        ts["alpha"] = alpha
    _require(ts, q.dtype)
    code = _dtype_code(q)
    for name, t in (("h0", h0), ("dhT", dhT)):
        if t is not None:
            _require({name: t}, torch.float32)
    need = int(lib().ckda_deltaproduct2_bwd_workspace_size(B, H, T, dk, dv, code))
    if need == 0:
        raise CkdaError(ERR_UNSUPPORTED, f"unsupported sizes dk={dk} dv={dv}")
    if workspace is None:
        workspace = _scratch(need, q.device, stream)
    f32 = dict(dtype=torch.float32, device=q.device)
    gq = torch.empty((B, H, T, dk), **f32)
    gk = torch.empty((B, H, T, 2, dk), **f32)
    gv = torch.empty((B, H, T, 2, dv), **f32)
    galpha = torch.empty((B, H, T), **f32) if alpha is not None else None
    gbeta = torch.empty((B, H, T, 2), **f32)
    gh0 = torch.empty((B, H, dk, dv), **f32) if want_dh0 else None
    _check(lib().ckda_deltaproduct2_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0), _ptr(do),
                                        _ptr(dhT), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(galpha), _ptr(gbeta), _ptr(gh0),
                                        B, H, T, dk, dv, code, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))
    return gq, gk, gv, galpha, gbeta, gh0
