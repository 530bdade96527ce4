"""Seeded synthetic inputs for the CKDA chunkwise forward and decode step.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the recurrence's arithmetic; the tests hand the same bytes
to the GPU library and to the fp64 oracle.

Workloads (shapes and value laws of the pages' settings: 16 heads at
d_k = d_v = 128 and 2k-32k lengths in the "Complex KDA" throughput figure,
Fig. 5; key/query channel selection halving d_k in the state-reduction slides;
KDA ranges alpha in (0,1], beta in [0,1] and CKDA ranges alpha in [-1,1],
beta in [0,2], "Complex KDA" Sec. 3):

* ``tiny_fp32``        B1 H1 T64 d_k=d_v=16 chunk 16, fp32, alpha~U[-1,1], beta~U[0,2], h0=0
* ``kda_bf16``         B4 H16 T2048 d128 chunk 64, bf16, alpha=sigmoid(N(2,1)), beta=sigmoid(N(0,1)), h0=0
* ``ckda_bf16``        B4 H16 T4096 d128 chunk 64, bf16, alpha=tanh(N(0,1.5)), beta=2 sigmoid(N(0,1)), h0~N(0,0.1) fp32
* ``ckda_long_dk64``   B2 H32 T32768 d_k=64 d_v=128 chunk 64, bf16, gates as ckda_bf16, h0=0
* decode               256 sequences x 32 heads, d128, 128 steps, bf16 inputs,
                       alpha~U[-1,1], beta~U[0,2], fp32 state ~N(0,0.1)

The fused prologue's inputs (make_logit_inputs, decode_logit_inputs) are
logits and unnormalised vectors of the same shapes; the comparators' inputs
(make_scalar_gate_inputs: one gate per token and head; make_dp2_inputs and
dp2_decode_inputs: two keys, values and betas per token) follow the same laws.

N(mu, s) means standard deviation s.  Draw order per workload: q, k, v, alpha,
beta, h0, each as a full C-order float32 array from numpy's PCG64 stream
seeded with the workload's seed.  k is L2-normalised per (b, h, t) in fp32
before rounding.  bf16 rounding is round-to-nearest-even (torch).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int
    dtype: str          # "f32" or "bf16"
    gates: str          # gate law, see _gates()
    h0: str             # "zero", "none" or "normal"
    seed: int


WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 1, 1, 64, 16, 16, 16, "f32", "ckda_uniform", "zero", 1001),
    "kda_bf16": Workload("kda_bf16", 4, 16, 2048, 128, 128, 64, "bf16", "kda", "zero", 1002),
    "ckda_bf16": Workload("ckda_bf16", 4, 16, 4096, 128, 128, 64, "bf16", "ckda_tanh", "normal", 1003),
    "ckda_long_dk64": Workload("ckda_long_dk64", 2, 32, 32768, 64, 128, 64, "bf16", "ckda_tanh", "zero", 1004),
}


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: str
    state_seed: int
    step_seed: int


DECODE = DecodeWorkload("decode_n256_h32_d128", 256, 32, 128, 128, 128, "bf16", 1005, 5000)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _gates(rng, law: str, shape_a, shape_b):
    """Draw (alpha, beta) as float32 arrays following the named law."""
    if law == "ckda_uniform":
        a = rng.uniform(-1.0, 1.0, size=shape_a).astype(np.float32)
        b = rng.uniform(0.0, 2.0, size=shape_b).astype(np.float32)
    elif law == "kda":
        a = _sigmoid(rng.standard_normal(shape_a, dtype=np.float32) + np.float32(2.0))
        b = _sigmoid(rng.standard_normal(shape_b, dtype=np.float32))
    elif law == "ckda_tanh":
        a = np.tanh(np.float32(1.5) * rng.standard_normal(shape_a, dtype=np.float32))
        b = np.float32(2.0) * _sigmoid(rng.standard_normal(shape_b, dtype=np.float32))
    elif law == "zero_and_unit":
        # Stress law: gates exactly in {-1, 0, +1} mixed with U[-1,1]; beta in {0, 1, 2}.
        a = rng.uniform(-1.0, 1.0, size=shape_a).astype(np.float32)
        pick = rng.integers(0, 5, size=shape_a)
        a = np.where(pick == 0, np.float32(0.0), a)
        a = np.where(pick == 1, np.float32(1.0), a)
        a = np.where(pick == 2, np.float32(-1.0), a)
        b = rng.integers(0, 3, size=shape_b).astype(np.float32)
    elif law == "orthogonal":
        # beta = 2 and alpha in {-1, +1}: every transition is orthogonal.
        a = np.where(rng.integers(0, 2, size=shape_a) == 0, -1.0, 1.0).astype(np.float32)
        b = np.full(shape_b, 2.0, np.float32)
    elif law == "mild_overrange":
        # Range violation: |alpha| up to 1.25 (outside the CKDA range), beta ~ U[0, 2].
        a = rng.uniform(-1.25, 1.25, size=shape_a).astype(np.float32)
        b = rng.uniform(0.0, 2.0, size=shape_b).astype(np.float32)
    elif law == "small_gates":
        # Stress law: |alpha| spread log-uniformly down to 1e-12 with random signs.
        mag = np.exp(rng.uniform(np.log(1e-12), 0.0, size=shape_a)).astype(np.float32)
        sgn = np.where(rng.integers(0, 2, size=shape_a) == 0, -1.0, 1.0).astype(np.float32)
        a = mag * sgn
        b = rng.uniform(0.0, 2.0, size=shape_b).astype(np.float32)
    else:
        raise ValueError(f"unknown gate law {law!r}")
    return a, b


def _normalise(k):
    n = np.sqrt(np.sum(k.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    n = np.maximum(n, np.float32(1e-30))
    return (k / n).astype(np.float32)


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch_dtype(dtype)).contiguous()


def make_inputs(w: Workload, repeated_keys: bool = False, keys: str = "normal", values: str = "normal"):
    """Return dict(q, k, v, alpha, beta, h0) of CPU torch tensors for workload w.

    q, k, v, alpha, beta are in w.dtype; h0 is float32 [B,H,dk,dv] or None.
    Stress options (the same random draws, transformed):
      repeated_keys / keys="repeated": every token of a head reuses one key
        (worst conditioning of the intra-chunk triangular system);
      keys="near_parallel": token t's key is normalise(k_0 + 1e-3 k_t) with
        the head's first draw k_0 and its own draw k_t (distinct, nearly
        parallel unit keys);
      values="zero": v = 0 (with beta = 2 and alpha = +-1 every step is then
        an orthogonal map of the state, which keeps its Frobenius norm).
    """
    rng = np.random.default_rng(w.seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    k = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    if repeated_keys or keys == "repeated":
        k = np.broadcast_to(k[:, :, :1, :], k.shape).copy()
    elif keys == "near_parallel":
        k = k[:, :, :1, :] + np.float32(1e-3) * k
    elif keys != "normal":
        raise ValueError(f"unknown key law {keys!r}")
    k = _normalise(k)
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    if values == "zero":
        v = np.zeros_like(v)
    elif values != "normal":
        raise ValueError(f"unknown value law {values!r}")
    a, b = _gates(rng, w.gates, (B, H, T, dk), (B, H, T))
    if w.h0 == "normal":
        h0 = torch.from_numpy(np.float32(0.1) * rng.standard_normal((B, H, dk, dv), dtype=np.float32))
    elif w.h0 == "zero":
        h0 = torch.zeros((B, H, dk, dv), dtype=torch.float32)
    elif w.h0 == "none":
        h0 = None
    else:
        raise ValueError(w.h0)
    return dict(q=_to(q, w.dtype), k=_to(k, w.dtype), v=_to(v, w.dtype),
                alpha=_to(a, w.dtype), beta=_to(b, w.dtype), h0=h0)


def make_logit_inputs(w: Workload, zero_rows: float = 0.0):
    """Inputs for the fused prologue: dict(q, k, v, a, b, h0) of CPU tensors.

    a, b are logits of alpha and beta (a ~ N(0, 3): gates from the e^-5 floor
    to 1 with both signs; b ~ N(0, 1.5)); q and k are N(0, 1) and NOT
    normalised.  zero_rows: fraction of (b, h, t) whose key and query rows are
    all zero (exercises the zero-vector guard).  w.gates is ignored.
    Draw order: q, k, v, a, b, zero mask, h0."""
    rng = np.random.default_rng(w.seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    k = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    a = np.float32(3.0) * rng.standard_normal((B, H, T, dk), dtype=np.float32)
    bl = np.float32(1.5) * rng.standard_normal((B, H, T), dtype=np.float32)
    zero = rng.uniform(size=(B, H, T, 1)) < zero_rows
    q = np.where(zero, np.float32(0.0), q)
    k = np.where(zero, np.float32(0.0), k)
    if w.h0 == "normal":
        h0 = torch.from_numpy(np.float32(0.1) * rng.standard_normal((B, H, dk, dv), dtype=np.float32))
    elif w.h0 == "zero":
        h0 = torch.zeros((B, H, dk, dv), dtype=torch.float32)
    else:
        h0 = None
    return dict(q=_to(q, w.dtype), k=_to(k, w.dtype), v=_to(v, w.dtype),
                alpha=_to(a, w.dtype), beta=_to(bl, w.dtype), h0=h0)


def decode_logit_inputs(step: int, d: DecodeWorkload = DECODE, N=None, H=None):
    """Decode-step inputs for the fused prologue (laws of make_logit_inputs)."""
    N = d.N if N is None else N
    H = d.H if H is None else H
    rng = np.random.default_rng(d.step_seed + step)
    q = rng.standard_normal((N, H, d.dk), dtype=np.float32)
    k = rng.standard_normal((N, H, d.dk), dtype=np.float32)
    v = rng.standard_normal((N, H, d.dv), dtype=np.float32)
    a = np.float32(3.0) * rng.standard_normal((N, H, d.dk), dtype=np.float32)
    bl = np.float32(1.5) * rng.standard_normal((N, H), dtype=np.float32)
    return dict(q=_to(q, d.dtype), k=_to(k, d.dtype), v=_to(v, d.dtype),
                alpha=_to(a, d.dtype), beta=_to(bl, d.dtype))


def retained_channels(H: int, dk_in: int, dk: int, seed: int) -> torch.Tensor:
    """A per-head retained channel set [H, dk] int32: dk distinct channels of
    dk_in per head, drawn uniformly (a stand-in for a calibrated selection),
    in increasing order."""
    rng = np.random.default_rng(seed)
    idx = np.stack([np.sort(rng.choice(dk_in, dk, replace=False)) for _ in range(H)])
    return torch.from_numpy(idx.astype(np.int32))


def make_gather_inputs(w: Workload, dk_in: int, idx: torch.Tensor):
    """Full-width inputs for the channel gather: dict(q, k, v, alpha, beta, h0)
    with q, k, alpha [B, H, T, dk_in] (w.dk is the kept width).  Laws as
    make_inputs; the kept channels of each key row have unit norm, the others
    are N(0, 1).  Draw order: q, k, v, alpha, beta, h0."""
    rng = np.random.default_rng(w.seed)
    B, H, T, dv = w.B, w.H, w.T, w.dv
    q = rng.standard_normal((B, H, T, dk_in), dtype=np.float32)
    k = rng.standard_normal((B, H, T, dk_in), dtype=np.float32)
    ix = idx.numpy().astype(np.int64)
    for h in range(H):
        k[:, h][..., ix[h]] = _normalise(k[:, h][..., ix[h]])
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    a, b = _gates(rng, w.gates, (B, H, T, dk_in), (B, H, T))
    if w.h0 == "normal":
        h0 = torch.from_numpy(np.float32(0.1) * rng.standard_normal((B, H, w.dk, dv), dtype=np.float32))
    elif w.h0 == "zero":
        h0 = torch.zeros((B, H, w.dk, dv), dtype=torch.float32)
    else:
        h0 = None
    return dict(q=_to(q, w.dtype), k=_to(k, w.dtype), v=_to(v, w.dtype),
                alpha=_to(a, w.dtype), beta=_to(b, w.dtype), h0=h0)


def gather_channels(x: torch.Tensor, idx: torch.Tensor) -> torch.Tensor:
    """x[b, h, ..., idx[h]] for x [B, H, ..., dk_in] (CPU; for the oracle side)."""
    out = [x[:, h][..., idx[h].long()] for h in range(x.shape[1])]
    return torch.stack(out, dim=1).contiguous()


def make_scalar_gate_inputs(w: Workload):
    """Inputs with one gate per token and head (Gated DeltaNet's scalar gate):
    dict(q, k, v, alpha [B,H,T], beta, h0); laws as make_inputs with the gate
    law applied to the [B,H,T] scalars.  Draw order: q, k, v, alpha, beta, h0."""
    rng = np.random.default_rng(w.seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    k = _normalise(rng.standard_normal((B, H, T, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, dv), dtype=np.float32)
    a, b = _gates(rng, w.gates, (B, H, T), (B, H, T))
    h0 = _h0(rng, w)
    return dict(q=_to(q, w.dtype), k=_to(k, w.dtype), v=_to(v, w.dtype),
                alpha=_to(a, w.dtype), beta=_to(b, w.dtype), h0=h0)


def make_dp2_inputs(w: Workload, gated: bool = True):
    """DeltaProduct_2 inputs: dict(q [B,H,T,dk], k [B,H,T,2,dk] unit rows,
    v [B,H,T,2,dv], alpha [B,H,T] scalar gates (None when not gated),
    beta [B,H,T,2], h0).  Gate law w.gates on the scalars and on beta.
    Draw order: q, k, v, alpha, beta, h0."""
    rng = np.random.default_rng(w.seed)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q = rng.standard_normal((B, H, T, dk), dtype=np.float32)
    k = _normalise(rng.standard_normal((B, H, T, 2, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, T, 2, dv), dtype=np.float32)
    a, b = _gates(rng, w.gates, (B, H, T), (B, H, T, 2))
    h0 = _h0(rng, w)
    return dict(q=_to(q, w.dtype), k=_to(k, w.dtype), v=_to(v, w.dtype),
                alpha=_to(a, w.dtype) if gated else None, beta=_to(b, w.dtype), h0=h0)


def _h0(rng, w: Workload):
    if w.h0 == "normal":
        return torch.from_numpy(np.float32(0.1) * rng.standard_normal((w.B, w.H, w.dk, w.dv), dtype=np.float32))
    if w.h0 == "zero":
        return torch.zeros((w.B, w.H, w.dk, w.dv), dtype=torch.float32)
    return None


def dp2_decode_inputs(step: int, d: DecodeWorkload = DECODE, N=None, H=None, gated: bool = True):
    """DeltaProduct_2 decode-step inputs: q [N,H,dk], k [N,H,2,dk] unit rows,
    v [N,H,2,dv], beta [N,H,2] ~ U[0,2], alpha [N,H] ~ U[-1,1] (or None)."""
    N = d.N if N is None else N
    H = d.H if H is None else H
    rng = np.random.default_rng(d.step_seed + step)
    q = rng.standard_normal((N, H, d.dk), dtype=np.float32)
    k = _normalise(rng.standard_normal((N, H, 2, d.dk), dtype=np.float32))
    v = rng.standard_normal((N, H, 2, d.dv), dtype=np.float32)
    a, b = _gates(rng, "ckda_uniform", (N, H), (N, H, 2))
    return dict(q=_to(q, d.dtype), k=_to(k, d.dtype), v=_to(v, d.dtype),
                alpha=_to(a, d.dtype) if gated else None, beta=_to(b, d.dtype))


def make_output_grads(w: Workload, seed: int):
    """Upstream gradients for the backward: do ~ N(0, 1) [B,H,T,dv] in w.dtype
    and dhT ~ N(0, 0.1) [B,H,dk,dv] fp32 (draw order: do, dhT)."""
    rng = np.random.default_rng(seed)
    do = rng.standard_normal((w.B, w.H, w.T, w.dv), dtype=np.float32)
    dhT = np.float32(0.1) * rng.standard_normal((w.B, w.H, w.dk, w.dv), dtype=np.float32)
    return _to(do, w.dtype), torch.from_numpy(dhT)


def decode_state(d: DecodeWorkload = DECODE, N=None, H=None):
    """Initial fp32 decode state [N,H,dk,dv] ~ N(0, 0.1)."""
    N = d.N if N is None else N
    H = d.H if H is None else H
    rng = np.random.default_rng(d.state_seed)
    return torch.from_numpy(np.float32(0.1) * rng.standard_normal((N, H, d.dk, d.dv), dtype=np.float32))


def decode_step_inputs(step: int, d: DecodeWorkload = DECODE, N=None, H=None, gates="ckda_uniform"):
    """Inputs of decode step `step`: dict(q, k, v, alpha, beta) CPU tensors in d.dtype."""
    N = d.N if N is None else N
    H = d.H if H is None else H
    rng = np.random.default_rng(d.step_seed + step)
    q = rng.standard_normal((N, H, d.dk), dtype=np.float32)
    k = _normalise(rng.standard_normal((N, H, d.dk), dtype=np.float32))
    v = rng.standard_normal((N, H, d.dv), dtype=np.float32)
    a, b = _gates(rng, gates, (N, H, d.dk), (N, H))
    return dict(q=_to(q, d.dtype), k=_to(k, d.dtype), v=_to(v, d.dtype),
                alpha=_to(a, d.dtype), beta=_to(b, d.dtype))


def raw(t: torch.Tensor) -> np.ndarray:
    """The exact element bytes of a CPU tensor as numpy (bf16 -> uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def variant(w: Workload, **kw) -> Workload:
    """A copy of workload w with some fields replaced (smaller T, other gates...)."""
    return replace(w, **kw)
