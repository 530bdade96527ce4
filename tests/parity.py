"""Shared helpers for the GPU parity tests: the error metric, oracle runners on
the exact bytes handed to the GPU, and case logging.

Metric (per output tensor): for every (batch, head) slice, max |x - y| divided
by max |y| of that slice; the reported error is the maximum over slices.
Tolerances: 1e-4 for fp32 inputs, 2e-2 for bf16 inputs (fp32 states).
Logged beside it, for information: the elementwise relative error
|x - y| / max(|y|, 1e-3 max|y|), the floor taken per slice, maximised over
all elements.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from gated_delta_rule_ckda_amd.inputs import raw

TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def slice_rel_err(x, y) -> float:
    """max over leading (batch, head) slices of max|x-y| / max|y|."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    lead = x.shape[:2]
    xs = x.reshape(int(np.prod(lead)), -1)
    ys = y.reshape(int(np.prod(lead)), -1)
    num = np.max(np.abs(xs - ys), axis=1)
    den = np.max(np.abs(ys), axis=1)
    den = np.where(den == 0, 1.0, den)
    if not np.all(np.isfinite(num)):
        return float("inf")
    return float(np.max(num / den))


def elem_rel_err(x, y, floor=1e-3) -> float:
    """max over all elements of |x - y| / max(|y|, floor * max|y| of the
    element's (batch, head) slice)."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    lead = x.shape[:2]
    xs = x.reshape(int(np.prod(lead)), -1)
    ys = y.reshape(int(np.prod(lead)), -1)
    fl = floor * np.max(np.abs(ys), axis=1, keepdims=True)
    den = np.maximum(np.abs(ys), fl)
    den = np.where(den == 0, 1.0, den)
    e = np.abs(xs - ys) / den
    if not np.all(np.isfinite(e)):
        return float("inf")
    return float(np.max(e)) if e.size else 0.0


def errs(x, y) -> tuple:
    """(slice_rel_err, elem_rel_err) of x against y."""
    return slice_rel_err(x, y), elem_rel_err(x, y)


def fmt(name, e) -> str:
    return f"{name}={e[0]:.3e} (elem {e[1]:.3e})"


def oracle_fwd(inp, heads=None):
    """Oracle on the CPU bytes of inp (dict from inputs.make_inputs), optionally
    on a subset of flattened (b, h) head indices.  Returns (o, hT) float64 with
    shapes [n_heads_selected, 1, ...] when heads is given, else [B, H, ...]."""
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    h0 = inp.get("h0")
    if heads is not None:
        B, H = q.shape[:2]
        sel = lambda t: t.reshape(B * H, *t.shape[2:])[heads].unsqueeze(1).contiguous()
        q, k, v, a, b = (sel(t) for t in (q, k, v, a, b))
        h0 = None if h0 is None else sel(h0)
    return oracle.fwd(raw(q), raw(k), raw(v), raw(a), raw(b),
                      h0=None if h0 is None else raw(h0))


def select_heads(t: torch.Tensor, heads):
    B, H = t.shape[:2]
    return t.reshape(B * H, *t.shape[2:])[heads].unsqueeze(1)


def to_dev(inp, device="cuda"):
    return {k: (None if v is None else v.to(device)) for k, v in inp.items()}
