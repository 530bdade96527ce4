"""GPU parity of ckda_chunk_bwd_ex (the backward through the per-token
prologue, through the C ABI) against the oracle's fp64 bwd_fused: gradients
with respect to the gate and beta logits, the raw keys and queries, v and h0.
The gate's backward holds the sign constant and gives a zero gradient at a
zero logit (the convention of the discussion slides); both sides compute from
the exact input bytes, so both dtypes are held to fp32-level tolerances."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from gated_delta_rule_ckda_amd.inputs import raw
from parity import log, select_heads, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "da", "db", "dh0")
TOL = 1e-4


def _inputs(w, flags, zero_logits=0.0):
    """Logit inputs; the first channel's logit becomes the token's scalar gate
    with CKDA_GATE_SCALAR; without CKDA_FUSE_GATES the gates are linear
    (tanh of the logits, beta 2 sigma(b)), and without CKDA_FUSE_NORM_K the
    keys are given unit rows (the recurrence's contract), in the input dtype."""
    inp = gen.make_logit_inputs(w)
    if not flags & ck.FUSE_NORM_K:
        k = inp["k"].float()
        inp["k"] = (k / k.norm(dim=-1, keepdim=True)).to(inp["k"].dtype)
    a = inp["alpha"].float()
    b = inp["beta"].float()
    if zero_logits:
        r = np.random.default_rng(w.seed + 5)
        a = torch.where(torch.from_numpy(r.uniform(size=tuple(a.shape)) < zero_logits), torch.zeros(()), a)
    if flags & ck.GATE_SCALAR:
        a = a[..., 0].contiguous()
    if not flags & ck.FUSE_GATES:
        a = torch.tanh(a / 2)
        b = 2 * torch.sigmoid(b)
    dt = inp["q"].dtype
    inp["alpha"], inp["beta"] = a.to(dt), b.to(dt)
    return inp


def run(w, flags, heads=None, zero_logits=0.0, tol=TOL):
    log(f"chunk_bwd_ex {w} flags={flags}" + (f" heads={list(heads)}" if heads is not None else "")
        + (f" zero_logits={zero_logits}" if zero_logits else ""))
    inp = _inputs(w, flags, zero_logits)
    do, gT = gen.make_output_grads(w, w.seed + 19)
    d = to_dev(inp)
    got = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do.cuda(), h0=d["h0"], dhT=gT.cuda(),
                       fuse=flags)
    torch.cuda.synchronize()
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    dot, h0t, gTt = do, inp["h0"], gT
    if heads is not None:
        q, k, v, a, b, dot = (select_heads(t, heads).contiguous() for t in (q, k, v, a, b, dot))
        h0t = None if h0t is None else select_heads(h0t, heads).contiguous()
        gTt = select_heads(gTt, heads).contiguous()
        got = [None if g is None else select_heads(g, heads) for g in got]
    want = oracle.bwd_fused(raw(q), raw(k), raw(v), raw(a), raw(b), oracle._widen(raw(dot)),
                            dhT=gTt.numpy().astype(np.float64), h0=None if h0t is None else raw(h0t),
                            flags=flags & 7, scalar=bool(flags & ck.GATE_SCALAR))
    errs = {n: slice_rel_err(g.cpu().numpy(), wv) for n, g, wv in zip(NAMES, got, want)}
    log("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return got, want


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("flags", [1, 2, 3, 6, 7])
def test_flags(dtype, flags):
    w = gen.Workload("bwdx", 1, 2, 3 * 32 + 5, 64, 32, 64, dtype, "ckda_tanh", "normal", 7600 + flags)
    run(w, flags)


@pytest.mark.parametrize("flags", [8, 9, 11, 15])
def test_scalar_gate(flags):
    """One gate per token and head: its gradient sums the channels' gradients."""
    w = gen.Workload("bwdx", 2, 1, 70, 32, 64, 64, "bf16", "ckda_tanh", "normal", 7700 + flags)
    run(w, flags)


@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (128, 16)])
def test_shapes(dk, dv):
    w = gen.Workload("bwdx", 1, 2, 41, dk, dv, 64, "f32", "ckda_tanh", "normal", 7800 + dk + dv)
    run(w, 7)


def test_zero_logits_pass_no_gate_gradient():
    """Exact zero logits: d alpha / d a = 0 there (zero subgradient of |r| at
    0, the sign held constant), on the GPU bit for bit."""
    w = gen.Workload("bwdx", 1, 2, 66, 32, 32, 64, "f32", "ckda_tanh", "normal", 7900)
    got, want = run(w, 3, zero_logits=0.3)
    a = _inputs(w, 3, 0.3)["alpha"]
    zero = (a == 0).numpy()
    assert zero.sum() > 100
    assert np.all(got[3].cpu().numpy()[zero] == 0.0)
    assert np.all(want[3][zero] == 0.0)


def test_flags_zero_is_the_plain_backward():
    """ckda_chunk_bwd_ex with flags 0 gives the plain backward's bytes."""
    w = gen.Workload("bwdx", 1, 2, 50, 32, 32, 64, "bf16", "ckda_tanh", "normal", 7950)
    d = to_dev(gen.make_inputs(w))
    do, gT = (x.cuda() for x in gen.make_output_grads(w, 3))
    plain = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do, h0=d["h0"], dhT=gT)
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    f32 = dict(dtype=torch.float32, device="cuda")
    outs = [torch.empty((B, H, T, dk), **f32), torch.empty((B, H, T, dk), **f32), torch.empty((B, H, T, dv), **f32),
            torch.empty((B, H, T, dk), **f32), torch.empty((B, H, T), **f32), torch.empty((B, H, dk, dv), **f32)]
    need = ck.bwd_ex_workspace_size(B, H, T, dk, dv, ck.DTYPE_BF16, 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = ck.lib().ckda_chunk_bwd_ex(*(p(d[n]) for n in ("q", "k", "v", "alpha", "beta", "h0")), p(do), p(gT),
                                    *(p(t) for t in outs), B, H, T, dk, dv, ck.DTYPE_BF16, 0, p(ws), need,
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 0, ck.lib().ckda_last_error()
    for x, y in zip(plain, outs):
        assert torch.equal(x, y)


def test_zero_length_passes_dhT_through():
    e = torch.empty(1, 2, 0, 16, device="cuda")
    dhT = torch.randn(1, 2, 16, 16, device="cuda")
    got = ck.chunk_bwd(e, e, e, e, torch.empty(1, 2, 0, device="cuda"), e, dhT=dhT, fuse=7)
    torch.cuda.synchronize()
    assert torch.equal(got[5], dhT)


def test_full_size_sampled_heads():
    """B4 H16 T4096 d128 bf16 (the bench shape) with gates from logits and
    unit-norm keys; the oracle follows one of the 64 heads."""
    w = gen.variant(gen.WORKLOADS["ckda_bf16"], name="bwdx_full")
    run(w, 3, heads=[37])


def test_deterministic():
    """Two calls give the same bytes (no atomics, fixed reduction orders)."""
    w = gen.Workload("bwdx", 1, 2, 77, 64, 64, 64, "bf16", "ckda_tanh", "normal", 7990)
    d = to_dev(_inputs(w, 7))
    do, gT = (x.cuda() for x in gen.make_output_grads(w, 5))
    a = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do, h0=d["h0"], dhT=gT, fuse=7)
    b = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do, h0=d["h0"], dhT=gT, fuse=7)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
