"""GPU parity of the comparator variants through the C ABI: the scalar
(Gated DeltaNet) gate (CKDA_GATE_SCALAR) and DeltaProduct_2
(ckda_deltaproduct2_fwd / _decode_step), against the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from gated_delta_rule_ckda_amd.inputs import raw
from parity import TOL, log, select_heads, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

GK = ck.FUSE_GATES | ck.FUSE_NORM_K


def bcast(alpha, dk):
    return alpha.unsqueeze(-1).expand(*alpha.shape, dk).contiguous()


def errs(o, hT, o_ref, h_ref):
    return slice_rel_err(o.float().cpu().numpy(), o_ref), slice_rel_err(hT.cpu().numpy(), h_ref)


# ---------------------------------------------------------------- scalar gate

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,chunk,law", [(64, 64, "ckda_tanh"), (128, 64, "kda"), (32, 16, "ckda_uniform"),
                                          (128, 32, "zero_and_unit")])
def test_scalar_gate_forward(dtype, dk, chunk, law):
    w = gen.Workload("gdn", 2, 2, 2 * chunk + 9, dk, 64, chunk, dtype, law, "normal", 6100 + dk + chunk)
    log(f"chunk_fwd_ex GATE_SCALAR {w}")
    inp = gen.make_scalar_gate_inputs(w)
    d = to_dev(inp)
    o, hT = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=chunk, fuse=ck.GATE_SCALAR)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.fwd(raw(inp["q"]), raw(inp["k"]), raw(inp["v"]), raw(bcast(inp["alpha"], dk)),
                              raw(inp["beta"]), h0=raw(inp["h0"]))
    eo, eh = errs(o, hT, o_ref, h_ref)
    log(f"  err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_gate_forward_with_prologue(dtype):
    w = gen.Workload("gdn", 1, 3, 170, 128, 128, 64, dtype, "ckda_uniform", "normal", 6200)
    inp = gen.make_logit_inputs(w)
    inp["alpha"] = inp["alpha"][..., 0].contiguous()          # one logit per token and head
    d = to_dev(inp)
    o, hT = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=64,
                         fuse=ck.GATE_SCALAR | GK)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.fwd_fused(raw(inp["q"]), raw(inp["k"]), raw(inp["v"]), raw(bcast(inp["alpha"], 128)),
                                    raw(inp["beta"]), h0=raw(inp["h0"]), flags=GK)
    eo, eh = errs(o, hT, o_ref, h_ref)
    log(f"scalar gate + prologue {dtype}: err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL[dtype] and eh <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_gate_decode(dtype):
    N, H, dk, dv, steps = 3, 4, 128, 64, 5
    dec = gen.DecodeWorkload("t", N, H, dk, dv, steps, dtype, 83, 980)
    S0 = gen.decode_state(dec)
    S = S0.cuda()
    S_ref = S0.to(torch.float64).numpy().copy()
    worst = 0.0
    for s in range(steps):
        inp = gen.decode_step_inputs(s, dec)
        inp["alpha"] = inp["alpha"][..., 0].contiguous()
        d = {k: v.cuda() for k, v in inp.items()}
        o = ck.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S, fuse=ck.GATE_SCALAR)
        o_ref = oracle.decode(raw(inp["q"]), raw(inp["k"]), raw(inp["v"]), raw(bcast(inp["alpha"], dk)),
                              raw(inp["beta"]), S_ref)
        worst = max(worst, slice_rel_err(o.float().cpu().numpy(), o_ref))
    torch.cuda.synchronize()
    es = slice_rel_err(S.cpu().numpy(), S_ref)
    log(f"decode GATE_SCALAR {dtype}: err o={worst:.2e} state={es:.2e}")
    assert es <= 1e-5 and worst <= (1e-5 if dtype == "f32" else TOL["bf16"])


# ---------------------------------------------------------------- DeltaProduct_2

def dp2_check(w, gated, flags=0, heads=None):
    log(f"deltaproduct2_fwd gated={gated} flags={flags} {w}" + (f" heads={list(heads)}" if heads is not None else ""))
    inp = gen.make_dp2_inputs(w, gated=gated)
    d = to_dev(inp)
    o, hT = ck.deltaproduct2_fwd(d["q"], d["k"], d["v"], d["beta"], alpha=d["alpha"], h0=d["h0"], chunk=w.chunk,
                                 fuse=flags)
    torch.cuda.synchronize()
    q, k, v, a, b, h0 = (inp[n] for n in ("q", "k", "v", "alpha", "beta", "h0"))
    if heads is not None:
        q, k, v, b, h0 = (select_heads(t, heads).contiguous() for t in (q, k, v, b, h0))
        a = None if a is None else select_heads(a, heads).contiguous()
        o, hT = select_heads(o, heads), select_heads(hT, heads)
    q, k, v, b, h0 = raw(q), raw(k), raw(v), raw(b), raw(h0)
    a = None if a is None else raw(a)
    if flags:
        # the prologue by its oracle definition: sub-step keys normalised per row,
        # beta (and the scalar gate) from logits
        Bq, Hq, T, dk = q.shape
        kr = k.reshape(Bq, Hq, 2 * T, dk)
        _, bf, kf, _ = oracle.prologue(np.zeros_like(kr), b.reshape(Bq, Hq, 2 * T), kr, kr, flags)
        k, b = kf.reshape(Bq, Hq, T, 2, dk), bf.reshape(Bq, Hq, T, 2)
        qf = oracle._widen(q)
        if a is not None:
            af, _, _, _ = oracle.prologue(a[..., None], np.zeros(a.shape, a.dtype), np.ones(a.shape + (1,), a.dtype),
                                          np.ones(a.shape + (1,), a.dtype), ck.FUSE_GATES)
            a = af[..., 0]
        v = oracle._widen(v)
        q = qf
    o_ref, h_ref = oracle.deltaproduct2(q, k, v, a, b, h0=h0)
    eo, eh = errs(o, hT, o_ref, h_ref)
    log(f"  err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL[w.dtype] and eh <= TOL[w.dtype], (eo, eh)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dk,chunk", [(128, 64), (64, 32), (16, 16)])
def test_deltaproduct2_forward(dtype, gated, dk, chunk):
    w = gen.Workload("dp2", 2, 2, chunk + 13, dk, 32, chunk, dtype, "ckda_uniform", "normal", 6300 + dk + chunk)
    dp2_check(w, gated)


@pytest.mark.parametrize("gated", [False, True])
def test_deltaproduct2_forward_with_prologue(gated):
    w = gen.Workload("dp2", 1, 3, 150, 128, 64, 64, "bf16", "ckda_tanh", "normal", 6400)
    dp2_check(w, gated, flags=GK)


def test_deltaproduct2_full_size_sampled_heads():
    """B4 H16 T4096 d128 chunk 64 bf16, ungated (the pages' benchmark
    setting), oracle on 2 of the 64 heads."""
    w = gen.Workload("dp2", 4, 16, 4096, 128, 128, 64, "bf16", "ckda_uniform", "normal", 6500)
    dp2_check(w, False, heads=[3, 60])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 32), (16, 16)])
def test_deltaproduct2_decode(dtype, gated, dk, dv):
    N, H, steps = 3, 4, 5
    dec = gen.DecodeWorkload("t", N, H, dk, dv, steps, dtype, 84, 990)
    S0 = gen.decode_state(dec)
    S = S0.cuda()
    S_ref = S0.to(torch.float64).numpy().copy()
    worst = 0.0
    for s in range(steps):
        inp = gen.dp2_decode_inputs(s, dec, gated=gated)
        d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
        o = ck.deltaproduct2_decode_step(d["q"], d["k"], d["v"], d["beta"], S, alpha=d["alpha"])
        o_ref = oracle.deltaproduct2_decode(raw(inp["q"]), raw(inp["k"]), raw(inp["v"]),
                                            None if inp["alpha"] is None else raw(inp["alpha"]), raw(inp["beta"]),
                                            S_ref)
        worst = max(worst, slice_rel_err(o.float().cpu().numpy(), o_ref))
    torch.cuda.synchronize()
    es = slice_rel_err(S.cpu().numpy(), S_ref)
    log(f"deltaproduct2 decode {dtype} gated={gated} dk={dk} dv={dv}: err o={worst:.2e} state={es:.2e}")
    assert es <= 1e-5 and worst <= (1e-5 if dtype == "f32" else TOL["bf16"])


def test_deltaproduct2_prefill_then_decode():
    """The chunked DeltaProduct_2 forward hands its state to the decode step:
    forward over T tokens then one decode step equals the oracle over T + 1."""
    w = gen.Workload("dp2", 1, 2, 100, 64, 64, 64, "f32", "ckda_uniform", "normal", 6600)
    inp = gen.make_dp2_inputs(w, gated=True)
    d = to_dev(inp)
    T = w.T - 1
    sl = lambda x: x[:, :, :T].contiguous()
    o, hT = ck.deltaproduct2_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["beta"]), alpha=sl(d["alpha"]),
                                 h0=d["h0"], chunk=64)
    last = lambda x: x[:, :, T].contiguous()
    o_last = ck.deltaproduct2_decode_step(last(d["q"]), last(d["k"]), last(d["v"]), last(d["beta"]), hT,
                                          alpha=last(d["alpha"]))
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.deltaproduct2(raw(inp["q"]), raw(inp["k"]), raw(inp["v"]), raw(inp["alpha"]),
                                        raw(inp["beta"]), h0=raw(inp["h0"]))
    eo = slice_rel_err(o_last.cpu().numpy()[:, :, None], o_ref[:, :, T:])
    eh = slice_rel_err(hT.cpu().numpy(), h_ref)
    log(f"deltaproduct2 prefill + decode: err o={eo:.2e} hT={eh:.2e}")
    assert eo <= 1e-4 and eh <= 1e-4
