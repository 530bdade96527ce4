"""GPU parity of ckda_deltaproduct2_bwd (through the C ABI) against the
oracle's DeltaProduct_2 backward (pinned by finite differences of the
separately written DeltaProduct_2 forward), gradient by gradient; fp32-level
tolerances for both dtypes, as for the plain backward."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from gated_delta_rule_ckda_amd.inputs import raw
from parity import log, select_heads, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dalpha", "dbeta", "dh0")
TOL = 1e-4


def run(w, gated, heads=None, h0=True, dhT=True):
    log(f"deltaproduct2_bwd {w} gated={gated}" + (f" heads={list(heads)}" if heads is not None else ""))
    inp = gen.make_dp2_inputs(w, gated=gated)
    do, gT = gen.make_output_grads(w, w.seed + 23)
    if not h0:
        inp["h0"] = None
    if not dhT:
        gT = None
    d = to_dev(inp)
    got = ck.deltaproduct2_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do.cuda(), h0=d["h0"],
                               dhT=None if gT is None else gT.cuda())
    torch.cuda.synchronize()
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    h0t, dot = inp["h0"], do
    if heads is not None:
        pick = lambda t: None if t is None else select_heads(t, heads).contiguous()
        q, k, v, a, b, dot, h0t, gT = (pick(t) for t in (q, k, v, a, b, dot, h0t, gT))
        got = [pick(g) for g in got]
    want = oracle.deltaproduct2_bwd(raw(q), raw(k), raw(v), None if a is None else raw(a), raw(b),
                                    oracle._widen(raw(dot)), dhT=None if gT is None else gT.double().numpy(),
                                    h0=None if h0t is None else raw(h0t))
    errs = {}
    for n, g, wv in zip(NAMES, got, want):
        if wv is None:
            assert g is None
            continue
        errs[n] = slice_rel_err(g.cpu().numpy(), wv)
    log("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gated", [True, False])
def test_small(dtype, gated):
    w = gen.Workload("dp2b", 1, 2, 45, 32, 64, 64, dtype, "ckda_uniform", "normal", 8100 + gated)
    run(w, gated)


@pytest.mark.parametrize("dk,dv", [(16, 16), (128, 128), (64, 16)])
def test_shapes(dk, dv):
    w = gen.Workload("dp2b", 2, 1, 37, dk, dv, 64, "bf16", "ckda_tanh", "normal", 8200 + dk + dv)
    run(w, True)


@pytest.mark.parametrize("T", [1, 16, 17, 100])
def test_ragged_lengths(T):
    w = gen.Workload("dp2b", 1, 1, T, 64, 32, 64, "f32", "ckda_tanh", "normal", 8300 + T)
    run(w, True)


def test_optional_terms_absent():
    w = gen.Workload("dp2b", 1, 2, 30, 32, 32, 64, "bf16", "ckda_tanh", "zero", 8400)
    run(w, False, h0=False, dhT=False)


def test_full_size_sampled_heads():
    """The bench shape (B4 H16 T4096 d128 bf16, 8192 sub-steps per head),
    ungated as the pages' comparator; the oracle follows one head."""
    run(gen.variant(gen.WORKLOADS["ckda_bf16"], name="dp2b_full"), False, heads=[22])


def test_deterministic():
    w = gen.Workload("dp2b", 1, 2, 60, 64, 64, 64, "bf16", "ckda_tanh", "normal", 8500)
    d = to_dev(gen.make_dp2_inputs(w, gated=True))
    do, gT = (x.cuda() for x in gen.make_output_grads(w, 5))
    a = ck.deltaproduct2_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do, h0=d["h0"], dhT=gT)
    b = ck.deltaproduct2_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do, h0=d["h0"], dhT=gT)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
