"""GPU parity of ckda_decode_step against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from gated_delta_rule_ckda_amd.inputs import raw
from parity import TOL, log, slice_rel_err

pytestmark = pytest.mark.gpu


def run_steps(dec, N, H, steps, gates="ckda_uniform", sample=None):
    """Run `steps` decode steps on GPU and oracle; compare o each step and the
    final state.  sample: flattened state indices the oracle follows (None = all)."""
    S0 = gen.decode_state(dec, N, H)
    S_gpu = S0.cuda()
    idx = np.arange(N * H) if sample is None else np.asarray(sample)
    S_ref = S0.reshape(N * H, dec.dk, dec.dv)[idx].to(torch.float64).numpy()[:, None].copy()
    worst_o = 0.0
    for s in range(steps):
        inp = gen.decode_step_inputs(s, dec, N, H, gates=gates)
        d = {k: v.cuda() for k, v in inp.items()}
        o = ck.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_gpu)
        sel = lambda t: raw(t.reshape(N * H, *t.shape[2:])[idx].unsqueeze(1).contiguous())
        o_ref = oracle.decode(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["alpha"]), sel(inp["beta"]),
                              S_ref)
        o_gpu = o.reshape(N * H, -1)[idx].float().cpu().numpy()[:, None]
        worst_o = max(worst_o, slice_rel_err(o_gpu, o_ref))
    torch.cuda.synchronize()
    S_fin = S_gpu.reshape(N * H, dec.dk, dec.dv)[idx].cpu().numpy()[:, None]
    return worst_o, slice_rel_err(S_fin, S_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 128), (128, 32), (128, 128)])
def test_decode_shapes(dtype, dk, dv):
    dec = gen.DecodeWorkload("t", 3, 5, dk, dv, 6, dtype, 77, 900)
    log(f"decode dtype={dtype} dk={dk} dv={dv} N=3 H=5 steps=6")
    eo, es = run_steps(dec, 3, 5, 6)
    log(f"  err o={eo:.2e} state={es:.2e}")
    assert es <= 1e-5
    assert eo <= (1e-5 if dtype == "f32" else TOL["bf16"])


@pytest.mark.parametrize("gates", ["zero_and_unit", "orthogonal", "small_gates"])
def test_decode_stress_gates(gates):
    dec = gen.DecodeWorkload("t", 4, 4, 64, 64, 20, "f32", 78, 950)
    log(f"decode stress gates={gates}")
    eo, es = run_steps(dec, 4, 4, 20, gates=gates)
    log(f"  err o={eo:.2e} state={es:.2e}")
    assert es <= 1e-5 and eo <= 1e-4


def test_decode_full_config_sampled():
    """256 sequences x 32 heads, 128 in-place steps; the oracle follows 48
    sampled states (every state is independent, so this is exact for them)."""
    dec = gen.DECODE
    rng = np.random.default_rng(5)
    sample = np.sort(rng.choice(dec.N * dec.H, 48, replace=False))
    log(f"decode full N={dec.N} H={dec.H} d={dec.dk} steps={dec.steps} (48 sampled states)")
    eo, es = run_steps(dec, dec.N, dec.H, dec.steps, sample=sample)
    log(f"  err o={eo:.2e} state={es:.2e}")
    assert es <= 1e-4            # fp32 state after 128 steps
    assert eo <= TOL["bf16"]     # bf16 outputs


def test_decode_zero_problem_and_nan_propagation():
    N, H, d = 2, 2, 32
    q = torch.randn(N, H, d, device="cuda")
    k = torch.nn.functional.normalize(torch.randn(N, H, d, device="cuda"), dim=-1)
    v = torch.randn(N, H, d, device="cuda")
    a = torch.rand(N, H, d, device="cuda")
    b = torch.rand(N, H, device="cuda")
    S = torch.randn(N, H, d, d, device="cuda")
    a[0, 1, 3] = float("nan")
    o = ck.decode_step(q, k, v, a, b, S)
    torch.cuda.synchronize()
    assert torch.isnan(S[0, 1]).any() and torch.isnan(o[0, 1]).any()
    assert torch.isfinite(S[1]).all() and torch.isfinite(o[1]).all() and torch.isfinite(S[0, 0]).all()
