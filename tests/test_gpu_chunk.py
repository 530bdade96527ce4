"""GPU parity of ckda_chunk_fwd against the fp64 oracle (through the C ABI).

Small shapes are compared element by element over every head; the full-size
workloads are compared on sampled heads, which the oracle computes exactly
because every (batch, head) recurrence is independent."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from parity import TOL, errs, fmt, log, oracle_fwd, select_heads, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu


def gpu_fwd(inp, chunk, h0=True):
    d = to_dev(inp)
    o, hT = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"] if h0 else None, chunk=chunk)
    torch.cuda.synchronize()
    return o, hT


def check(w: gen.Workload, heads=None, tol=None, repeated_keys=False, h0=True, keys="normal", values="normal",
          inp=None, out=None):
    log(f"chunk_fwd {w} keys={keys} values={values}" + (f" heads={list(heads)}" if heads is not None else ""))
    if inp is None:
        inp = gen.make_inputs(w, repeated_keys=repeated_keys, keys=keys, values=values)
    if not h0:
        inp["h0"] = None
    o, hT = gpu_fwd(inp, w.chunk) if out is None else out
    o_ref, h_ref = oracle_fwd(inp, heads)
    if heads is not None:
        o, hT = select_heads(o, heads), select_heads(hT, heads)
    eo = errs(o.float().cpu().numpy(), o_ref)
    eh = errs(hT.cpu().numpy(), h_ref)
    log(f"  err {fmt('o', eo)} {fmt('hT', eh)}")
    tol = TOL[w.dtype] if tol is None else tol
    assert eo[0] <= tol and eh[0] <= tol, (eo, eh)
    return eo[0], eh[0]


def test_tiny_fp32_workload():
    w = gen.WORKLOADS["tiny_fp32"]
    check(w)
    check(w, h0=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [16, 32, 64])
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
def test_shapes_all_dk_chunk(dtype, chunk, dk):
    w = gen.Workload("shape", 1, 2, 3 * chunk + 5, dk, 32, chunk, dtype, "ckda_uniform", "normal", 2000 + dk + chunk)
    check(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dv", [16, 64, 128])
def test_shapes_dv(dtype, dv):
    w = gen.Workload("shape", 2, 2, 150, 64, dv, 64, dtype, "ckda_tanh", "normal", 3000 + dv)
    check(w)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200])
def test_ragged_lengths(T):
    w = gen.Workload("ragged", 1, 3, T, 64, 64, 64, "f32", "ckda_uniform", "normal", 4000 + T)
    check(w)


@pytest.mark.parametrize("law", ["zero_and_unit", "orthogonal", "small_gates", "kda"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stress_gates(law, dtype):
    w = gen.Workload("stress", 1, 4, 512, 64, 64, 64, dtype, law, "normal", 5000 + len(law))
    check(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_repeated_keys(dtype):
    w = gen.Workload("repkeys", 1, 2, 256, 64, 64, 64, dtype, "ckda_uniform", "normal", 6000)
    check(w, repeated_keys=True)


@pytest.mark.parametrize("name", ["kda_bf16", "ckda_bf16"])
def test_workload_shortened_all_heads(name):
    """The full-size workloads' value laws and head layout at T=512, every head."""
    w = gen.variant(gen.WORKLOADS[name], T=512)
    check(w)


@pytest.mark.parametrize("name", ["kda_bf16", "ckda_bf16", "ckda_long_dk64"])
def test_workload_full_size_sampled_heads(name):
    w = gen.WORKLOADS[name]
    rng = np.random.default_rng(11)
    heads = np.sort(rng.choice(w.B * w.H, 3, replace=False))
    check(w, heads=heads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_isometric_full_shape(dtype):
    """beta = 2, alpha in {-1, +1}, v = 0 at the bench shape (B4 H16 T4096
    d128, chunk 64, h0 ~ N(0, 0.1)): every transition is orthogonal ("Complex
    KDA" paper, Thm. 1), so ||H_T||_F = ||h0||_F exactly for every head.  The
    drift of the Frobenius norm over the 4096 steps is logged for all 64 heads
    and bounded by the tolerance; o and hT are compared with the oracle on
    sampled heads (App. B "Precision and finite reachability": a small
    rotation error can pile up over many updates)."""
    w = gen.Workload("isometric", 4, 16, 4096, 128, 128, 64, dtype, "orthogonal", "normal", 8100)
    inp = gen.make_inputs(w, values="zero")
    o, hT = gpu_fwd(inp, w.chunk)
    n0 = torch.linalg.norm(inp["h0"].double().reshape(64, -1), dim=1)
    nT = torch.linalg.norm(hT.double().cpu().reshape(64, -1), dim=1)
    drift = (nT / n0 - 1.0).abs()
    log(f"isometric {dtype}: Frobenius norm drift over T=4096: max {drift.max().item():.3e} "
        f"mean {drift.mean().item():.3e} (64 heads)")
    assert drift.max().item() <= TOL[dtype]
    heads = np.array([0, 27, 63])
    check(w, heads=heads, inp=inp, out=(o, hT))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_near_parallel_keys(dtype):
    """Distinct but nearly parallel unit keys (normalise(k_0 + 1e-3 k_t)) with
    beta = 2 and |alpha| = 1: the intra-chunk triangular system is then far
    from the identity, the hardest case of the solve short of equal keys."""
    w = gen.Workload("nearpar", 1, 4, 512, 128, 64, 64, dtype, "orthogonal", "normal", 8200)
    check(w, keys="near_parallel")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_mild_range_violation(dtype):
    """Gates of modulus up to 1.25, outside the CKDA range, are computed as
    given (the chunk kernels' factor ranges hold while products of a chunk's
    gates stay far from the fp32 limits)."""
    w = gen.Workload("overrange", 1, 4, 256, 64, 64, 64, dtype, "mild_overrange", "normal", 8300)
    check(w)


def test_resume_in_place_matches_single_pass():
    """fwd(T1) -> hT, then fwd(T2) continuing in place (hT == h0) equals the
    oracle over T1 + T2."""
    w = gen.Workload("resume", 2, 2, 300, 64, 64, 64, "bf16", "ckda_tanh", "normal", 7000)
    inp = gen.make_inputs(w)
    d = to_dev(inp)
    T1 = 137
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    state = d["h0"].clone()
    o1, _ = ck.chunk_fwd(*(sl(d[n], 0, T1) for n in ("q", "k", "v", "alpha")), sl(d["beta"], 0, T1), state,
                         chunk=64, hT=state)
    o2, _ = ck.chunk_fwd(*(sl(d[n], T1, w.T) for n in ("q", "k", "v", "alpha")), sl(d["beta"], T1, w.T), state,
                         chunk=64, hT=state)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_fwd(inp)
    eo = slice_rel_err(torch.cat([o1, o2], dim=2).float().cpu().numpy(), o_ref)
    eh = slice_rel_err(state.cpu().numpy(), h_ref)
    log(f"resume err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL["bf16"] and eh <= TOL["bf16"]


def test_prefill_then_decode():
    """A chunked prefill's final state continued by decode steps equals the
    oracle over the whole sequence."""
    w = gen.Workload("pd", 2, 3, 200, 64, 64, 64, "f32", "ckda_uniform", "normal", 7100)
    inp = gen.make_inputs(w)
    d = to_dev(inp)
    Tp = 190
    sl = lambda t, a, b: t[:, :, a:b].contiguous()
    _, state = ck.chunk_fwd(*(sl(d[n], 0, Tp) for n in ("q", "k", "v", "alpha")), sl(d["beta"], 0, Tp), d["h0"],
                            chunk=64)
    outs = []
    for t in range(Tp, w.T):
        outs.append(ck.decode_step(*(d[n][:, :, t].contiguous() for n in ("q", "k", "v", "alpha")),
                                   d["beta"][:, :, t].contiguous(), state))
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_fwd(inp)
    eo = slice_rel_err(torch.stack(outs, dim=2).cpu().numpy(), o_ref[:, :, Tp:])
    eh = slice_rel_err(state.cpu().numpy(), h_ref)
    log(f"prefill+decode err o={eo:.3e} hT={eh:.3e}")
    assert eo <= TOL["f32"] and eh <= TOL["f32"]


def test_deterministic():
    w = gen.Workload("det", 2, 4, 700, 128, 128, 64, "bf16", "ckda_tanh", "normal", 7200)
    inp = gen.make_inputs(w)
    o1, h1 = gpu_fwd(inp, 64)
    o2, h2 = gpu_fwd(inp, 64)
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def test_zero_length_copies_state():
    h0 = torch.randn(2, 3, 32, 32, device="cuda")
    e = torch.empty(2, 3, 0, 32, device="cuda")
    o, hT = ck.chunk_fwd(e, e, e, e, torch.empty(2, 3, 0, device="cuda"), h0, chunk=32)
    torch.cuda.synchronize()
    assert torch.equal(hT, h0) and o.numel() == 0
    _, hz = ck.chunk_fwd(e, e, e, e, torch.empty(2, 3, 0, device="cuda"), None, chunk=32)
    torch.cuda.synchronize()
    assert torch.count_nonzero(hz) == 0


def test_nan_gate_propagates_to_its_head_only():
    w = gen.Workload("nan", 1, 3, 100, 32, 32, 32, "f32", "ckda_uniform", "normal", 7300)
    inp = gen.make_inputs(w)
    inp["alpha"][0, 1, 40, 5] = float("nan")
    o, hT = gpu_fwd(inp, 32)
    assert torch.isnan(o[0, 1, 40:]).any() and torch.isnan(hT[0, 1]).any()
    assert torch.isfinite(o[0, 0]).all() and torch.isfinite(o[0, 2]).all()
    assert torch.isfinite(o[0, 1, :32]).all()


def test_timed_entry_point_matches_and_times():
    """ckda_chunk_fwd_timed gives the same bits as ckda_chunk_fwd and its
    events bracket the two kernels in order."""
    w = gen.Workload("timed_small", 2, 3, 300, 64, 32, 64, "bf16", "ckda_tanh", "normal", 77)
    log(f"chunk_fwd_timed {w}")
    d = to_dev(gen.make_inputs(w))
    o1, h1 = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in ev:
        e.record()   # creates the events
    o2, h2 = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk, events=ev)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)
    t_gram, t_state = ev[0].elapsed_time(ev[1]), ev[1].elapsed_time(ev[2])
    log(f"  gram {t_gram * 1e3:.1f} us, state {t_state * 1e3:.1f} us")
    assert t_gram > 0 and t_state > 0
