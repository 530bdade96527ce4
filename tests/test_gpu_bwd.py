"""GPU parity of ckda_chunk_bwd (through the C ABI) against the oracle's
sequential fp64 backward, gradient by gradient: dq, dk, dv, dalpha, dbeta,
dh0.  The kernels compute in fp32 from the exact input bytes (bf16 inputs
included; with bf16 inputs at dk >= 64 the sequential passes multiply split
bf16 pairs, about 16 bits), so both dtypes are held to fp32-level tolerances."""
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
BTOL = {"f32": 1e-4, "bf16": 1e-4}


def run(w, heads=None, h0=True, dhT=True, tol=None):
    log(f"chunk_bwd {w}" + (f" heads={list(heads)}" if heads is not None else "") + f" h0={h0} dhT={dhT}")
    inp = gen.make_inputs(w)
    do, gT = gen.make_output_grads(w, w.seed + 17)
    if not h0:
        inp["h0"] = None
    if not dhT:
        gT = None
    d = to_dev(inp)
    got = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do.cuda(), h0=d["h0"],
                       dhT=None if gT is None else gT.cuda())
    torch.cuda.synchronize()
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    h0t = inp["h0"]
    dot = do
    if heads is not None:
        q, k, v, a, b, dot = (select_heads(t, heads).contiguous() for t in (q, k, v, a, b, dot))
        h0t = None if h0t is None else select_heads(h0t, heads).contiguous()
        gT = None if gT is None else select_heads(gT, heads).contiguous()
        got = [None if g is None else select_heads(g, heads) for g in got]
    want = oracle.bwd(raw(q), raw(k), raw(v), raw(a), raw(b), oracle._widen(raw(dot)),
                      dhT=None if gT is None else gT.numpy().astype(np.float64),
                      h0=None if h0t is None else raw(h0t))
    tol = BTOL[w.dtype] if tol is None else tol
    errs = {}
    for name, g, wv in zip(NAMES, got, want):
        e = slice_rel_err(g.cpu().numpy(), wv)
        errs[name] = e
    log("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, bad
    return errs


def test_tiny_fp32_workload():
    run(gen.WORKLOADS["tiny_fp32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16)])
def test_shapes(dtype, dk, dv):
    w = gen.Workload("bwd", 1, 2, 3 * 32 + 5, dk, dv, 64, dtype, "ckda_uniform", "normal", 7000 + dk + dv)
    run(w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,T", [(16, 89), (32, 89), (64, 89), (64, 33), (128, 89), (128, 160), (16, 1)])
def test_odd_chunk_counts(dtype, dk, T):
    """The reverse state pass takes two chunks per loop iteration; an odd
    number of 32-position chunks ends with a step that must change nothing
    (one wave per slice at dk 16; two waves at dk 32, 64 and 128, which sum
    their partial dU through an LDS buffer chosen by the chunk's parity, so
    the dead step must not write the buffer the last live step exchanged
    through)."""
    w = gen.Workload("bwd", 1, 2, T, dk, 32, 64, dtype, "ckda_tanh", "normal", 7250 + dk + T)
    run(w)


@pytest.mark.parametrize("law", ["zero_and_unit", "small_gates", "orthogonal", "kda"])
def test_stress_gates(law):
    """Exact zero and +-1 gates, gates down to 1e-12, orthogonal steps: the
    gate derivatives divide by no gate, so none of these is a special case."""
    w = gen.Workload("bwd", 1, 2, 77, 32, 32, 64, "f32", law, "normal", 7100)
    run(w)


@pytest.mark.parametrize("law", ["zero_and_unit", "small_gates", "orthogonal", "kda"])
def test_stress_gates_split_path(law):
    """bf16 inputs at dk >= 64: the sequential passes multiply split bf16
    pairs (hi + lo, about 16 bits) instead of fp32; the same stress laws, an
    odd number of chunks, held to the same bar."""
    w = gen.Workload("bwd", 1, 2, 333, 128, 64, 64, "bf16", law, "normal", 7150)
    run(w)


def test_isometric_full_shape_sampled_heads():
    """The bench shape with orthogonal steps (beta = 2, alpha = +-1): no step
    damps a rounding error, over 128 chunks forward (chunk-start states) and
    128 back (state gradients), so errors of the split products add up here
    if anywhere; the oracle follows 2 of the 64 heads."""
    b = gen.WORKLOADS["ckda_bf16"]
    w = gen.Workload("bwd_isometric", b.B, b.H, b.T, b.dk, b.dv, b.chunk, "bf16", "orthogonal", "normal", 7160)
    run(w, heads=[0, 63])


@pytest.mark.parametrize("dtype,dk,dv,B,H,T", [
    ("bf16", 128, 128, 4, 16, 77), ("bf16", 64, 128, 4, 16, 77), ("bf16", 64, 64, 8, 16, 45),
    ("bf16", 128, 32, 16, 16, 3), ("bf16", 64, 32, 16, 16, 40), ("f32", 128, 128, 4, 16, 77)])
def test_two_slices_per_wave(dtype, dk, dv, B, H, T):
    """With split products (bf16 inputs, dk >= 64, dv a multiple of 32), grids
    with B H dv / 16 of at least twice the compute units (512 on a 256-CU
    part) run the forward state pass of the backward with two 16-column value
    slices per wave, both slices' products sharing each record fragment;
    ragged lengths, dv 32 (one slice pair per head) to 128, and an fp32 grid of
    the same size (one slice per wave); the oracle follows the first, a middle
    and the last head."""
    w = gen.Workload("bwd_two_slices", B, H, T, dk, dv, 64, dtype, "ckda_tanh", "normal", 7600 + dk + dv + T)
    run(w, heads=[0, B * H // 2 + 1, B * H - 1])


def test_two_slices_without_initial_or_final_state():
    """The two-slice forward pass and the four-wave reverse pass (bench-sized
    grid, bf16, dk 128) with neither h0 nor dhT, an odd number of 32-position
    chunks (the reverse pass ends with a step that must change nothing)."""
    w = gen.Workload("bwd_two_slices", 4, 16, 99, 128, 128, 64, "bf16", "ckda_tanh", "normal", 7690)
    run(w, heads=[0, 33, 63], h0=False, dhT=False)


@pytest.mark.parametrize("dtype,dk,dv,B,H,T", [
    ("bf16", 128, 128, 8, 16, 77), ("f32", 128, 64, 8, 16, 77), ("bf16", 64, 64, 16, 16, 77),
    ("f32", 32, 32, 16, 16, 50)])
def test_prep_loops_over_chunks(dtype, dk, dv, B, H, T):
    """The backward's prep kernel runs as many workgroups as fit on the GPU at
    once and loops over the chunks, fetching the next chunk's inputs while it
    computes the current one: with more chunks than resident workgroups (384
    to 768 here, ragged last chunks) some workgroups handle two or three, and
    the sampled heads lie on both sides of the first pass."""
    w = gen.Workload("bwd_prep_loop", B, H, T, dk, dv, 64, dtype, "ckda_tanh", "normal", 7700 + dk + dv + T)
    run(w, heads=[0, B * H * 2 // 3, B * H - 1])


@pytest.mark.parametrize("T", [1, 31, 32, 33, 64, 200])
def test_ragged_lengths(T):
    w = gen.Workload("bwd", 1, 1, T, 64, 64, 64, "f32", "ckda_tanh", "normal", 7200 + T)
    run(w)


def test_optional_terms_absent():
    w = gen.Workload("bwd", 2, 1, 50, 32, 32, 64, "bf16", "ckda_tanh", "normal", 7300)
    run(w, h0=False, dhT=False)


def test_full_size_sampled_heads():
    """B4 H16 T4096 d128 bf16 (the bench shape, CKDA gates, h0 ~ N(0, 0.1));
    the oracle follows 2 of the 64 heads."""
    run(gen.WORKLOADS["ckda_bf16"], heads=[1, 62])


def test_zero_length_passes_dhT_through():
    w = gen.Workload("bwd", 1, 2, 0, 16, 16, 64, "f32", "ckda_uniform", "normal", 7400)
    inp = to_dev(gen.make_inputs(w))
    dhT = torch.randn(1, 2, 16, 16, device="cuda")
    e = torch.empty(1, 2, 0, 16, device="cuda")
    got = ck.chunk_bwd(e, e, e, e, torch.empty(1, 2, 0, device="cuda"), e, h0=inp["h0"], dhT=dhT)
    torch.cuda.synchronize()
    assert torch.equal(got[5], dhT)


def test_deterministic():
    w = gen.Workload("bwd", 1, 2, 100, 64, 64, 64, "bf16", "ckda_tanh", "normal", 7500)
    d = to_dev(gen.make_inputs(w))
    do, gT = gen.make_output_grads(w, 1)
    a = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do.cuda(), h0=d["h0"], dhT=gT.cuda())
    b = ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], do.cuda(), h0=d["h0"], dhT=gT.cuda())
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
