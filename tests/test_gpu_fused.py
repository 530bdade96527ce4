"""GPU parity of the fused per-token prologue (ckda_chunk_fwd_ex,
ckda_decode_step_ex) against the fp64 oracle run on the prologue's own
definition (oracle.prologue, then the recurrence), through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from gated_delta_rule_ckda_amd.inputs import raw
from parity import TOL, log, select_heads, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

ALL = ck.FUSE_GATES | ck.FUSE_NORM_K | ck.FUSE_NORM_Q
GK = ck.FUSE_GATES | ck.FUSE_NORM_K


def oracle_fused(inp, flags, heads=None):
    q, k, v, a, b = (inp[n] for n in ("q", "k", "v", "alpha", "beta"))
    h0 = inp.get("h0")
    if heads is not None:
        q, k, v, a, b = (select_heads(t, heads).contiguous() for t in (q, k, v, a, b))
        h0 = None if h0 is None else select_heads(h0, heads).contiguous()
    return oracle.fwd_fused(raw(q), raw(k), raw(v), raw(a), raw(b), h0=None if h0 is None else raw(h0),
                            flags=flags)


def check_fwd(w, flags, heads=None, zero_rows=0.0, tol=None):
    log(f"chunk_fwd_ex flags={flags} {w} zero_rows={zero_rows}" + (f" heads={list(heads)}" if heads is not None else ""))
    inp = gen.make_logit_inputs(w, zero_rows=zero_rows)
    if flags & ck.FUSE_GATES == 0:
        # gates used as given: keep them in the CKDA ranges
        inp["alpha"] = torch.tanh(inp["alpha"].float()).to(inp["alpha"].dtype)
        inp["beta"] = (2 * torch.sigmoid(inp["beta"].float())).to(inp["beta"].dtype)
    if flags & ck.FUSE_NORM_K == 0:
        kf = inp["k"].float()
        inp["k"] = (kf / kf.norm(dim=-1, keepdim=True).clamp_min(1e-30)).to(inp["k"].dtype)
    d = to_dev(inp)
    o, hT = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk, fuse=flags)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle_fused(inp, flags, heads)
    if heads is not None:
        o, hT = select_heads(o, heads), select_heads(hT, heads)
    eo = slice_rel_err(o.float().cpu().numpy(), o_ref)
    eh = slice_rel_err(hT.cpu().numpy(), h_ref)
    log(f"  err o={eo:.3e} hT={eh:.3e}")
    tol = TOL[w.dtype] if tol is None else tol
    assert eo <= tol and eh <= tol, (eo, eh)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,chunk", [(16, 16), (32, 32), (64, 64), (128, 64), (128, 32)])
def test_fused_forward_shapes(dtype, dk, chunk):
    w = gen.Workload("fused", 1, 2, 3 * chunk + 7, dk, 32, chunk, dtype, "ckda_uniform", "normal", 4100 + dk + chunk)
    check_fwd(w, GK)


@pytest.mark.parametrize("flags", [1, 2, 3, 4, 5, 6, 7])
def test_fused_forward_each_flag_combination(flags):
    w = gen.Workload("fused", 2, 2, 150, 64, 64, 64, "f32", "ckda_uniform", "normal", 4200 + flags)
    check_fwd(w, flags)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_forward_zero_key_rows(dtype):
    w = gen.Workload("fused", 1, 3, 200, 128, 128, 64, dtype, "ckda_uniform", "zero", 4300)
    check_fwd(w, ALL, zero_rows=0.1)


def test_fused_forward_full_size_sampled_heads():
    """B4 H16 T4096 d128 chunk 64 bf16, h0 ~ N(0, 0.1), logits as inputs; the
    oracle follows 3 of the 64 heads (each head's recurrence is independent)."""
    w = gen.variant(gen.WORKLOADS["ckda_bf16"], seed=4400)
    check_fwd(w, GK, heads=[0, 29, 63])


def test_ex_with_no_flags_is_the_plain_forward_bitwise():
    w = gen.variant(gen.WORKLOADS["ckda_bf16"], B=1, H=4, T=300)
    d = to_dev(gen.make_inputs(w))
    args = (d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"])
    o1, h1 = ck.chunk_fwd(*args, chunk=64)
    L = ck.lib()
    o2, h2 = torch.empty_like(o1), torch.empty_like(h1)
    ws = torch.empty(ck.workspace_size(1, 4, 300, 128, 128, 64, 1), dtype=torch.uint8, device="cuda")
    rc = L.ckda_chunk_fwd_ex(*(t.data_ptr() for t in args), o2.data_ptr(), h2.data_ptr(), 1, 4, 300, 128, 128, 64,
                             1, 0, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(h1, h2)


def run_decode(dec, N, H, steps, flags, sample=None):
    S0 = gen.decode_state(dec, N, H)
    S_gpu = S0.cuda()
    idx = np.arange(N * H) if sample is None else np.asarray(sample)
    S_ref = S0.reshape(N * H, dec.dk, dec.dv)[idx].to(torch.float64).numpy()[:, None].copy()
    worst = 0.0
    for s in range(steps):
        inp = gen.decode_logit_inputs(s, dec, N, H)
        d = {k: v.cuda() for k, v in inp.items()}
        o = ck.decode_step(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_gpu, fuse=flags)
        sel = lambda t: raw(t.reshape(N * H, *t.shape[2:])[idx].unsqueeze(1).contiguous())
        o_ref = oracle.decode_fused(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["alpha"]),
                                    sel(inp["beta"]), S_ref, flags=flags)
        worst = max(worst, slice_rel_err(o.reshape(N * H, -1)[idx].float().cpu().numpy()[:, None], o_ref))
    torch.cuda.synchronize()
    S_fin = S_gpu.reshape(N * H, dec.dk, dec.dv)[idx].cpu().numpy()[:, None]
    return worst, slice_rel_err(S_fin, S_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 128), (128, 128)])
@pytest.mark.parametrize("flags", [GK, ALL])
def test_fused_decode(dtype, dk, dv, flags):
    dec = gen.DecodeWorkload("t", 3, 5, dk, dv, 6, dtype, 79, 960)
    log(f"decode_step_ex flags={flags} dtype={dtype} dk={dk} dv={dv}")
    eo, es = run_decode(dec, 3, 5, 6, flags)
    log(f"  err o={eo:.2e} state={es:.2e}")
    assert es <= 1e-5
    assert eo <= (1e-5 if dtype == "f32" else TOL["bf16"])


def test_fused_decode_full_config_sampled():
    dec = gen.DECODE
    rng = np.random.default_rng(6)
    sample = np.sort(rng.choice(dec.N * dec.H, 32, replace=False))
    log(f"decode_step_ex full N={dec.N} H={dec.H} steps=16 (32 sampled states)")
    eo, es = run_decode(dec, dec.N, dec.H, 16, GK, sample=sample)
    log(f"  err o={eo:.2e} state={es:.2e}")
    assert es <= 1e-4 and eo <= TOL["bf16"]
