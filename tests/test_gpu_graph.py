"""The forward and the decode step captured in a HIP graph (torch.cuda.CUDAGraph
on the library's stream argument): every replay, with eager work and
synchronisations between replays, gives the eager call's bytes.  The
library's launches hold no memset and allocate nothing, so they capture as
plain kernel nodes."""
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from parity import log, to_dev

pytestmark = pytest.mark.gpu


def test_forward_graph_replays_match_eager():
    w = gen.Workload("graph", 2, 4, 300, 128, 64, 64, "bf16", "ckda_tanh", "normal", 9100)
    log(f"graph capture of chunk_fwd {w}")
    d = to_dev(gen.make_inputs(w))
    ws = torch.empty(ck.workspace_size(w.B, w.H, w.T, w.dk, w.dv, w.chunk, ck.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=torch.bfloat16, device="cuda")
    hT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device="cuda")
    want_o, want_h = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk, workspace=ws, o=o,
                         hT=hT)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        o.zero_()
        hT.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, want_o), rep
        assert torch.equal(hT, want_h), rep
        # eager work between replays
        ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], None, chunk=w.chunk)
        torch.cuda.synchronize()


def test_decode_graph_replays_match_eager():
    N, H, dk, dv = 16, 4, 128, 128
    S0 = gen.decode_state(N=N, H=H).cuda()
    steps = [to_dev(gen.decode_step_inputs(i, N=N, H=H)) for i in range(3)]
    # eager reference: three steps from S0
    S = S0.clone()
    want = []
    for x in steps:
        want.append(ck.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S).clone())
    want_S = S.clone()
    # one graph of the three steps on a state buffer
    Sg = S0.clone()
    outs = [torch.empty((N, H, dv), dtype=torch.bfloat16, device="cuda") for _ in steps]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for x, oo in zip(steps, outs):
                ck.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], Sg, o=oo)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        Sg.copy_(S0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs, want):
            assert torch.equal(a, b), rep
        assert torch.equal(Sg, want_S), rep
        S.copy_(S0)   # eager work between replays
        ck.decode_step(steps[0]["q"], steps[0]["k"], steps[0]["v"], steps[0]["alpha"], steps[0]["beta"], S)
        torch.cuda.synchronize()
