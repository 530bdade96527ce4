"""ckda_chunk_fwd_noalloc (the forward with no workspace, for callers that
cannot allocate) against ckda_chunk_fwd on the same inputs, through the C
ABI: two calls in a row, the first large enough to run its heads in several
batches through the fixed scratch, the second smaller (the scratch keeps the
first call's records; nothing of them may leak into the second).  Both
entry points run the same kernels on the same bytes, so the results must be
identical; the first call is also checked against the oracle on sampled
heads."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs as gen
from parity import TOL, errs, fmt, log, oracle_fwd, select_heads, to_dev

pytestmark = pytest.mark.gpu


def run_both(w):
    inp = gen.make_inputs(w)
    d = to_dev(inp)
    o_ref, h_ref = ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk)
    o = torch.full_like(o_ref, float("nan"))
    hT = torch.full_like(h_ref, float("nan"))
    ck.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], o, hT, chunk=w.chunk)
    torch.cuda.synchronize()
    return inp, o, hT, o_ref, h_ref


def test_noalloc_matches_chunk_fwd_twice():
    # 32 heads x 4096 positions at d128 bf16: 4.4 MB of records per head, so
    # the 64 MiB scratch takes 15 heads per batch (three batches)
    w1 = gen.Workload("noalloc1", 2, 16, 4096, 128, 128, 64, "bf16", "ckda_tanh", "normal", 9100)
    log(f"noalloc {w1}")
    inp, o, hT, o_ref, h_ref = run_both(w1)
    assert torch.equal(o, o_ref) and torch.equal(hT, h_ref)
    heads = np.array([0, 15, 16, 31])
    ro, rh = oracle_fwd(inp, heads)
    eo = errs(select_heads(o, heads).float().cpu().numpy(), ro)
    eh = errs(select_heads(hT, heads).cpu().numpy(), rh)
    log(f"  vs oracle {fmt('o', eo)} {fmt('hT', eh)}")
    assert eo[0] <= TOL["bf16"] and eh[0] <= TOL["bf16"]
    # a smaller second call right after (other shape, dtype and chunk)
    w2 = gen.Workload("noalloc2", 1, 3, 200, 64, 32, 32, "f32", "ckda_uniform", "normal", 9200)
    log(f"noalloc {w2}")
    _, o2, hT2, o2_ref, h2_ref = run_both(w2)
    assert torch.equal(o2, o2_ref) and torch.equal(hT2, h2_ref)


def test_noalloc_rejects_a_head_larger_than_the_scratch():
    # T = 65536 at d128 bf16 needs 70 MB of records for one head
    L = ck.lib()
    base = 1 << 40   # never dereferenced: the size check fails first
    mb = 1 << 30
    rc = L.ckda_chunk_fwd_noalloc(base, base + mb, base + 2 * mb, base + 3 * mb, base + 4 * mb, None,
                                  base + 5 * mb, None, 1, 1, 65536, 128, 128, 64, 1, None)
    assert rc == ck.ERR_WORKSPACE, rc
    assert b"scratch" in L.ckda_last_error()
