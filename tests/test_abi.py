"""The C ABI without a GPU: the library loads, exports every function that
include/ckda.h declares, and rejects bad arguments before launching anything
(so these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_ckda_amd as ck

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckda.h")

BASE = 0x7F0000000000   # fake, never-dereferenced device addresses
MB = 1 << 20
HIP, WS = ck.ERR_HIP, ck.ERR_WORKSPACE   # 5 and 6


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ckda_\w+)\s*\(", text)))


def test_library_exports_every_declared_function():
    L = ck.lib()
    names = declared_functions()
    assert set(names) == set(ck.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.ckda_abi_version() == 1


def test_status_numbering():
    """Codes 0-5 keep the boundary's original numbering (CKDA_ERR_HIP = 5);
    the workspace and flag codes were added after it."""
    text = open(HEADER).read()
    vals = dict((n, int(v)) for n, v in re.findall(r"\b(CKDA_(?:OK|ERR_\w+))\s*=\s*(\d+)", text))
    assert vals == {"CKDA_OK": 0, "CKDA_ERR_NULL": 1, "CKDA_ERR_DIM": 2, "CKDA_ERR_UNSUPPORTED": 3,
                    "CKDA_ERR_ALIAS": 4, "CKDA_ERR_HIP": 5, "CKDA_ERR_WORKSPACE": 6, "CKDA_ERR_FLAGS": 7}
    assert {v: "CKDA_" + k for v, k in ((v, n[5:]) for n, v in vals.items())} == ck.STATUS
    L = ck.lib()
    assert L.ckda_status_string(5) == b"HIP runtime error"
    assert b"workspace" in L.ckda_status_string(6)


def test_status_strings():
    L = ck.lib()
    for s in range(8):
        assert L.ckda_status_string(s) != b"unknown status"
    assert L.ckda_status_string(99) == b"unknown status"


def test_workspace_size():
    L = ck.lib()
    ws = L.ckda_chunk_fwd_workspace_size
    # bf16, chunk 64, d_k 128: the record is a sequence of 1 KB fragments --
    # TB, its lo part and M (4 row tiles x 2 K blocks, less the 2 blocks
    # above the diagonal), W and Q~ (4 x 4 each), KR (8 x 2) and one block for
    # the d_k fp32 chunk decays
    per_chunk = ws(1, 1, 64, 128, 128, 64, 1)
    assert per_chunk == 1024 * (3 * 6 + 2 * 16 + 16 + 1)
    assert ws(1, 1, 64, 64, 128, 64, 1) == 1024 * (3 * 6 + 2 * 8 + 8 + 1)
    assert ws(1, 1, 32, 128, 128, 32, 1) == 1024 * (3 * 2 + 2 * 8 + 8 + 1)
    # fp32: K blocks of 16 elements (lower triangle of 4 x 4 blocks)
    assert ws(1, 1, 64, 128, 128, 64, 0) == 1024 * (2 * 10 + 2 * 32 + 32 + 1)
    assert ws(4, 16, 4096, 128, 128, 64, 1) == 64 * 64 * per_chunk
    assert ws(1, 1, 65, 128, 128, 64, 1) == 2 * per_chunk       # ragged tail = one more chunk
    assert ws(1, 1, 64, 128, 128, 48, 1) == 0                  # unsupported chunk
    assert ws(1, 1, 64, 96, 128, 64, 1) == 0                   # unsupported dk
    assert ws(1, 1, 64, 128, 128, 64, 7) == 0                  # unsupported dtype
    assert ws(-1, 1, 64, 128, 128, 64, 1) == 0
    assert ws(1, 1, 64, 16, 16, 16, 0) > 0


def call_fwd(**kw):
    L = ck.lib()
    B, H, T, dk, dv = kw.get("B", 1), kw.get("H", 2), kw.get("T", 64), kw.get("dk", 64), kw.get("dv", 64)
    chunk, dtype = kw.get("chunk", 64), kw.get("dtype", 1)
    p = dict(q=BASE, k=BASE + 1 * MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB,
             h0=BASE + 5 * MB, o=BASE + 6 * MB, hT=BASE + 7 * MB, ws=BASE + 8 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    wsb = kw.get("wsb", 64 * MB)
    args = (p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["h0"], p["o"], p["hT"], B, H, T, dk, dv, chunk, dtype)
    if "flags" in kw:
        rc = L.ckda_chunk_fwd_ex(*args, kw["flags"], p["ws"], wsb, None)
    else:
        rc = L.ckda_chunk_fwd(*args, p["ws"], wsb, None)
    return rc, L.ckda_last_error().decode()


def call_dec(**kw):
    L = ck.lib()
    N, H, dk, dv, dtype = kw.get("N", 2), kw.get("H", 2), kw.get("dk", 64), kw.get("dv", 64), kw.get("dtype", 1)
    p = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB,
             S=BASE + 5 * MB, o=BASE + 6 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    args = (p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["S"], p["o"], N, H, dk, dv, dtype)
    if "flags" in kw:
        rc = L.ckda_decode_step_ex(*args, kw["flags"], None)
    else:
        rc = L.ckda_decode_step(*args, None)
    return rc, L.ckda_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(beta=None), 1),
    (dict(T=-1), 2), (dict(B=-2), 2),
    (dict(T=1 << 24, dv=128), 2),                                 # one head's output over 2 GiB
    (dict(dk=48), 3), (dict(dv=256), 3), (dict(chunk=128), 3), (dict(dtype=2), 3),
    (dict(q=BASE + 2), 2),                                        # misaligned
    (dict(o=BASE + 2 * MB + 64), 4),                              # o overlaps v
    (dict(hT=BASE + 16), 4),                                      # hT overlaps q
    (dict(hT=BASE + 5 * MB + 16), 4),                             # hT partially overlaps h0
    (dict(ws=BASE + 6 * MB), 4),                                  # workspace overlaps o
    (dict(ws=None), WS), (dict(wsb=1024), WS), (dict(ws=BASE + 8 * MB + 16), WS),
])
def test_chunk_fwd_rejects(kw, status):
    rc, msg = call_fwd(**kw)
    assert rc == status, (rc, msg)
    assert msg.startswith("ckda_chunk_fwd")


@pytest.mark.parametrize("flags", [16, 32, -1, 1 << 16, 1 << 30])
def test_fused_entry_points_reject_unknown_flags(flags):
    rc, msg = call_fwd(flags=flags)
    assert rc == 7 and msg.startswith("ckda_chunk_fwd"), (rc, msg)
    rc, msg = call_dec(flags=flags)
    assert rc == 7 and msg.startswith("ckda_decode_step"), (rc, msg)


@pytest.mark.parametrize("flags", [0, 1, 2, 3, 4, 7])
def test_fused_entry_points_check_arguments_like_the_plain_ones(flags):
    # valid flags reach the same argument checks (these all fail before a launch)
    assert call_fwd(flags=flags, q=None)[0] == 1
    assert call_fwd(flags=flags, dk=48)[0] == 3
    assert call_fwd(flags=flags, o=BASE + 2 * MB + 64)[0] == 4
    assert call_fwd(flags=flags, wsb=1024)[0] == WS
    assert call_fwd(flags=flags, B=0)[0] == 0
    assert call_dec(flags=flags, S=None)[0] == 1
    assert call_dec(flags=flags, o=BASE + 5 * MB)[0] == 4
    assert call_dec(flags=flags, N=0, q=None)[0] == 0


def call_fwd_gather(**kw):
    L = ck.lib()
    B, H, T, dk, dv, dk_in = kw.get("B", 1), kw.get("H", 2), kw.get("T", 64), kw.get("dk", 64), 64, kw.get("dk_in", 128)
    p = dict(q=BASE, k=BASE + 1 * MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB,
             h0=BASE + 5 * MB, o=BASE + 6 * MB, hT=BASE + 7 * MB, ws=BASE + 8 * MB, idx=BASE + 80 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    rc = L.ckda_chunk_fwd_gather(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["h0"], p["o"], p["hT"], B, H, T,
                                 dk_in, p["idx"], dk, dv, 64, 1, kw.get("flags", 0), p["ws"], 64 * MB, None)
    return rc, L.ckda_last_error().decode()


def call_dec_gather(**kw):
    L = ck.lib()
    p = dict(q=BASE, k=BASE + MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB,
             S=BASE + 5 * MB, o=BASE + 6 * MB, idx=BASE + 80 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    rc = L.ckda_decode_step_gather(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["S"], p["o"], 2, 2,
                                   kw.get("dk_in", 128), p["idx"], 64, 64, 1, kw.get("flags", 0), None)
    return rc, L.ckda_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(idx=None), 1), (dict(dk_in=0), 2), (dict(dk_in=1 << 20), 2), (dict(idx=BASE + 80 * MB + 4), 2),
    (dict(o=BASE + 80 * MB), 4),                       # o overlaps idx
    (dict(flags=16), 7), (dict(dk=48), 3),
    (dict(o=BASE + 20000), 4),                       # o inside q's full-width rows (past its kept width)
])
def test_gather_entry_points_reject(kw, status):
    rc, msg = call_fwd_gather(**kw)
    assert rc == status, (rc, msg)
    if "dk" not in kw and kw.get("o") != BASE + 20000:
        rc, msg = call_dec_gather(**kw)
        assert rc == status and msg.startswith("ckda_decode_step"), (rc, msg)


def test_gather_entry_points_accept_valid_empty_calls():
    assert call_fwd_gather(B=0, idx=None)[0] == 0
    assert call_fwd_gather(H=0, idx=None)[0] == 0


def call_dp2(**kw):
    L = ck.lib()
    B, H, T, dk, dv = 1, 2, kw.get("T", 64), 64, 64
    p = dict(q=BASE, k=BASE + 1 * MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB,
             h0=BASE + 5 * MB, o=BASE + 6 * MB, hT=BASE + 7 * MB, ws=BASE + 8 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    rc = L.ckda_deltaproduct2_fwd(p["q"], p["k"], p["v"], p["alpha"], p["beta"], p["h0"], p["o"], p["hT"], B, H, T,
                                  dk, dv, 64, 1, kw.get("flags", 0), p["ws"], kw.get("wsb", 64 * MB), None)
    return rc, L.ckda_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(beta=None), 1), (dict(flags=8), 7), (dict(flags=1 << 16), 7),
    (dict(o=BASE + 1 * MB + 20000), 4),                # o inside k: 2 T sub-step rows of k (32 KB)
    (dict(wsb=ck.lib().ckda_chunk_fwd_workspace_size(1, 2, 64, 64, 64, 64, 1)), WS),   # sized for T, not 2 T
])
def test_deltaproduct2_rejects(kw, status):
    rc, msg = call_dp2(**kw)
    assert rc == status, (rc, msg)
    assert msg.startswith("ckda_deltaproduct2_fwd")


def test_deltaproduct2_decode_rejects():
    L = ck.lib()
    args = [BASE, BASE + MB, BASE + 2 * MB, None, BASE + 4 * MB, BASE + 5 * MB, BASE + 6 * MB, 2, 2, 64, 64, 1]
    assert L.ckda_deltaproduct2_decode_step(*args, 8, None) == 7
    bad = list(args)
    bad[6] = BASE + 5 * MB + 64                              # o overlaps the state
    assert L.ckda_deltaproduct2_decode_step(*bad, 0, None) == 4
    bad = list(args)
    bad[0] = None
    assert L.ckda_deltaproduct2_decode_step(*bad, 0, None) == 1


def test_scalar_gate_flag_checks():
    # scalar gate: alpha is [B, H, T]; it does not combine with a gather
    assert call_fwd(flags=8, o=BASE + 3 * MB + 128)[0] == 4      # o inside the 256-byte scalar alpha
    assert call_fwd(flags=8, o=BASE + 3 * MB + 512)[0] == HIP     # past it: checks pass (no device here)
    assert call_fwd(flags=0, o=BASE + 3 * MB + 512)[0] == 4      # per-channel alpha is larger
    assert call_fwd_gather(flags=8)[0] == 3


def call_bwd(**kw):
    L = ck.lib()
    B, H, T, dk, dv = 1, 2, kw.get("T", 64), kw.get("dk", 64), 64
    p = dict(q=BASE, k=BASE + 1 * MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB, h0=BASE + 5 * MB,
             do=BASE + 6 * MB, dhT=BASE + 7 * MB, dq=BASE + 8 * MB, dk=BASE + 9 * MB, dv=BASE + 10 * MB,
             da=BASE + 11 * MB, db=BASE + 12 * MB, dh0=BASE + 13 * MB, ws=BASE + 16 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    ptrs = (p[n] for n in ("q", "k", "v", "alpha", "beta", "h0", "do", "dhT", "dq", "dk", "dv", "da", "db", "dh0"))
    if "flags" in kw:
        rc = L.ckda_chunk_bwd_ex(*ptrs, B, H, T, dk, dv, kw.get("dtype", 1), kw["flags"], p["ws"],
                                 kw.get("wsb", 64 * MB), None)
    else:
        rc = L.ckda_chunk_bwd(*ptrs, B, H, T, dk, dv, kw.get("dtype", 1), p["ws"], kw.get("wsb", 64 * MB), None)
    return rc, L.ckda_last_error().decode()


def test_bwd_workspace_size():
    L = ck.lib()
    # per 32-position chunk: (5*32*32 + 5*32*dk + dk) floats rounded to 64, plus 2 dk dv floats
    per = ((5 * 32 * 32 + 5 * 32 * 128 + 128 + 63) // 64 * 64 + 2 * 128 * 128) * 4
    assert L.ckda_chunk_bwd_workspace_size(1, 1, 32, 128, 128, 1) == per
    assert L.ckda_chunk_bwd_workspace_size(4, 16, 4096, 128, 128, 1) == 64 * 128 * per
    assert L.ckda_chunk_bwd_workspace_size(1, 1, 33, 128, 128, 1) == 2 * per
    assert L.ckda_chunk_bwd_workspace_size(1, 1, 32, 96, 128, 1) == 0
    assert L.ckda_chunk_bwd_workspace_size(1, 1, 32, 128, 128, 5) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(da=None), 1),
    (dict(T=-1), 2), (dict(dk=48), 3), (dict(dtype=3), 3),
    (dict(ws=None), WS), (dict(wsb=1024), WS),
    (dict(dq=BASE + 2), 2),
    (dict(dq=BASE + 1 * MB), 4),                 # dq overlaps k
    (dict(dv=BASE + 8 * MB + 64), 4),            # dv overlaps dq
    (dict(dh0=BASE + 16 * MB + 256), 4),         # dh0 inside the workspace
])
def test_bwd_rejects(kw, status):
    rc, msg = call_bwd(**kw)
    assert rc == status, (rc, msg)
    assert msg.startswith("ckda_chunk_bwd")


def test_bwd_ex_workspace_size():
    L = ck.lib()
    B, H, T, dk, dv = 2, 3, 100, 64, 32
    plain = L.ckda_chunk_bwd_workspace_size(B, H, T, dk, dv, 1)
    assert L.ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, 1, 0) == plain
    part = lambda n: (n + 63) // 64 * 64 * 4     # fp32 parts, 256-byte aligned
    ntok = B * H * T
    extra = 3 * part(ntok * dk) + 2 * part(ntok * dv) + part(ntok)
    assert L.ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, 1, 7) == plain + extra
    assert L.ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, 1, 8 | 1) == plain + extra + part(ntok * dk)
    assert L.ckda_chunk_bwd_ex_workspace_size(B, H, T, dk, dv, 1, 16) == 0      # unknown flag bit
    assert L.ckda_chunk_bwd_ex_workspace_size(B, H, T, 48, dv, 1, 7) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(flags=16), 7),                                   # unknown flag bit
    (dict(flags=7, wsb=4096), WS),                         # too small for the prologue's fp32 copies
    (dict(flags=7, q=None), 1),
    (dict(flags=7, dq=BASE + 1 * MB), 4),                  # dq overlaps k
    (dict(flags=1, da=BASE + 3 * MB + 512), 4),            # per-channel alpha (16 KB) overlaps dalpha ...
])
def test_bwd_ex_rejects(kw, status):
    rc, msg = call_bwd(**kw)
    assert rc == status, (rc, msg)
    assert msg.startswith("ckda_chunk_bwd_ex")


def test_bwd_ex_scalar_gate_sizes():
    # with one gate per token alpha and dalpha are B*H*T long (256 bytes of
    # bf16 here): a dalpha 128 bytes into alpha overlaps it
    rc, msg = call_bwd(flags=9, da=BASE + 3 * MB + 128)
    assert rc == 4, (rc, msg)
    assert "dalpha overlaps alpha" in msg


def test_dp2_bwd_workspace_size():
    L = ck.lib()
    B, H, T, dk, dv = 1, 2, 40, 64, 32
    part = lambda n: (n + 255) // 256 * 256
    nsub = 2 * B * H * T
    want = 2 * part(nsub * dk * 2) + part(nsub * dv * 2) + 2 * part(nsub * dk * 4) + \
        L.ckda_chunk_bwd_workspace_size(B, H, 2 * T, dk, dv, 1)
    assert L.ckda_deltaproduct2_bwd_workspace_size(B, H, T, dk, dv, 1) == want
    assert L.ckda_deltaproduct2_bwd_workspace_size(B, H, 1 << 30, dk, dv, 1) == 0
    assert L.ckda_deltaproduct2_bwd_workspace_size(B, H, T, 24, dv, 1) == 0


def _call_dp2_bwd(**kw):
    L = ck.lib()
    B, H, T, dk, dv = 1, 2, kw.get("T", 64), 64, 64
    p = dict(q=BASE, k=BASE + 1 * MB, v=BASE + 2 * MB, alpha=BASE + 3 * MB, beta=BASE + 4 * MB, h0=BASE + 5 * MB,
             do=BASE + 6 * MB, dhT=BASE + 7 * MB, dq=BASE + 8 * MB, dk=BASE + 9 * MB, dv=BASE + 10 * MB,
             da=BASE + 11 * MB, db=BASE + 12 * MB, dh0=BASE + 13 * MB, ws=BASE + 16 * MB)
    p.update({k: v for k, v in kw.items() if k in p})
    rc = L.ckda_deltaproduct2_bwd(*(p[n] for n in ("q", "k", "v", "alpha", "beta", "h0", "do", "dhT", "dq", "dk",
                                                   "dv", "da", "db", "dh0")), B, H, T, dk, dv, 1, p["ws"],
                                  kw.get("wsb", 4096), None)
    return rc, L.ckda_last_error().decode()


@pytest.mark.parametrize("kw,status", [
    (dict(da=None), 1),                          # a gated call needs dalpha
    (dict(T=-1), 2), (dict(T=1 << 30), 2),
    (dict(wsb=4096), WS),                       # too small
    (dict(dq=BASE + 1 * MB, wsb=64 * MB), 4),    # dq overlaps k (2 T sub-steps of keys)
    (dict(dk=BASE + 9 * MB + 4, wsb=64 * MB), 2),
])
def test_dp2_bwd_rejects(kw, status):
    rc, msg = _call_dp2_bwd(**kw)
    assert rc == status, (rc, msg)
    assert msg.startswith("ckda_deltaproduct2_bwd")


def test_prologue_flag_values_agree():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define (CKDA_FUSE_\w+) (\d+)", text))
    assert {k: int(v) for k, v in defs.items()} == {"CKDA_FUSE_GATES": ck.FUSE_GATES,
                                                     "CKDA_FUSE_NORM_K": ck.FUSE_NORM_K,
                                                     "CKDA_FUSE_NORM_Q": ck.FUSE_NORM_Q}
    import oracle
    assert (oracle.GATES, oracle.NORM_K, oracle.NORM_Q) == (ck.FUSE_GATES, ck.FUSE_NORM_K, ck.FUSE_NORM_Q)


def test_chunk_fwd_empty_problems_are_noops():
    assert call_fwd(B=0)[0] == 0
    assert call_fwd(H=0, q=None, o=None)[0] == 0
    assert call_fwd(T=0, hT=None, q=None, k=None, v=None, alpha=None, beta=None, o=None, ws=None)[0] == 0


@pytest.mark.parametrize("kw,status", [
    (dict(S=None), 1), (dict(o=None), 1),
    (dict(N=-1), 2), (dict(dk=8), 3), (dict(dtype=5), 3),
    (dict(o=BASE + 5 * MB), 4),                                   # o overlaps the state
    (dict(S=BASE + 16), 4),                                       # state overlaps q
    (dict(alpha=BASE + 3 * MB + 4), 2),                           # misaligned
])
def test_decode_rejects(kw, status):
    rc, msg = call_dec(**kw)
    assert rc == status, (rc, msg)
    assert msg.startswith("ckda_decode_step")


def test_decode_empty_is_noop():
    assert call_dec(N=0, q=None)[0] == 0


def test_python_binding_requires_gpu_tensors():
    import torch
    x = torch.zeros((1, 1, 16, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ck.chunk_fwd(x, x, x, x, torch.zeros((1, 1, 16), dtype=torch.bfloat16), chunk=16)
