"""The Python binding rejects wrong-shaped tensors before anything reaches the
C ABI (which receives bare pointers and cannot see shapes).  CPU tensors are
enough: the shape checks run before the device check, so a correctly shaped
CPU tensor fails on the device check instead, which shows that the shapes
passed."""
import pytest
import torch

import gated_delta_rule_ckda_amd as ck

B, H, T, DK, DV = 2, 3, 40, 16, 32
bf = dict(dtype=torch.bfloat16)
f32 = dict(dtype=torch.float32)


def fwd_args(**over):
    a = dict(q=torch.zeros(B, H, T, DK, **bf), k=torch.zeros(B, H, T, DK, **bf), v=torch.zeros(B, H, T, DV, **bf),
             alpha=torch.zeros(B, H, T, DK, **bf), beta=torch.zeros(B, H, T, **bf), h0=torch.zeros(B, H, DK, DV, **f32),
             o=torch.zeros(B, H, T, DV, **bf), hT=torch.zeros(B, H, DK, DV, **f32))
    a.update(over)
    return a


def call_fwd(**over):
    a = fwd_args(**over)
    return ck.chunk_fwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["h0"], chunk=16, o=a["o"], hT=a["hT"],
                        fuse=a.get("fuse", 0))


def test_chunk_fwd_good_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        call_fwd()


@pytest.mark.parametrize("name,shape", [
    ("k", (B, H, T, DK + 1)), ("k", (B, H, T - 1, DK)), ("v", (B, H, T + 1, DV)), ("alpha", (B, H, T, 8)),
    ("alpha", (B, H, T)), ("beta", (B, H, T, 1)), ("beta", (B, H, T + 1)), ("h0", (B, H, DV, DK + 1)),
    ("h0", (B, 1, DK, DV)), ("o", (B, H, T, DV // 2)), ("hT", (B, H, DK, DV + 16)), ("q", (B, H, T)),
])
def test_chunk_fwd_rejects_wrong_shapes(name, shape):
    dt = bf if name in ("q", "k", "v", "alpha", "beta", "o") else f32
    with pytest.raises(ValueError, match="shape|dimensions"):
        call_fwd(**{name: torch.zeros(*shape, **dt)})


def test_chunk_fwd_scalar_gate_shape():
    # with the scalar gate alpha is [B, H, T]; a per-channel alpha is then wrong
    with pytest.raises(ValueError, match="GPU tensor"):
        call_fwd(alpha=torch.zeros(B, H, T, **bf), fuse=ck.GATE_SCALAR)
    with pytest.raises(ValueError, match="shape"):
        call_fwd(fuse=ck.GATE_SCALAR)


def test_chunk_fwd_gather_shapes():
    dk_in = 2 * DK
    a = fwd_args(q=torch.zeros(B, H, T, dk_in, **bf), k=torch.zeros(B, H, T, dk_in, **bf),
                 alpha=torch.zeros(B, H, T, dk_in, **bf))
    idx = torch.zeros(H, DK, dtype=torch.int32)
    run = lambda **o: ck.chunk_fwd(*(o.get(n, a[n]) for n in ("q", "k", "v", "alpha", "beta", "h0")), chunk=16,
                                   o=a["o"], hT=a["hT"], idx=o.get("idx", idx))
    with pytest.raises(ValueError, match="GPU tensor"):
        run()
    with pytest.raises(ValueError, match="shape"):
        run(k=torch.zeros(B, H, T, DK, **bf))           # keys must be full-width rows
    with pytest.raises(ValueError, match="idx"):
        run(idx=torch.zeros(H + 1, DK, dtype=torch.int32))


def dec_args(**over):
    N = 4
    a = dict(q=torch.zeros(N, H, DK, **bf), k=torch.zeros(N, H, DK, **bf), v=torch.zeros(N, H, DV, **bf),
             alpha=torch.zeros(N, H, DK, **bf), beta=torch.zeros(N, H, **bf), S=torch.zeros(N, H, DK, DV, **f32),
             o=torch.zeros(N, H, DV, **bf))
    a.update(over)
    return a


@pytest.mark.parametrize("name,shape", [
    (None, None), ("k", (4, H, DK + 16)), ("v", (4, H + 1, DV)), ("alpha", (4, H)), ("beta", (4, H, 1)),
    ("S", (4, H, DK, DV - 16)), ("S", (3, H, DK, DV)), ("o", (4, H, DK)),
])
def test_decode_step_shapes(name, shape):
    a = dec_args() if name is None else dec_args(**{name: torch.zeros(*shape, **(f32 if name == "S" else bf))})
    with pytest.raises(ValueError, match="GPU tensor" if name is None else "shape"):
        ck.decode_step(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["S"], o=a["o"])


@pytest.mark.parametrize("name,shape", [
    (None, None), ("k", (B, H, T, DK * 2)), ("alpha", (B, H, T, DK - 1)), ("beta", (B, H, 1)),
    ("do", (B, H, T, DK)), ("h0", (B, H, DK, DK)), ("dhT", (H, B, DK, DV)),
])
def test_chunk_bwd_shapes(name, shape):
    a = fwd_args()
    a["do"] = torch.zeros(B, H, T, DV, **bf)
    a["dhT"] = torch.zeros(B, H, DK, DV, **f32)
    if name is not None:
        a[name] = torch.zeros(*shape, **(f32 if name in ("h0", "dhT") else bf))
    with pytest.raises(ValueError, match="GPU tensor" if name is None else "shape"):
        ck.chunk_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["do"], h0=a["h0"], dhT=a["dhT"])


@pytest.mark.parametrize("name,shape", [
    (None, None), ("k", (B, H, T, DK)), ("v", (B, H, T, 2, DV + 16)), ("beta", (B, H, T)),
    ("alpha", (B, H, T, DK)), ("h0", (B, H, DK + 16, DV)), ("o", (B, H, 2 * T, DV)), ("hT", (B, H, DV, DV)),
])
def test_deltaproduct2_fwd_shapes(name, shape):
    a = dict(q=torch.zeros(B, H, T, DK, **bf), k=torch.zeros(B, H, T, 2, DK, **bf),
             v=torch.zeros(B, H, T, 2, DV, **bf), beta=torch.zeros(B, H, T, 2, **bf), alpha=torch.zeros(B, H, T, **bf),
             h0=torch.zeros(B, H, DK, DV, **f32), o=torch.zeros(B, H, T, DV, **bf), hT=torch.zeros(B, H, DK, DV, **f32))
    if name is not None:
        a[name] = torch.zeros(*shape, **(f32 if name in ("h0", "hT") else bf))
    with pytest.raises(ValueError, match="GPU tensor" if name is None else "shape"):
        ck.deltaproduct2_fwd(a["q"], a["k"], a["v"], a["beta"], alpha=a["alpha"], h0=a["h0"], o=a["o"], hT=a["hT"])


@pytest.mark.parametrize("name,shape", [
    (None, None), ("k", (4, H, DK)), ("beta", (4, H)), ("alpha", (4, H, DK)), ("S", (4, H, DK, 16)),
    ("o", (4, H, 2, DV)),
])
def test_deltaproduct2_decode_shapes(name, shape):
    N = 4
    a = dict(q=torch.zeros(N, H, DK, **bf), k=torch.zeros(N, H, 2, DK, **bf), v=torch.zeros(N, H, 2, DV, **bf),
             beta=torch.zeros(N, H, 2, **bf), alpha=torch.zeros(N, H, **bf), S=torch.zeros(N, H, DK, DV, **f32),
             o=torch.zeros(N, H, DV, **bf))
    if name is not None:
        a[name] = torch.zeros(*shape, **(f32 if name == "S" else bf))
    with pytest.raises(ValueError, match="GPU tensor" if name is None else "shape"):
        ck.deltaproduct2_decode_step(a["q"], a["k"], a["v"], a["beta"], a["S"], alpha=a["alpha"], o=a["o"])


@pytest.mark.parametrize("name,shape", [
    (None, None), ("k", (B, H, T, DK)), ("do", (B, H, T, 2, DV)), ("dhT", (B, H, DK, DV + 1)),
])
def test_deltaproduct2_bwd_shapes(name, shape):
    a = dict(q=torch.zeros(B, H, T, DK, **bf), k=torch.zeros(B, H, T, 2, DK, **bf),
             v=torch.zeros(B, H, T, 2, DV, **bf), beta=torch.zeros(B, H, T, 2, **bf), alpha=None,
             do=torch.zeros(B, H, T, DV, **bf), h0=None, dhT=torch.zeros(B, H, DK, DV, **f32))
    if name is not None:
        a[name] = torch.zeros(*shape, **(f32 if name == "dhT" else bf))
    with pytest.raises(ValueError, match="GPU tensor" if name is None else "shape"):
        ck.deltaproduct2_bwd(a["q"], a["k"], a["v"], a["alpha"], a["beta"], a["do"], h0=a["h0"], dhT=a["dhT"])
