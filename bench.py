#!/usr/bin/env python3
"""Benchmark of the CKDA hot path on one MI355X.

One step = one chunkwise forward of the ckda_bf16 workload (B4 H16 T4096,
d_k = d_v = 128, chunk 64, full CKDA gate ranges, h0 ~ N(0, 0.1)): gate sign
and magnitude split, Gram matrices, triangular solve, state pass and output,
plus the final state.  The decode step (256 sequences x 32 heads, d128, fp32
state updated in place) is timed in the same run and reported under "decode",
both again with the per-token prologue fused (gates from logits, unit-norm
keys) under "fused_prologue", the state-reduced workload (B2 H32 T32768,
d_k 64 kept of 128 channels by an in-kernel gather) under "channel_gather",
the KDA workload (B4 H16 T2048, positive gates) under "kda", the
comparators (scalar gate; DeltaProduct_2 forward and decode) under
"comparators", and the backward (all gradients) with the forward + backward
throughput under "backward".

Prints ONE JSON line.  `value` is tokens/s of the forward (a token is one
(batch, position) across all heads), inputs resident in HBM: tokens per step
divided by `ms_per_step`, the wall time of the K timed steps (synchronised on
both sides) divided by K.  HIP events on the kernels' stream give the per-call
time and, in a second run of K steps, each kernel's duration ("roofline").
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix cores, TFLOP/s
METRIC = "CKDA chunkwise fwd tokens/s (B4 H16 T4096 d128, %MFMA) + decode state GB/s"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--decode-steps", type=int, default=128)
    p.add_argument("--workload", default="ckda_bf16",
                   help="forward workload name (default: the headline ckda_bf16)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skip-extras", action="store_true",
                   help="headline forward and decode only (for counter runs)")
    p.add_argument("--protocol-trials", type=int, default=3,
                   help="trials of 100 calls for the median-of-medians timing (0: skip, for counter runs)")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="about this much oracle work for the CPU baseline (whole-workload passes)")
    return p.parse_args()


def kernel_algorithmic(w):
    """Algorithmic HBM bytes of each of the forward's two kernels: the method's
    own inputs and outputs that the kernel reads or writes.  The Gram kernel
    reads q, k, alpha and beta; the state-pass kernel reads v and h0 and writes
    o and hT.  The chunk records the first writes and the second reads are
    this design's intermediate ("record_bytes"), not algorithmic traffic."""
    es = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    state = w.B * w.H * w.dk * w.dv * 4 * (2 if w.h0 == "normal" else 1)
    return {"chunk_gram_kernel": th * (3 * w.dk + 1) * es,
            "chunk_state_kernel": th * 2 * w.dv * es + state}


KERNEL_SOURCES = {"chunk_gram_kernel": "chunk_gram.hip", "chunk_state_kernel": "chunk_state.hip"}
DEVICE_HEADERS = ("chunk_common.hpp", "ckda_device.hpp")


def kernel_source_sha(kernel):
    """sha256 of the kernel's source file followed by the device headers it
    includes (the counters belong to the code all of them make)."""
    import hashlib
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel],) + DEVICE_HEADERS:
        with open(os.path.join(ROOT, "gated_delta_rule_ckda_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_from_profile(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None when the kernel's source changed after the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"{kernel}_ckda_bf16_hbm_counters.md")
    try:
        text = open(path).read()
        sha = kernel_source_sha(kernel)
    except OSError:
        return None
    m_sha = re.search(r"source sha256: `([0-9a-f]{64})`", text)
    m_b = re.search(r"HBM bytes per launch: ([0-9]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sha:
        return None
    return int(m_b.group(1))


def counters_from_profile(name, kernels):
    """Executed matrix-core figures per kernel from a committed counter summary
    (profiles/<name>.md: lines `kernel <name> mfma_busy_frac <x>`), or None
    when any listed kernel's source changed after the counters were taken."""
    import re
    path = os.path.join(ROOT, "profiles", f"{name}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    out = {}
    for k in kernels:
        sha = kernel_source_sha(k)
        m_sha = re.search(rf"{k} source sha256: `([0-9a-f]{{64}})`", text)
        m_v = re.search(rf"kernel {k} mfma_busy_frac ([0-9.]+)", text)
        if not m_sha or not m_v or m_sha.group(1) != sha:
            return None
        out[k] = float(m_v.group(1))
    return out


def trial_medians(fn, stream, trials=3, calls=100, warmup=10):
    """The pages' timing protocol (the state-reduction slides: 10 warm-ups,
    100 measured steps, median of 3 trials): HIP events on `stream` around
    each call, the median per trial, then the median of the trial medians (ms)."""
    import numpy as np
    import torch
    if trials <= 0:
        return None, []
    for _ in range(warmup):
        fn()
    meds = []
    for _ in range(trials):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        meds.append(float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])))
    return float(np.median(meds)), meds


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def fwd_algorithmic(w):
    """Algorithmic HBM bytes and matrix-core flops of one chunkwise forward.
    Bytes: q, k, alpha, v read, o written ((3 dk + 2 dv + 1) elements per
    token-head, beta included), plus the state read (h0) and written (hT).
    Flops: 6 dk dv + 3 C dk + 2 C dv per token-head (the products W H, Q H,
    KR U at 2 dk dv each; the Gram matrices A, M and T (beta K) at ~C dk each;
    T (beta V) and M U at ~C dv each; triangles counted once)."""
    es = 2 if w.dtype == "bf16" else 4
    th = w.B * w.H * w.T
    state = w.B * w.H * w.dk * w.dv * 4 * (2 if w.h0 == "normal" else 1)
    nbytes = th * (3 * w.dk + 2 * w.dv + 1) * es + state
    flops = th * (6 * w.dk * w.dv + 3 * w.chunk * w.dk + 2 * w.chunk * w.dv)
    return nbytes, flops


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                          "(heads and decode states shard across GPUs without exchange, "
                          "but no multi-GPU path is built)"}))
        return 2

    import numpy as np
    import torch

    import gated_delta_rule_ckda_amd as ck
    from gated_delta_rule_ckda_amd import inputs as gen

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = gen.WORKLOADS[a.workload]
    log = lambda m: print(m, file=sys.stderr, flush=True)
    log(f"[bench] generating {w}")
    inp = gen.make_inputs(w)
    d = {k: (None if v is None else v.to(dev)) for k, v in inp.items()}
    ws = torch.empty(ck.workspace_size(w.B, w.H, w.T, w.dk, w.dv, w.chunk, ck.DTYPE_BF16 if w.dtype == "bf16"
                                       else ck.DTYPE_F32), dtype=torch.uint8, device=dev)
    o = torch.empty((w.B, w.H, w.T, w.dv), dtype=d["q"].dtype, device=dev)
    hT = torch.empty((w.B, w.H, w.dk, w.dv), dtype=torch.float32, device=dev)

    stream = torch.cuda.current_stream()

    def step(events=None):
        ck.chunk_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["h0"], chunk=w.chunk,
                     workspace=ws, o=o, hT=hT, events=events)

    log(f"[bench] warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    # Timed region 1: K steps bracketed by synchronisation, events before and
    # after each call (the tokens/s value and the per-call time).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    log(f"[bench] timing {a.steps} forward steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(a.steps):
        ev[s][0].record(stream)
        step()
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    # Timed region 2: K more steps through ckda_chunk_fwd_timed, whose events
    # (recorded by the library on this stream before the Gram kernel, between
    # the kernels and after the state-pass kernel) give each kernel's duration.
    kev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
    for e3 in kev:
        for e in e3:
            e.record(stream)   # creates the event
    torch.cuda.synchronize()
    for s in range(a.steps):
        step(kev[s])
    torch.cuda.synchronize()
    gram_ms = [e[0].elapsed_time(e[1]) for e in kev]
    state_ms = [e[1].elapsed_time(e[2]) for e in kev]
    # Timed region 3: the same call captured once in a HIP graph and replayed K
    # times (events around each replay): the launch path without the host.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            step()
    stream.wait_stream(cap)
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    graph.replay()
    torch.cuda.synchronize()
    for e0, e1 in gev:
        e0.record(stream)
        graph.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    graph_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in gev]))
    del graph
    # Timed region 4: the pages' protocol (3 trials of 100 calls after 10
    # warm-ups, median of the trial medians), per-call events
    log("[bench] protocol timing: 3 trials x 100 calls")
    proto_ms, proto_trials = trial_medians(step, stream, trials=a.protocol_trials)
    # This very output on two sampled heads (the heads are independent
    # recurrences), kept for the comparison with the oracle in the CPU leg
    step()
    torch.cuda.synchronize()
    heads = [0, w.B * w.H - 1]
    sel = lambda t: t.reshape(w.B * w.H, *t.shape[2:])[heads].unsqueeze(1).contiguous()
    gpu_sample = (sel(o.float().cpu()).numpy(), sel(hT.cpu()).numpy())
    call_ms = float(np.mean(per_call_ms))
    call_ms_median = float(np.median(per_call_ms))
    kern_ms = {"chunk_gram_kernel": float(np.mean(gram_ms)), "chunk_state_kernel": float(np.mean(state_ms))}
    ms_per_step = wall * 1e3 / a.steps
    tokens = w.B * w.T
    value = tokens / (ms_per_step * 1e-3)
    nbytes, flops = fwd_algorithmic(w)
    achieved_gbs = nbytes / (call_ms * 1e-3) / 1e9
    achieved_tflops = flops / (call_ms * 1e-3) / 1e12
    kbytes = kernel_algorithmic(w)
    record_bytes = ws.numel()
    dominant = max(kern_ms, key=kern_ms.get)
    dom_gbs = kbytes[dominant] / (kern_ms[dominant] * 1e-3) / 1e9

    # ---- decode: 256 x 32 states, fp32 128x128 each, updated in place
    dec = gen.DECODE
    log(f"[bench] decode {dec}")
    S = gen.decode_state(dec).to(dev)
    dsteps = [gen.decode_step_inputs(s % 8, dec) for s in range(8)]
    dsteps = [{k: v.to(dev) for k, v in x.items()} for x in dsteps]
    do = torch.empty((dec.N, dec.H, dec.dv), dtype=torch.bfloat16, device=dev)

    def dstep(s):
        x = dsteps[s % 8]
        ck.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S, o=do)

    # one step on sampled states: the states before and after and the output,
    # kept for the comparison with the oracle in the CPU leg
    ds_idx = [0, 4099, dec.N * dec.H - 1]
    S_flat = S.view(dec.N * dec.H, dec.dk, dec.dv)
    dsel = lambda t: t.reshape(dec.N * dec.H, *t.shape[2:])[ds_idx].unsqueeze(1).contiguous()
    S_before = S_flat[ds_idx].double().cpu().numpy()[:, None].copy()
    dstep(0)
    torch.cuda.synchronize()
    dec_sample = (S_before, {n: dsel(dsteps[0][n]).cpu() for n in ("q", "k", "v", "alpha", "beta")},
                  dsel(do.float()).cpu().numpy(), S_flat[ds_idx].unsqueeze(1).cpu().numpy())
    for s in range(a.warmup):
        dstep(s)
    torch.cuda.synchronize()
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(a.decode_steps)]
    t1 = time.perf_counter()
    for s in range(a.decode_steps):
        dev_ev[s][0].record(stream)
        dstep(s)
        dev_ev[s][1].record(stream)
    torch.cuda.synchronize()
    dwall = time.perf_counter() - t1
    dms = [e0.elapsed_time(e1) for e0, e1 in dev_ev]
    dec_ms = float(np.mean(dms))
    dec_proto_ms, dec_proto_trials = trial_medians(lambda: dstep(0), stream, trials=a.protocol_trials)
    state_bytes = dec.N * dec.H * dec.dk * dec.dv * 4 * 2
    io_bytes = dec.N * dec.H * (3 * dec.dk + 2 * dec.dv + 1) * 2
    dec_gbs_state = state_bytes / (dec_ms * 1e-3) / 1e9
    dec_gbs_total = (state_bytes + io_bytes) / (dec_ms * 1e-3) / 1e9

    def extras():
        """The variants beside the headline: fused prologue, channel gather,
        backward, comparators (each timed with HIP events on the stream)."""
        # ---- the same forward and decode step with the per-token prologue fused
        # (gates and beta from logits, unit-norm keys): ckda_chunk_fwd_ex and
        # ckda_decode_step_ex, per-call HIP events on the same stream
        fuse = ck.FUSE_GATES | ck.FUSE_NORM_K
        log(f"[bench] fused prologue, flags {fuse}")
        lg = {k: (None if v is None else v.to(dev)) for k, v in gen.make_logit_inputs(w).items()}

        def fstep():
            ck.chunk_fwd(lg["q"], lg["k"], lg["v"], lg["alpha"], lg["beta"], lg["h0"], chunk=w.chunk,
                         workspace=ws, o=o, hT=hT, fuse=fuse)

        for _ in range(a.warmup):
            fstep()
        torch.cuda.synchronize()
        fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
        for s in range(a.steps):
            fev[s][0].record(stream)
            fstep()
            fev[s][1].record(stream)
        torch.cuda.synchronize()
        fused_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in fev]))
        dlg = [{k: v.to(dev) for k, v in gen.decode_logit_inputs(s, dec).items()} for s in range(8)]
        for s in range(a.warmup):
            x = dlg[s % 8]
            ck.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S, o=do, fuse=fuse)
        torch.cuda.synchronize()
        for s in range(a.decode_steps):
            x = dlg[s % 8]
            dev_ev[s][0].record(stream)
            ck.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], S, o=do, fuse=fuse)
            dev_ev[s][1].record(stream)
        torch.cuda.synchronize()
        fdec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dev_ev]))

        # ---- state-reduced workload (B2 H32 T32768, d_k 64 kept of 128 channels,
        # d_v 128) with the channel gather inside the kernels, beside the plain
        # forward on inputs gathered beforehand
        gw, dk_in = gen.WORKLOADS["ckda_long_dk64"], 128
        log(f"[bench] channel gather {gw} from {dk_in} channels")
        gidx = gen.retained_channels(gw.H, dk_in, gw.dk, 4242)
        gin = gen.make_gather_inputs(gw, dk_in, gidx)
        gd = {k: (None if v is None else v.to(dev)) for k, v in gin.items()}
        gidx_d = gidx.to(dev)
        pre = {n: torch.stack([gd[n][:, h].index_select(-1, gidx_d[h].long()) for h in range(gw.H)], 1).contiguous()
               for n in ("q", "k", "alpha")}
        gws = torch.empty(ck.workspace_size(gw.B, gw.H, gw.T, gw.dk, gw.dv, gw.chunk, ck.DTYPE_BF16), dtype=torch.uint8,
                          device=dev)
        go = torch.empty((gw.B, gw.H, gw.T, gw.dv), dtype=torch.bfloat16, device=dev)
        ghT = torch.empty((gw.B, gw.H, gw.dk, gw.dv), dtype=torch.float32, device=dev)

        def timed(fn, n):
            for _ in range(max(1, a.warmup)):
                fn()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            for e0, e1 in evs:
                e0.record(stream)
                fn()
                e1.record(stream)
            torch.cuda.synchronize()
            return float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))

        gsteps = max(3, a.steps // 3)
        gather_ms = timed(lambda: ck.chunk_fwd(gd["q"], gd["k"], gd["v"], gd["alpha"], gd["beta"], gd["h0"],
                                               chunk=gw.chunk, workspace=gws, o=go, hT=ghT, idx=gidx_d), gsteps)
        pregathered_ms = timed(lambda: ck.chunk_fwd(pre["q"], pre["k"], gd["v"], pre["alpha"], gd["beta"], gd["h0"],
                                                    chunk=gw.chunk, workspace=gws, o=go, hT=ghT), gsteps)
        del pre, gd, gws, go

        # ---- the KDA workload (B4 H16 T2048: positive gates, beta in (0, 1), h0 = 0)
        kw = gen.WORKLOADS["kda_bf16"]
        log(f"[bench] KDA workload {kw}")
        kin = {k: (None if v is None else v.to(dev)) for k, v in gen.make_inputs(kw).items()}
        kws = torch.empty(ck.workspace_size(kw.B, kw.H, kw.T, kw.dk, kw.dv, kw.chunk, ck.DTYPE_BF16), dtype=torch.uint8,
                          device=dev)
        ko = torch.empty((kw.B, kw.H, kw.T, kw.dv), dtype=torch.bfloat16, device=dev)
        khT = torch.empty((kw.B, kw.H, kw.dk, kw.dv), dtype=torch.float32, device=dev)
        kda_ms = timed(lambda: ck.chunk_fwd(kin["q"], kin["k"], kin["v"], kin["alpha"], kin["beta"], kin["h0"],
                                            chunk=kw.chunk, workspace=kws, o=ko, hT=khT), a.steps)
        kda_bytes, _ = fwd_algorithmic(kw)
        del kin, kws, ko, khT

        # ---- backward on the bench workload (ckda_chunk_bwd, fp32 gradients)
        log("[bench] backward")
        bdo, bdhT = gen.make_output_grads(w, 99)
        bdo, bdhT = bdo.to(dev), bdhT.to(dev)
        bws = torch.empty(ck.bwd_workspace_size(w.B, w.H, w.T, w.dk, w.dv, ck.DTYPE_BF16), dtype=torch.uint8, device=dev)
        bwd_ms = timed(lambda: ck.chunk_bwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], bdo, h0=d["h0"], dhT=bdhT,
                                            workspace=bws), max(3, a.steps // 3))
        del bws
        # the same through the prologue (ckda_chunk_bwd_ex): gradients with respect to
        # the gate and beta logits and the raw keys, on the fused prologue's inputs
        bws = torch.empty(ck.bwd_ex_workspace_size(w.B, w.H, w.T, w.dk, w.dv, ck.DTYPE_BF16, fuse), dtype=torch.uint8,
                          device=dev)
        bwdx_ms = timed(lambda: ck.chunk_bwd(lg["q"], lg["k"], lg["v"], lg["alpha"], lg["beta"], bdo, h0=lg["h0"],
                                             dhT=bdhT, workspace=bws, fuse=fuse), max(3, a.steps // 3))
        del bws, lg

        # ---- comparators on the bench shape: the scalar (Gated DeltaNet) gate and
        # ungated DeltaProduct_2 (two delta-rule updates per token), and the
        # DeltaProduct_2 decode step on the decode workload
        log("[bench] comparators")
        sg = {k: (None if v is None else v.to(dev)) for k, v in gen.make_scalar_gate_inputs(w).items()}
        scalar_ms = timed(lambda: ck.chunk_fwd(sg["q"], sg["k"], sg["v"], sg["alpha"], sg["beta"], sg["h0"],
                                               chunk=w.chunk, workspace=ws, o=o, hT=hT, fuse=ck.GATE_SCALAR), a.steps)
        bws = torch.empty(ck.bwd_ex_workspace_size(w.B, w.H, w.T, w.dk, w.dv, ck.DTYPE_BF16, ck.GATE_SCALAR),
                          dtype=torch.uint8, device=dev)
        scalar_bwd_ms = timed(lambda: ck.chunk_bwd(sg["q"], sg["k"], sg["v"], sg["alpha"], sg["beta"], bdo, h0=sg["h0"],
                                                   dhT=bdhT, workspace=bws, fuse=ck.GATE_SCALAR), max(3, a.steps // 3))
        del sg, bws
        dp = {k: (None if v is None else v.to(dev)) for k, v in gen.make_dp2_inputs(w, gated=False).items()}
        dws = torch.empty(ck.workspace_size(w.B, w.H, 2 * w.T, w.dk, w.dv, w.chunk, ck.DTYPE_BF16), dtype=torch.uint8,
                          device=dev)
        dp2_ms = timed(lambda: ck.deltaproduct2_fwd(dp["q"], dp["k"], dp["v"], dp["beta"], h0=dp["h0"], chunk=w.chunk,
                                                    workspace=dws, o=o, hT=hT), a.steps)
        del dws
        dws = torch.empty(int(ck.lib().ckda_deltaproduct2_bwd_workspace_size(w.B, w.H, w.T, w.dk, w.dv, ck.DTYPE_BF16)),
                          dtype=torch.uint8, device=dev)
        dp2_bwd_ms = timed(lambda: ck.deltaproduct2_bwd(dp["q"], dp["k"], dp["v"], None, dp["beta"], bdo, h0=dp["h0"],
                                                        dhT=bdhT, workspace=dws), max(3, a.steps // 3))
        del dp, dws
        dd = [{k: v.to(dev) for k, v in gen.dp2_decode_inputs(s, dec, gated=False).items() if v is not None}
              for s in range(4)]
        cnt = [0]

        def dp2_dec():
            x = dd[cnt[0] % 4]
            cnt[0] += 1
            ck.deltaproduct2_decode_step(x["q"], x["k"], x["v"], x["beta"], S, o=do)

        dp2_dec_ms = timed(dp2_dec, a.decode_steps)
        return {
            "backward": {
                "workload": w.name,
                "call_ms_mean": round(bwd_ms, 4),
                "tokens_per_s": round(tokens / (bwd_ms * 1e-3), 1),
                "forward_plus_backward_tokens_per_s": round(tokens / ((bwd_ms + call_ms) * 1e-3), 1),
                "gradients": "fp32 dq, dk, dv, dalpha, dbeta, dh0",
                "fused_prologue_call_ms_mean": round(bwdx_ms, 4),
                "fused_prologue_gradients": "with respect to the gate and beta logits and the raw keys "
                                            "(CKDA_FUSE_GATES | CKDA_FUSE_NORM_K)",
            },
            "comparators": {
                "scalar_gate_forward_call_ms_mean": round(scalar_ms, 4),
                "scalar_gate_tokens_per_s": round(tokens / (scalar_ms * 1e-3), 1),
                "scalar_gate_backward_call_ms_mean": round(scalar_bwd_ms, 4),
                "scalar_gate_forward_plus_backward_tokens_per_s": round(tokens / ((scalar_ms + scalar_bwd_ms) * 1e-3), 1),
                "deltaproduct2_forward_call_ms_mean": round(dp2_ms, 4),
                "deltaproduct2_tokens_per_s": round(tokens / (dp2_ms * 1e-3), 1),
                "deltaproduct2_backward_call_ms_mean": round(dp2_bwd_ms, 4),
                "deltaproduct2_forward_plus_backward_tokens_per_s": round(tokens / ((dp2_ms + dp2_bwd_ms) * 1e-3), 1),
                "deltaproduct2_decode_ms_per_step": round(dp2_dec_ms, 4),
                "deltaproduct2_decode_total_GB_s": round(
                    (state_bytes + dec.N * dec.H * (3 * dec.dk + 3 * dec.dv + 2) * 2) / (dp2_dec_ms * 1e-3) / 1e9, 1),
            },
            "kda": {
                "workload": kw.name,
                "forward_call_ms_mean": round(kda_ms, 4),
                "forward_tokens_per_s": round(kw.B * kw.T / (kda_ms * 1e-3), 1),
                "algorithmic_GB_s": round(kda_bytes / (kda_ms * 1e-3) / 1e9, 1),
            },
            "channel_gather": {
                "workload": f"{gw.name} (d_k {gw.dk} kept of {dk_in})",
                "forward_call_ms_mean": round(gather_ms, 4),
                "forward_tokens_per_s": round(gw.B * gw.T / (gather_ms * 1e-3), 1),
                "pregathered_plain_call_ms_mean": round(pregathered_ms, 4),
                "gather_overhead_vs_pregathered": round(gather_ms / pregathered_ms - 1.0, 4),
            },
            "fused_prologue": {
                "flags": "CKDA_FUSE_GATES | CKDA_FUSE_NORM_K",
                "inputs": "gate and beta logits, unnormalised keys (same shapes)",
                "forward_call_ms_mean": round(fused_ms, 4),
                "forward_tokens_per_s": round(tokens / (fused_ms * 1e-3), 1),
                "forward_overhead_vs_plain": round(fused_ms / call_ms - 1.0, 4),
                "decode_ms_per_step_events": round(fdec_ms, 4),
                "decode_total_GB_s": round((state_bytes + io_bytes) / (fdec_ms * 1e-3) / 1e9, 1),
            },
        }

    sections = {} if a.skip_extras else extras()

    # ---- reference device copy of the decode state's size (practical ceiling)
    src = torch.empty(dec.N * dec.H * dec.dk * dec.dv, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    ce1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 / (ce0.elapsed_time(ce1) / 10 * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "dk": w.dk, "dv": w.dv,
                   "chunk": w.chunk, "gates": w.gates, "h0": w.h0},
        "roofline": {
            "bound": "hbm",
            "kernel": dominant,
            "achieved": round(dom_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(dominant),
            "algorithmic_bytes": kbytes[dominant],
            "kernel_us_mean": round(kern_ms[dominant] * 1e3, 2),
            "kernels": {k: {"us_mean": round(kern_ms[k] * 1e3, 2), "algorithmic_bytes": kbytes[k],
                            "algorithmic_GB_s": round(kbytes[k] / (kern_ms[k] * 1e-3) / 1e9, 1),
                            "record_bytes": record_bytes,
                            "traffic": traffic_from_profile(k)} for k in kern_ms},
            "mfma_executed_busy_frac": counters_from_profile("chunk_fwd_ckda_bf16_mfma_counters",
                                                             ["chunk_gram_kernel", "chunk_state_kernel"]),
            "forward": {"call_ms_mean": round(call_ms, 4), "call_ms_median": round(call_ms_median, 4),
                        "protocol_ms_median_of_3x100": None if proto_ms is None else round(proto_ms, 4),
                        "protocol_trial_medians_ms": [round(x, 4) for x in proto_trials],
                        "graph_replay_ms_mean": round(graph_ms, 4),
                        "algorithmic_bytes": nbytes, "algorithmic_GB_s": round(achieved_gbs, 1),
                        "frac_of_hbm_peak": round(achieved_gbs / HBM_PEAK_GBS, 4),
                        "mfma_algorithmic_tflops": round(achieved_tflops, 2),
                        "mfma_frac_of_bf16_peak": round(achieved_tflops / BF16_PEAK_TFLOPS, 4)},
        },
        "decode": {
            "workload": dec.name, "steps": a.decode_steps,
            "ms_per_step_events": round(dec_ms, 4),
            "protocol_ms_median_of_3x100": None if dec_proto_ms is None else round(dec_proto_ms, 4),
            "ms_per_step_wall": round(dwall * 1e3 / a.decode_steps, 4),
            "state_GB_s": round(dec_gbs_state, 1),
            "total_GB_s": round(dec_gbs_total, 1),
            "frac_of_hbm_peak": round(dec_gbs_total / HBM_PEAK_GBS, 4),
            "device_copy_GB_s": round(copy_gbs, 1),
        },
    }

    out.update(sections)
    if not a.no_cpu_baseline:
        import oracle
        from gated_delta_rule_ckda_amd.inputs import raw
        args = [raw(inp[n]) for n in ("q", "k", "v", "alpha", "beta")]
        h0 = None if inp["h0"] is None else raw(inp["h0"])
        nt = oracle.num_threads()
        log(f"[bench] oracle cpu baseline: whole workload passes for ~{a.cpu_seconds:.0f} s, {nt} threads")
        c0 = time.perf_counter()
        oracle.fwd(*args, h0=h0)
        passes = 1
        first = time.perf_counter() - c0
        more = max(0, int(a.cpu_seconds / max(first, 1e-3)) - 1)
        for _ in range(more):
            oracle.fwd(*args, h0=h0)
        passes += more
        csec = time.perf_counter() - c0
        # one thread on one (batch, head), extrapolated to the B*H heads; the
        # sampled heads' results also check the GPU output measured above
        one = [raw(sel(inp[n])[:1]) for n in ("q", "k", "v", "alpha", "beta")]
        h01 = None if inp["h0"] is None else raw(sel(inp["h0"])[:1])
        c1 = time.perf_counter()
        oracle.fwd(*one, h0=h01, nthreads=1)
        one_s = time.perf_counter() - c1
        ro, rh = oracle.fwd(*[raw(sel(inp[n])) for n in ("q", "k", "v", "alpha", "beta")],
                            h0=None if inp["h0"] is None else raw(sel(inp["h0"])))

        def rel(x, y):
            x = np.asarray(x, np.float64).reshape(x.shape[0], -1)
            y = np.asarray(y, np.float64).reshape(y.shape[0], -1)
            return float(np.max(np.max(np.abs(x - y), 1) / np.maximum(np.max(np.abs(y), 1), 1e-300)))

        S_ref = dec_sample[0].copy()
        d_ref = oracle.decode(*[raw(dec_sample[1][n]) for n in ("q", "k", "v", "alpha", "beta")], S_ref)
        parity = {"metric": "per sampled head: max|gpu - oracle| / max|oracle|, the maximum over the heads",
                  "forward": {"workload": w.name, "heads": heads, "o_rel_err": rel(gpu_sample[0], ro),
                              "hT_rel_err": rel(gpu_sample[1], rh),
                              "tolerance": 2e-2 if w.dtype == "bf16" else 1e-4},
                  "decode": {"workload": dec.name, "states": ds_idx, "steps": 1,
                             "o_rel_err": rel(dec_sample[2], d_ref), "state_rel_err": rel(dec_sample[3], S_ref),
                             "tolerance": 2e-2}}
        out["cpu_baseline"] = {"value": round(passes * w.B * w.T / csec, 1), "unit": "tokens/s", "cores": nt,
                               "kind": "oracle",
                               "sample": f"the whole {w.name} forward ({w.B * w.H} heads x {w.T} positions) "
                                         f"{passes} times, {csec:.1f} s",
                               "cpu_model": cpu_model(), "nproc": os.cpu_count(),
                               "one_thread": {"seconds_one_head": round(one_s, 4),
                                              "extrapolated_tokens_per_s": round(w.B * w.T / (one_s * w.B * w.H), 1),
                                              "sample": f"one head x {w.T} positions, 1 thread, "
                                                        f"extrapolated x{w.B * w.H} heads"},
                               "parity_of_this_run": parity}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
