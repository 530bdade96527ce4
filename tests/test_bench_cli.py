"""Host-side checks of bench.py: the one-GPU guard and the algorithmic byte
and flop counts it reports (no GPU needed)."""
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_algorithmic_counts_of_the_bench_workload():
    from gated_delta_rule_ckda_amd import inputs as gen
    b = _bench_module()
    w = gen.WORKLOADS["ckda_bf16"]
    nbytes, flops = b.fwd_algorithmic(w)
    th = 4 * 16 * 4096
    # q, k, alpha, v read and o written in bf16, beta, plus h0 read and hT written in fp32
    assert nbytes == th * (3 * 128 + 2 * 128 + 1) * 2 + 2 * 4 * 16 * 128 * 128 * 4 == 344_457_216
    assert flops == th * (6 * 128 * 128 + 3 * 64 * 128 + 2 * 64 * 128)
    k = b.kernel_algorithmic(w)
    assert k["chunk_gram_kernel"] + k["chunk_state_kernel"] == nbytes
    # the KDA workload starts from a zero state: only hT is written
    kw = gen.WORKLOADS["kda_bf16"]
    kb, _ = b.fwd_algorithmic(kw)
    assert kb == 4 * 16 * 2048 * (3 * 128 + 2 * 128 + 1) * 2 + 4 * 16 * 128 * 128 * 4


def test_counter_summaries_go_stale_with_any_device_source(tmp_path):
    """The bench reports a committed counter figure only while the kernel's
    source and the device headers it includes are those the counters were
    taken from: a change to a header makes the figure null."""
    import shutil
    b = _bench_module()
    csrc = tmp_path / "gated_delta_rule_ckda_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    for f in ("chunk_gram.hip", "chunk_state.hip", "chunk_common.hpp", "ckda_device.hpp"):
        shutil.copy(os.path.join(ROOT, "gated_delta_rule_ckda_amd", "csrc", f), csrc / f)
    for k in ("chunk_gram_kernel", "chunk_state_kernel"):
        shutil.copy(os.path.join(ROOT, "profiles", f"{k}_ckda_bf16_hbm_counters.md"), tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "profiles", "chunk_fwd_ckda_bf16_mfma_counters.md"), tmp_path / "profiles")
    b.ROOT = str(tmp_path)
    fresh = {k: b.traffic_from_profile(k) for k in ("chunk_gram_kernel", "chunk_state_kernel")}
    mfma = b.counters_from_profile("chunk_fwd_ckda_bf16_mfma_counters", ["chunk_gram_kernel", "chunk_state_kernel"])
    if None in fresh.values() or mfma is None:
        import pytest
        pytest.skip("the committed counter summaries belong to other kernel sources")
    assert all(isinstance(v, int) and v > 0 for v in fresh.values())
    with open(csrc / "ckda_device.hpp", "a") as fh:
        fh.write("\n// changed\n")
    assert b.traffic_from_profile("chunk_gram_kernel") is None
    assert b.traffic_from_profile("chunk_state_kernel") is None
    assert b.counters_from_profile("chunk_fwd_ckda_bf16_mfma_counters", ["chunk_gram_kernel"]) is None
