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
