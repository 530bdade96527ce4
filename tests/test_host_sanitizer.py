"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two drivers are built with the sanitizers and run:
* tests/sanitize/oracle_driver.c with oracle/ckda_oracle.c (gcc): every oracle
  entry point on small inputs in every dtype, with and without the optional
  arguments, and on rejected arguments; leak checking on.
* tests/sanitize/api_driver.cpp with the library's sources (hipcc; the
  sanitizers apply to host code only, device code is built as usual): every
  C ABI entry point through its argument checks and, with no GPU visible,
  through the host side of its launches, which then fail for want of a
  device.  Its fake device addresses are never dereferenced on the host.
Any sanitizer finding aborts the driver; the test needs exit status 0."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_delta_rule_ckda_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, out = run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
                   "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
                   os.path.join(ROOT, "oracle", "ckda_oracle.c"), os.path.join(ROOT, "tests", "sanitize",
                                                                                 "oracle_driver.c"),
                   "-o", exe, "-lm"])
    if rc != 0 and "asan" in out.lower():
        pytest.skip("no sanitizer runtime for gcc here: " + out[-300:])
    assert rc == 0, out
    rc, out = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1"))
    assert rc == 0 and "0 failures" in out, out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_c_abi_host_code_under_asan_ubsan(tmp_path):
    srcs = ["ckda_api.cpp", "decode.hip", "chunk_gram.hip", "chunk_state.hip", "chunk_bwd.hip", "prologue_bwd.hip",
            "dp2_bwd.hip", "noalloc.hip"]
    base = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", *SAN_HOST,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]

    def compile_one(src):
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        return run(base + ["-c", path, "-o", obj]), obj

    allsrc = srcs + [os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp")]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, allsrc))
    for (rc, out), _ in results:
        assert rc == 0, out[-2000:]
    exe = str(tmp_path / "api_driver")
    rc, out = run([HIPCC, "--offload-arch=gfx950", *SAN_HOST[:4], *[o for _, o in results], "-o", exe])
    assert rc == 0, out[-2000:]
    # the HIP runtime's own allocations are not the library's: no leak check
    rc, out = run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1"))
    assert rc == 0 and "0 failures" in out, out[-3000:]
