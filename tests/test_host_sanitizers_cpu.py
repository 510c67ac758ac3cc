"""The library's host code (request validation, launch planning) under
AddressSanitizer and UndefinedBehaviorSanitizer: every source is compiled
with the sanitizers on its host side only, into a fuzz driver (host_fuzz.cpp)
that feeds s1_validate and s1k_attention_plan random requests honouring the
calling contract.  No GPU is needed and no kernel is launched."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "prefill_only_decision_amd", "csrc")
SOURCES = ["abi.cpp", "executor.cpp", "gemm.hip", "attention.hip", "scan.hip", "misc.hip", "vocab.hip", "gdn.hip",
           "peak.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def fuzz_binary(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is not installed")
    from concurrent.futures import ThreadPoolExecutor
    out = tmp_path_factory.mktemp("san")
    exe = str(out / "host_fuzz")
    # sanitizers on the host side of each compilation only (-Xarch_host);
    # the device code is compiled as for the library
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]

    def compile_one(path):
        obj = str(out / (os.path.basename(path) + ".o"))
        cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++20", "-Xclang", "-target-feature",
               "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", *san, "-c", path, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    paths = [os.path.join(CSRC, x) for x in SOURCES] + [os.path.join(HERE, "host_fuzz.cpp")]
    with ThreadPoolExecutor(min(len(paths), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(compile_one, paths))
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", "-o", exe, *objs], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_validation_and_planning_under_sanitizers(fuzz_binary):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([fuzz_binary, "20000", "7"], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    ok, inval, budget = (int(x) for x in r.stdout.split()[1:4])
    # the fuzz reaches every outcome
    assert ok > 100 and inval > 100 and budget > 100, r.stdout
