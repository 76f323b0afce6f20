"""The host planner under AddressSanitizer (with libstdc++'s container
annotations, so a read or write past a reused vector's size is caught even
inside its capacity) and UndefinedBehaviorSanitizer: 20000 random batches
(head counts, group sizes, page sizes, windows, non-causal, explicit decode
splits, compute-unit counts, host-only size queries) planned on one thread.
Host code only; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_fuzz_under_sanitizers(tmp_path):
    exe = tmp_path / "planner_fuzz"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-D_GLIBCXX_SANITIZE_VECTOR", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "paged_chunked_prefill_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "planner_fuzz.cpp"),
           os.path.join(ROOT, "paged_chunked_prefill_amd", "csrc", "planner.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # (verify_asan_link_order=0: the sanitizer runtime need not come first when
    # the environment preloads another library)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-3000:]
    ok, items = r.stdout.split()[1], r.stdout.split()[3]
    assert int(ok) > 15000 and int(items) > 0, r.stdout
