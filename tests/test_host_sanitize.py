"""The library's host logic (lora_host.cpp: validation, the metadata builder and
the tile plan) built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer
and driven by tests/host_sanitize.cpp: random pools and batches (up to 70 000
rows and 5 000 slots, bad ids, ranked plans), every output buffer of exactly the
documented size.  CPU only; no HIP code is compiled."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_host_logic_under_asan_ubsan():
    tmp = tempfile.mkdtemp(prefix="lora_host_asan_")
    try:
        exe = os.path.join(tmp, "host_sanitize")
        cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
               "-I" + os.path.join(ROOT, "include"),
               "-I" + os.path.join(ROOT, "lora_adapter_pool_amd", "csrc"),
               os.path.join(ROOT, "lora_adapter_pool_amd", "csrc", "lora_host.cpp"),
               os.path.join(HERE, "host_sanitize.cpp"), "-o", exe]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stdout
        # a library preloaded by the environment may precede the ASan runtime
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe, "1500"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                           text=True, timeout=300, env=env)
        print(r.stdout)
        assert r.returncode == 0, r.stdout
        assert "0 failed checks" in r.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
