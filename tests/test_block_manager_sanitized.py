"""The C++ block manager under host AddressSanitizer and UndefinedBehaviorSanitizer:
tests/native/bm_stress.cpp drives every entry point with random calls (failures
included) and checks reference counts, free counts and metadata padding after
each one. Built with the host compiler only; no GPU code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_block_manager_under_asan_ubsan(tmp_path):
    exe = tmp_path / "bm_stress"
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-static-libasan",
           f"-I{ROOT}/include",
           os.path.join(ROOT, "paged_kv_cache_slot_amd", "csrc", "block_manager.cpp"),
           os.path.join(ROOT, "tests", "native", "bm_stress.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    r = subprocess.run([str(exe), "20000"], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok after 20000 steps" in r.stdout
    assert "taken_back 0" not in r.stdout and "evicted 0" not in r.stdout
