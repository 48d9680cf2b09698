"""The CPU oracle under host sanitizers: tests/native/oracle_stress.cpp drives
oracle_store_kvcache, oracle_decode and oracle_prefill with random small cases
(padding rows, -1 slots, ragged lengths, row subsets, 1-3 threads, rejected
metadata) and checks thread-count independence, untouched rows and the
convex-combination bound of every output. Built twice with the host compiler
only: AddressSanitizer + UndefinedBehaviorSanitizer, and ThreadSanitizer (the
oracle's worker threads)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = [os.path.join(ROOT, "oracle", "oracle.cpp"),
           os.path.join(ROOT, "tests", "native", "oracle_stress.cpp")]


def _build_and_run(tmp_path, name, flags, cases, env_extra):
    exe = tmp_path / name
    cmd = ["g++", "-O1", "-g", "-std=c++17", "-pthread", "-fno-omit-frame-pointer", *flags,
           *SOURCES, "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, **env_extra)
    r = subprocess.run([str(exe), str(cases), "2024"], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert f"ok after {cases} cases" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "oracle_asan",
                   ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                    "-static-libasan"], 400, {"ASAN_OPTIONS": "detect_leaks=1"})


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_tsan(tmp_path):
    _build_and_run(tmp_path, "oracle_tsan", ["-fsanitize=thread"], 150,
                   {"TSAN_OPTIONS": "halt_on_error=1"})
