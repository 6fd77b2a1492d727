"""CPU tests of the host gradient-add team that host_grad_accumulate pools
use (csrc/host_add.cpp): built with g++ together with
tests/host_add_check.cpp, which stands in for the HIP event wait and drives
the team as the pool's writeback does (two staging areas used alternately,
each refilled only after its last add job has finished).  The tier must end
bit-identical to a serial, in-order reference; a ThreadSanitizer build must
report no data race."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_cache_chunk_amd", "csrc")
ROCM_INC = "/opt/rocm/include"


def _build(tmp_path, extra, name):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INC):
        pytest.skip("g++ or the ROCm headers are missing")
    exe = str(tmp_path / name)
    cmd = [gxx, "-std=c++17", "-g", "-pthread", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC,
           "-I", CSRC, *extra, os.path.join(HERE, "host_add_check.cpp"),
           os.path.join(CSRC, "host_add.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, threads, jobs, bf16, seed):
    r = subprocess.run([exe, str(threads), str(jobs), str(bf16), str(seed)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert r.stdout.split() == ["ok", str(jobs), str(jobs)], r.stdout
    return r


@pytest.mark.parametrize("threads,bf16,seed", [(1, 1, 0), (2, 0, 1), (8, 1, 2), (16, 1, 3), (5, 0, 4)])
def test_host_adds_match_serial_reference(tmp_path, threads, bf16, seed):
    exe = _build(tmp_path, ["-O2"], "check")
    _run(exe, threads, 300, bf16, seed)


def test_host_adds_thread_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    probe = subprocess.run([gxx or "g++", "-fsanitize=thread", "-x", "c++", "-", "-o",
                            str(tmp_path / "probe")], input="int main(){return 0;}",
                           capture_output=True, text=True)
    if probe.returncode != 0:
        pytest.skip("no ThreadSanitizer runtime")
    exe = _build(tmp_path, ["-O1", "-fsanitize=thread"], "check_tsan")
    r = _run(exe, 8, 120, 1, 7)
    assert "ThreadSanitizer" not in r.stderr, r.stderr
