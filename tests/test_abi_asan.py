"""CPU: the C ABI's host-side logic under AddressSanitizer.  Every library
source is compiled with the host pass instrumented (the gfx950 device code is
built as usual) and linked with tests/abi_asan_check.c, which calls every
entry point with null or malformed arguments and creates and destroys real
pools (without a GPU the allocations fail, which exercises the release of a
half-built pool).  The run must report the documented statuses and no ASan
error or leak in the library (leaks of the HIP runtime itself are
suppressed)."""
import concurrent.futures
import glob
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "paged_kv_cache_chunk_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def test_abi_host_logic_under_asan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc is missing")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Wno-unused-result", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        r = subprocess.run([HIPCC, *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with concurrent.futures.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = str(tmp_path / "abi_asan_check.o")
    r = subprocess.run([HIPCC, "-x", "c", "-O1", "-g", "-Xarch_host", "-fsanitize=address",
                        "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                        "-c", os.path.join(HERE, "abi_asan_check.c"), "-o", drv],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    exe = str(tmp_path / "abi_asan_check")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        *objs, drv, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    supp = tmp_path / "lsan.supp"
    supp.write_text("leak:libamdhip64\nleak:libhsa-runtime64\nleak:libdrm\n")
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               LSAN_OPTIONS=f"suppressions={supp}")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-5000:]
    assert "ERROR: LeakSanitizer" not in r.stderr, r.stderr[-5000:]
    assert r.returncode == 0, (r.stdout, r.stderr[-3000:])
    assert r.stdout.startswith("ok "), r.stdout
