"""Host AddressSanitizer / UndefinedBehaviorSanitizer run of the C ABI's
argument validation: locks_capi.hip is rebuilt with the sanitizers on its
host code only and linked, with the library's other objects, into
tests/capi_sanitize/driver.cpp, which calls every entry point with arguments
its validation must reject before anything is enqueued (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "kv_cache_page_amd")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host",
            "-fno-omit-frame-pointer"]


def test_capi_validation_under_host_sanitizers(tmp_path):
    from kv_cache_page_amd import build_lib
    hipcc = build_lib.HIPCC
    if not os.path.exists(hipcc) and not shutil.which(hipcc):
        pytest.skip("hipcc not available")
    objdir = build_lib.BUILD_DIR
    others = [os.path.join(objdir, f) for f in sorted(os.listdir(objdir))
              if f.endswith(".o") and f != "locks_capi.o"] if os.path.isdir(objdir) else []
    if len(others) != len(build_lib.sources()) - 1:
        pytest.skip("library objects not built (run the build first)")
    capi = os.path.join(str(tmp_path), "locks_capi_san.o")
    cmd = [hipcc, *build_lib.FLAGS, *HOST_SAN, "-c", os.path.join(build_lib.CSRC, "locks_capi.hip"),
           "-o", capi]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    drv = os.path.join(str(tmp_path), "driver.o")
    cmd = [hipcc, f"--offload-arch={build_lib.ARCH}", "-O1", "-std=c++17", *HOST_SAN,
           "-I", build_lib.INCLUDE, "-c", os.path.join(ROOT, "tests", "capi_sanitize", "driver.cpp"),
           "-o", drv]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    exe = os.path.join(str(tmp_path), "capi_driver")
    cmd = [hipcc, f"--offload-arch={build_lib.ARCH}", *HOST_SAN, drv, capi, *others, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert "all checks passed" in r.stdout
