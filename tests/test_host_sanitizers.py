"""The C-ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

api.hip -- argument checks, capacity, workspace carve-up, the entry points -- is compiled
for the host alone with both sanitizers and linked with the library's own objects into
tests/sanitize/abi_driver.cpp, which calls every host-only path and every reject case
(fake device addresses, never dereferenced).  The run must end cleanly; two planted
mistakes in the driver itself (a heap overflow, a signed overflow) show that the build
is instrumented.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "sparse_mixture_experts_switchffn_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Host-side sanitizers only: each flag goes to the host compilation.
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=ENV)
    return r.returncode, r.stdout


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    objs = [os.path.join(PKG, "_build", f + ".o") for f in ("router", "dispatch", "ffn", "bwd")]
    if not all(os.path.exists(o) for o in objs):
        from sparse_mixture_experts_switchffn_amd.build import build
        build()
    out = tmp_path_factory.mktemp("san")
    api = str(out / "api_san.o")
    drv = str(out / "drv.o")
    exe = str(out / "abi_driver")
    common = ["--offload-host-only", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer", *SAN]
    for src, obj in ((os.path.join(PKG, "csrc", "api.hip"), api),
                     (os.path.join(HERE, "sanitize", "abi_driver.cpp"), drv)):
        rc, log = _run([HIPCC, *common, "-c", src, "-o", obj])
        assert rc == 0, log[-3000:]
    rc, log = _run([HIPCC, *SAN, drv, api, *objs, "-o", exe])
    assert rc == 0, log[-3000:]
    return exe


def test_entry_points_clean_under_asan_and_ubsan(driver):
    rc, log = _run([driver])
    assert rc == 0, log[-4000:]
    assert "runtime error" not in log and "AddressSanitizer" not in log, log[-4000:]
    assert "all host-side cases passed" in log


def test_build_is_instrumented(driver):
    rc, log = _run([driver, "asan_probe"])
    assert rc != 0 and "heap-buffer-overflow" in log, log[-2000:]
    rc, log = _run([driver, "ubsan_probe"])
    assert rc != 0 and "runtime error" in log, log[-2000:]
