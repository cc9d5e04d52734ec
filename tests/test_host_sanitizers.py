"""libkvc's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The entry points (api.hip compiled for the host only), the block pool
(pool.cpp) and the budget schedules (schedule.cpp) are linked with stand-ins
for the kernel launchers and the few HIP runtime calls (tests/host_asan/
stubs.cpp) into a driver (tests/host_asan/driver.cpp) that calls every entry
point with valid and invalid arguments and runs the pool against a plain
model. No GPU and no device memory are involved; the sanitizers are on host
code only.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_kv_cache_kvc_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_asan")
HIPCC = "/opt/rocm/bin/hipcc"
SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _host_flags():
    flags = []
    for f in SAN:
        flags += ["-Xarch_host", f]
    return flags


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    out = tmp_path_factory.mktemp("host_asan")
    inc = [f"-I{ROOT}/include", f"-I{CSRC}"]

    def run(cmd):
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout + r.stderr
        return r

    hip_host = [HIPCC, "--cuda-host-only", "-O1", "-g", "-std=c++17", "-fPIC", *inc, *_host_flags()]
    api = str(out / "api.o")
    run([*hip_host, "-c", os.path.join(CSRC, "api.hip"), "-o", api])
    fatbin = re.findall(r"\b(__hip_fatbin_\w+)", run(["nm", "-u", api]).stdout)
    stub_def = [f"-DKVC_FATBIN_SYMBOL={fatbin[0]}"] if fatbin else []
    stubs = str(out / "stubs.o")
    run([*hip_host, *stub_def, "-c", os.path.join(HERE, "stubs.cpp"), "-x", "hip", "-o", stubs])
    objs = [api, stubs]
    for src in ("pool.cpp", "schedule.cpp"):
        o = str(out / (src + ".o"))
        run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", *inc, *SAN, "-c", os.path.join(CSRC, src), "-o", o])
        objs.append(o)
    drv = str(out / "driver.o")
    run(["g++", "-O1", "-g", "-std=c++17", *inc, *SAN, "-c", os.path.join(HERE, "driver.cpp"), "-o", drv])
    exe = str(out / "host_checks")
    run(["g++", *SAN, "-o", exe, drv, *objs, "-lpthread"])
    return exe


def test_host_code_is_sanitizer_clean(driver):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([driver], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
