"""The library's host C++ under the address and undefined-behaviour
sanitizers, on the CPU: tests/native/host_checks.cpp drives the checks of
device-resident arguments (check.hpp: every kind of bad offset, length and
page id, and that nothing outside a sequence's pages is read), the page pool
and capacity planner (pool.cpp) and the C ABI's host validation (api.hip) on
a layer handle with stand-in device pointers.  The host parts (api.hip,
check.hip, pool.cpp, the driver) are compiled with -fsanitize=address and
-fsanitize=undefined for the host only and linked with the library's other
objects; a sanitizer report, a leak or a failed expectation fails the test.
No GPU is touched: every GPU call the driver makes is refused by a host check."""
import importlib.util
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
SAN = os.path.join(BUILD, "san")
CSRC = os.path.join(ROOT, "mla_compressed_latent_amd", "csrc")
SANITIZED = ("api.hip", "check.hip", "pool.cpp")


def _build_module():
    spec = importlib.util.spec_from_file_location("mla_build", os.path.join(ROOT, "mla_compressed_latent_amd",
                                                                            "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _flags(b):
    return ["-x", "hip", f"--offload-arch={b.ARCH}", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stderr[-4000:]}"


@pytest.fixture(scope="module")
def host_checks():
    b = _build_module()
    others = [s for s in b.SOURCES if s not in SANITIZED]
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in others]
    if not all(os.path.exists(o) for o in objs):
        b.build()
    os.makedirs(SAN, exist_ok=True)
    hipcc = b.hipcc()
    san_objs = []
    for src in [os.path.join(CSRC, s) for s in SANITIZED] + [os.path.join(ROOT, "tests", "native",
                                                                         "host_checks.cpp")]:
        obj = os.path.join(SAN, os.path.splitext(os.path.basename(src))[0] + ".o")
        _run([hipcc, *_flags(b), "-c", src, "-o", obj])
        san_objs.append(obj)
    exe = os.path.join(SAN, "host_checks")
    _run([hipcc, f"--offload-arch={b.ARCH}", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
          "-fsanitize=undefined", *san_objs, *objs, "-o", exe])
    return exe


def test_host_code_under_sanitizers(host_checks):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([host_checks], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout, r.stderr[-3000:])
    assert r.returncode == 0, r.stderr[-3000:]
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    held, total = (int(w) for w in r.stdout.split("host checks: ")[1].split()[0:3:2])
    assert held == total and total >= 90
