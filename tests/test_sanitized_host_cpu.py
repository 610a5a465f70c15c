"""The host runtime (table build, layout, host image, export, fill, carry, write-back
bookkeeping, argument checks) under AddressSanitizer and UndefinedBehaviorSanitizer.

The host file is built with g++ and both sanitizers into a separate library
(ad_recommendation_amd.build.build_sanitized); the CPU tests of the C ABI, the PASS lifecycle,
the FTRL state and the device-build sizing then run against it in a child process started with
the ASan runtime preloaded (MI355EMB_LIB selects the library).  Any sanitizer report aborts the
child, so the test fails on the first invalid access or undefined operation.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUITES = ["tests/test_boundary_cpu.py", "tests/test_pass_lifecycle_cpu.py",
          "tests/test_ftrl_cpu.py", "tests/test_device_build_cpu.py"]


def _runtime(name):
    r = subprocess.run(["g++", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_runtime_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    sys.path.insert(0, ROOT)
    from ad_recommendation_amd import build as B
    lib = B.build_sanitized()
    env = dict(os.environ, MI355EMB_LIB=lib, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # the child first shows that the sanitized library is the one mapped, then runs the suites
    code = ("import sys; sys.path.insert(0, %r); from ad_recommendation_amd import emb; emb.lib(); "
            "maps = open('/proc/self/maps').read(); assert %r in maps, 'sanitized library not loaded'; "
            "import pytest; sys.exit(pytest.main(['-q', '-x', '-m', 'not gpu', '-p', 'no:cacheprovider'] + %r))"
            % (ROOT, os.path.basename(lib), SUITES))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=900)
    tail = "\n".join(r.stdout.splitlines()[-30:])
    assert r.returncode == 0, f"sanitized host run failed ({r.returncode}):\n{tail}"
    assert " passed" in tail
