"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.hip (argument checks, size arithmetic, dispatch and error reporting) is
built a second time with both sanitizers on its host pass, linked with the
ordinary kernel objects into _build/san/libfa_san.so, and tests/test_abi.py
runs against that library in a child process that preloads the compiler's
sanitizer runtime.  Any sanitizer report aborts the child (recovery is off),
so a clean pass means every validation path test_abi.py drives stayed in
bounds and free of undefined behaviour.  CPU only: no test here launches a
kernel.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _child_env(lib, runtime):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = runtime + (":" + pre if pre else "")
    # the Python interpreter itself is not instrumented and keeps memory to exit
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["FA_LIBRARY"] = lib
    return env


@pytest.fixture(scope="module")
def sanitized():
    from tiled_online_softmax_04_amd import build
    if not os.path.exists(build.HIPCC):
        pytest.skip("hipcc is not installed")
    return build.build_sanitized(), build.sanitizer_runtime()


def test_sanitized_library_is_instrumented(sanitized):
    lib, _ = sanitized
    out = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    names = [line.split()[-1] for line in out.splitlines() if line.strip()]
    assert any(n.startswith("__asan_report_") for n in names)
    assert any(n.startswith("__ubsan_handle_") for n in names)


def test_child_loads_the_sanitized_library(sanitized):
    lib, runtime = sanitized
    code = ("from tiled_online_softmax_04_amd import fa\n"
            "fa.load_library()\n"
            "maps = open('/proc/self/maps').read()\n"
            "print('SAN_LIB' if fa.LIB_PATH in maps else 'NO_SAN_LIB')\n"
            "print('SAN_RT' if 'libclang_rt.asan' in maps else 'NO_SAN_RT')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_child_env(lib, runtime),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "SAN_LIB" in r.stdout.split() and "SAN_RT" in r.stdout.split(), r.stdout


def test_abi_suite_passes_under_sanitizers(sanitized):
    lib, runtime = sanitized
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"),
                        "-q", "-x", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=_child_env(lib, runtime), capture_output=True, text=True,
                       timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    assert "runtime error" not in text and "AddressSanitizer" not in text, text[-4000:]
    assert " passed" in r.stdout
