"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU call): libdcp is rebuilt with host-side instrumentation
(device code unchanged) and the host ABI checks of test_abi_host.py run
against it in a child process with the ASan runtime preloaded. An overflow,
use after free or undefined behaviour in argument validation, the workspace
size queries or descriptor handling aborts the child and fails this test."""

import glob
import os
import subprocess
import sys

import pytest

from sequence_sharded_paged_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.fixture(scope="module")
def sanitized_lib():
    if not os.path.exists(build.HIPCC) or not ASAN_RT:
        pytest.skip("hipcc or the ASan runtime is not installed")
    return build.build(sanitize=True)


def _env(lib):
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = ASAN_RT[-1] + (":" + pre if pre else "")  # the ASan runtime must come first
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"  # the interpreter itself frees little at exit
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["DCP_LIB"] = lib
    return env


def test_child_loads_the_instrumented_library(sanitized_lib):
    code = ("from sequence_sharded_paged_amd import native; native.lib(); "
            "maps = open('/proc/self/maps').read(); "
            f"assert {sanitized_lib!r} in maps, 'sanitized libdcp not mapped'; "
            "assert 'libclang_rt.asan' in maps, 'ASan runtime not mapped'; print('ok')")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(sanitized_lib), capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr


def test_host_abi_checks_under_sanitizers(sanitized_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join("tests", "test_abi_host.py")],
                       cwd=ROOT, env=_env(sanitized_lib), capture_output=True, text=True, timeout=600)
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
