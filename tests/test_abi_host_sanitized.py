"""The host-side checks of the C-ABI library (tests/test_abi_host.py) again, against a build whose
host code carries AddressSanitizer and UndefinedBehaviorSanitizer: every source is compiled with
the sanitizers on the host pass only (the gfx950 device code is built as usual), the library is
linked into a temporary folder, and the host tests run in a child process with the sanitizer
runtime preloaded.  A heap overflow, use-after-free or undefined operation (signed overflow, bad
shift, misaligned access) in the configuration checks, the size and layout planning or the
argument validation ends that process with a report, and the test fails.  No GPU is touched: the
host tests stop before any device call."""
import os
import subprocess
import sys

import pytest

from hierarchical_global_local_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ASAN_RT = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.slow


def _sanitized_library(folder):
    objs = []
    for s in B.SOURCES:
        o = os.path.join(folder, s + ".o")
        B._run([B.HIPCC, *B.FLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, s), "-o", o])
        objs.append(o)
    lib = os.path.join(folder, "libbt_host_sanitized.so")
    B._run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_SAN, *objs, "-o", lib])
    return lib


@pytest.mark.skipif(not (os.path.exists(B.HIPCC) and os.path.exists(ASAN_RT)),
                    reason="hipcc or the clang AddressSanitizer runtime is not installed")
def test_host_tests_under_address_and_undefined_sanitizers(tmp_path):
    lib = _sanitized_library(str(tmp_path))
    # the host code is instrumented: it calls into both sanitizer runtimes
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], stdout=subprocess.PIPE, text=True,
                           check=True).stdout
    assert "__asan_report_" in undef and "__ubsan_handle_" in undef
    env = dict(os.environ)
    # the sanitizer runtime must be the first library loaded; anything already preloaded stays
    env["LD_PRELOAD"] = " ".join(x for x in (ASAN_RT, os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["BT_LIBRARY"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    report = r.stdout[-4000:]
    assert "ERROR: AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, report
    assert r.returncode == 0, report
    # and the child loaded that build, not the in-tree library
    probe = ("import hierarchical_global_local_amd as hg; L = hg.lib(); "
             "print(L._name, open('/proc/self/maps').read().count('libbt_host_sanitized.so') > 0)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.split()[-2:] == [lib, "True"], r.stdout[-2000:]
