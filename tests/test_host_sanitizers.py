"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is built a second time with both sanitizers on its host half
(errors fatal; device code as usual), and the validation tests of test_abi.py
and the allocation-free entry point's rejection test run against that build in
a child process with the sanitizer runtime preloaded.  CPU only: nothing here
launches a kernel, and no GPU run loads the sanitized build."""
import os
import subprocess
import sys

from long_context_attention_14_amd import build as lca_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_asan_and_ubsan():
    lib = lca_build.build(sanitize=True)
    env = dict(os.environ, LCA_LIB=lib, LD_PRELOAD=lca_build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", "test_abi.py"),
             os.path.join(ROOT, "tests", "test_zz_no_alloc.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *tests], env=env, capture_output=True, text=True, timeout=900, cwd=ROOT)
    out = r.stdout[-4000:] + "\n" + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, out
    assert " passed" in r.stdout, out


def test_sanitized_build_really_is_instrumented():
    """The sanitized library carries the sanitizer entry points (so the test above
    is not silently running an uninstrumented build)."""
    lib = lca_build.SAN_LIB
    if not os.path.exists(lib):
        lca_build.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_" in syms and "__ubsan_" in syms
