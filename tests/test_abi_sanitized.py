"""The C-ABI tests again, against the build whose host side (argument
validation, workspace sizing, launch set-up) is compiled with
AddressSanitizer and UndefinedBehaviorSanitizer.  CPU only: no kernel is
launched, so the sanitizers watch exactly the host layer.  The tests run in a
child process with the clang ASan runtime preloaded (python itself is not
built with it); any report aborts that process and fails this test."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale(lib):
    """True when the built library is missing or older than a source it is
    built from (the HIP sources, their headers, the C-ABI header)."""
    from contextual_token_sparsity_amd import build
    if not os.path.exists(lib):
        return True
    srcs = [os.path.join(build.CSRC, f) for f in os.listdir(build.CSRC)]
    srcs += [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))]
    built = os.path.getmtime(lib)
    return any(os.path.getmtime(f) > built for f in srcs)


def test_abi_tests_pass_under_asan_and_ubsan():
    from contextual_token_sparsity_amd import build
    if _stale(build.HOSTCHECK_LIB):
        build.build_host_check()
    env = dict(os.environ)
    env.update({
        "LEMO_LIB_PATH": build.HOSTCHECK_LIB,
        "LD_PRELOAD": build.asan_runtime(),
        # python and torch are not instrumented: leaks and cross-library checks
        # of theirs are out of scope
        "ASAN_OPTIONS": "detect_leaks=0:detect_odr_violation=0:alloc_dealloc_mismatch=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi_cpu.py"), "-q",
                        "-p", "no:cacheprovider", "-x"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "Sanitizer" not in r.stdout + r.stderr, tail
