"""The C-ABI host checks again, on a copy of the library whose host code
(argument validation, workspace planning, layer orchestration) is built with
AddressSanitizer and UndefinedBehaviorSanitizer (build.py --sanitize; device
code unchanged). test_abi_host.py runs in a child process with the ASan
runtime preloaded and LLATTE_LIBRARY pointing at the instrumented copy; any
sanitizer report aborts it."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_host_code_under_address_and_undefined_behavior_sanitizers():
    from target_aware_latent_amd import build as b
    lib = b.build(sanitize=True)
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "host code is not instrumented"
    env = dict(os.environ)
    env.update(LD_PRELOAD=b.asan_runtime(), LLATTE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi_host.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
