"""The host code of the library (block allocator, prefix sharing, scheduler,
timing bookkeeping) under AddressSanitizer and UndefinedBehaviorSanitizer:
build.build_sanitized() compiles it instrumented, and the CPU parity tests
of the host code (hypothesis operation sequences and hand-worked traces
against the oracle's allocator, seeded and hand-worked scheduler traces, the
four schedules) run again in a child process against that build, with the
sanitizer runtime preloaded and any report fatal."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_host_allocator.py", "tests/test_host_scheduler.py",
              "tests/test_host_sched_modes.py"]


def test_host_code_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from paged_kv_cache_host_amd import build

    lib = build.build_sanitized(str(tmp_path))
    syms = subprocess.run(["nm", "-D", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_report" in syms and "__ubsan_handle" in syms, "the build is not instrumented"
    env = dict(os.environ,
               PA_LIBRARY=lib,
               LD_PRELOAD=build.sanitizer_runtime(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", *HOST_TESTS, "-x", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=900)
    tail = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, tail
    assert " passed" in r.stdout and "failed" not in r.stdout, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
