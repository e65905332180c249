"""CPU: the host-side layer of the C ABI (argument validation, the host BlockMask builder, the
allocation-free entry point's bookkeeping) under AddressSanitizer and UndefinedBehaviorSanitizer.

The sanitized build instruments api.cpp and noalloc.hip on the host only and takes the kernel
launchers from the regular library. The host-logic tests (test_abi_cpu.py and
test_host_blockmask.py) run in a child process with the sanitizer runtime preloaded and
FLEXATTN_LIBRARY pointing at the sanitized build; any report fails the run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.slow
def test_host_layer_under_asan_and_ubsan():
    from block_sparse_masked_blockmask_amd import build as b
    lib = b.build_sanitized()
    rt = b.sanitizer_runtime()
    assert rt and os.path.exists(rt), "no AddressSanitizer runtime found"
    env = dict(os.environ, LD_PRELOAD=rt, FLEXATTN_LIBRARY=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    env.pop("FLEXATTN_DEVICE_ARCH", None)
    # The child loads the sanitized build (its exported entry points call the instrumented code).
    probe = subprocess.run([sys.executable, "-c", "import block_sparse_masked_blockmask_amd as fa; fa.lib(); "
                            "print(fa.LIB_PATH)"], cwd=ROOT, env=env, capture_output=True, text=True)
    assert probe.returncode == 0 and probe.stdout.strip() == lib, probe.stdout + probe.stderr
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm, "the build is not instrumented"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi_cpu.py",
                        "tests/test_host_blockmask.py", "-k", "not clamp_helpers"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
