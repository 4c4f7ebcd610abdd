"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer: the sanitizer
build of the library (build.py --variant asan: host code instrumented, device code unchanged) runs
the host-validation checks of test_abi.py in a child process with the sanitizer runtime preloaded.
Any heap or stack overrun, use after free or undefined behaviour on those paths aborts the child."""
import glob
import os
import subprocess
import sys

import pytest

from mla_latent_kv_27_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RUNTIME = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))


@pytest.mark.skipif(not RUNTIME, reason="no clang AddressSanitizer runtime in this ROCm install")
def test_abi_checks_clean_under_host_sanitizers():
    lib = B.build(variant="asan")
    # the host code really is instrumented: it calls into both sanitizer runtimes
    nm = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True, check=True).stdout
    assert "__asan_" in nm and "__ubsan_handle_" in nm
    env = dict(os.environ, MLA_LIBRARY=lib, LD_PRELOAD=RUNTIME[-1],
               # the interpreter's own allocations are not the library's: leak checking off
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = ("import ctypes, mla_latent_kv_27_amd as M; M.lib(); "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print(M.LIB_PATH)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
