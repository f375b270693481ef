"""The host side of the C ABI under AddressSanitizer (CPU only).

The library's host code is rebuilt with -fsanitize=address (device code is
unchanged and never runs here) and tests/test_abi.py is run against it in a
child process with the sanitizer runtime preloaded: every argument check,
status string, size helper and host validator then executes instrumented, and
any out-of-bounds or use-after-free access aborts the child."""
import os
import subprocess
import sys

from exact_io_aware_07_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_address_sanitizer():
    lib = B.build_asan()
    env = dict(os.environ, LD_PRELOAD=B.asan_runtime(), EXACT_ATTN_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    probe = ("import exact_io_aware_07_amd as ea; ea.lib(); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libclang_rt.asan' in maps and 'libattn_asan.so' in maps, 'sanitizer build not loaded'; "
             "print(ea.lib_path)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "libattn_asan.so" in r.stdout, r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout and "AddressSanitizer" not in r.stderr
