"""The host side of the C ABI under AddressSanitizer: the argument checks,
size queries and host planning of api.cpp, built with ASan (host code only),
run the CPU ABI tests in a child process with the ASan runtime preloaded. Any
out-of-bounds access or use after free in those paths aborts the child."""
import os
import subprocess
import sys

from speech_recognition_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_checks_under_host_asan():
    lib = build.build_asan()
    env = dict(os.environ, LD_PRELOAD=build.asan_runtime(), WHISPER_MI355X_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout, out
