"""The host layer of libvsa (argument validation, workspace and layout
arithmetic, the C ABI's error paths) under AddressSanitizer and
UndefinedBehaviorSanitizer: the checking build of build_lib (host pass
instrumented, device code unchanged) runs the host-ABI and binding tests in a
child process with the ASan runtime preloaded; any sanitizer report fails.
CPU only: no kernel is launched on these paths."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

build_lib = pytest.importorskip("block_sparse_attention_19_amd.build_lib")


def test_host_abi_under_asan_ubsan():
    try:
        lib = build_lib.build(sanitize=True)
        runtime = build_lib.asan_runtime()
    except (RuntimeError, OSError) as e:
        pytest.skip(f"sanitizer build unavailable: {e}")
    env = dict(os.environ)
    env.update({
        "VSA_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_lib_host.py", "test_binding_checks.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", *tests],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in out
