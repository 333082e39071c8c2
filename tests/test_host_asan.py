"""The C-ABI host runtime under AddressSanitizer (CPU only).

The library's host code (validation, workspace plan, error paths, the
allocation-free entry's checks) is rebuilt with host-side ASan, and the CPU
tests of the C ABI run against that build in a child process with the ASan
runtime preloaded.  Any invalid host memory access aborts the child."""

import os
import subprocess
import sys

from conftest import ROOT


def test_abi_cpu_tests_pass_under_address_sanitizer(tmp_path):
    from quantized_q8_dequant_amd.build_asan import asan_runtime, build_asan

    so = build_asan(str(tmp_path))
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    code = (
        "import sys; sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r});"
        "from quantized_q8_dequant_amd import _lib; _lib.LIB_PATH = {so!r};"
        "import pytest; sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', {test!r}]))"
    ).format(root=ROOT, tests=os.path.join(ROOT, "tests"), so=so, test=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "AddressSanitizer" not in r.stderr, out
    assert " passed" in r.stdout, out
