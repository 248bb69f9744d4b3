"""The host-side ABI tests again, against the host-sanitizer build of the
library (AddressSanitizer + UndefinedBehaviorSanitizer on the host code; see
dense_gpt_pretraining_nanochat_amd/sanitize.py), in a child process with the
sanitizer runtime preloaded: config validation, layout and workspace
planning and every argument check run with memory errors and undefined
behaviour turned into failures. CPU only."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc to build the sanitizer library")
def test_host_abi_under_address_and_ub_sanitizers():
    from dense_gpt_pretraining_nanochat_amd import sanitize
    lib = sanitize.build_asan()
    env = dict(os.environ)
    env["LD_PRELOAD"] = sanitize.runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["NANOCHAT_LIB"] = lib
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_host.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
