"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer:
``decode_step_token_amd/lib/host_check`` (built by ``build()`` from the same
sources with host-only sanitizer flags, driven by ``csrc/host_check.cpp``)
runs the C ABI's argument checks on the CPU, and with a GPU a short sequence
of every entry point; any sanitizer report or failed check ends it with a
non-zero status."""
import os
import subprocess

import pytest

from decode_step_token_amd import build as B


def _run():
    assert os.path.exists(B.HOST_CHECK), f"{B.HOST_CHECK} not built (run __graft_entry__.build())"
    env = dict(os.environ)
    # the HIP runtime keeps allocations until exit; leaks are not what this checks
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    p = subprocess.run([B.HOST_CHECK], env=env, capture_output=True, text=True, timeout=240)
    out = p.stdout + p.stderr
    assert p.returncode == 0 and "host sanitizers: ok" in p.stdout, out[-4000:]
    return out


def test_host_code_without_gpu_calls():
    """On any machine: the argument checks that fail before a HIP call (on a
    machine with a GPU the same run also covers the sequence below)."""
    out = _run()
    assert "part done, 0 failures" in out


@pytest.mark.gpu
def test_host_code_full_sequence():
    out = _run()
    assert "GPU part done, 0 failures" in out
