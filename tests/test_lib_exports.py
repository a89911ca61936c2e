"""The built library loads on a machine without a GPU and exports exactly the
entry points ``include/sampler.h`` declares (no compute calls here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sampler.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DST_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib_path():
    from decode_step_token_amd import LIB_PATH
    if not os.path.exists(LIB_PATH):
        from decode_step_token_amd.build import build
        build()
    return LIB_PATH


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("sampler_create", "sample_batch", "write_tokens", "sampler_wait", "sampler_destroy"):
        assert n in names


def test_library_exports_every_declared_symbol(lib_path):
    lib = ctypes.CDLL(lib_path)
    for name in _declared():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else(lib_path):
    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], capture_output=True, text=True,
                         check=True).stdout
    text_syms = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert text_syms == _declared()


def test_binding_names_match_header(lib_path):
    import decode_step_token_amd as pkg
    assert sorted(pkg.EXPORTS) == _declared()
    for name in _declared():
        assert callable(getattr(pkg, name, None)) or name in ("sampler_last_error",), name


def test_strerror_without_gpu(lib_path):
    import decode_step_token_amd as pkg
    pkg.load(lib_path)
    assert pkg.sampler_strerror(0) == "ok"
    assert "pinned" in pkg.sampler_strerror(-4)
    assert pkg.sampler_strerror(-99) == "unknown status"


def test_build_flags_target_gfx950_without_packed_fp32():
    from decode_step_token_amd import build as b
    assert "--offload-arch=gfx950" in b.CFLAGS
    i = b.CFLAGS.index("-packed-fp32-ops")
    assert b.CFLAGS[i - 1] == "-Xclang" and b.CFLAGS[i - 2] == "-target-feature"
