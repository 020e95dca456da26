"""The host-side C-ABI layer under AddressSanitizer (CPU only).

The library is rebuilt with its argument-validation and launch set-up code (csrc/mla_api.hip)
instrumented, and the C-ABI tests run against it in a child process with the sanitizer runtime
preloaded and Python's allocator routed to malloc (so the ctypes descriptors the tests pass are
heap blocks the sanitizer bounds). Every call in those tests is rejected (or is a no-op) before any
HIP call, so the run needs no GPU; an out-of-bounds read of a descriptor or a use of freed memory in
the validation code would end the child with a sanitizer report.
"""
import glob
import os
import subprocess
import sys

import pytest

from head_latent_attention_04_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def sanitized_env(tmp_path, runtime, lib=None):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": runtime, "PYTHONMALLOC": "malloc",
                "ASAN_OPTIONS": f"detect_leaks=0:halt_on_error=1:log_path={tmp_path}/asan"})
    if lib:
        env["MLA_LIBRARY"] = lib
    return env


def reports(tmp_path):
    return "".join(open(p).read() for p in glob.glob(str(tmp_path / "asan*")))


def test_abi_validation_under_address_sanitizer(tmp_path):
    try:
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    # the preloaded runtime does watch this process's heap: copying 72 bytes out of a 64-byte ctypes
    # buffer is reported
    canary = tmp_path / "canary"
    canary.mkdir()
    r = subprocess.run([sys.executable, "-c", "import ctypes; a = ctypes.create_string_buffer(64); "
                        "b = ctypes.create_string_buffer(128); ctypes.memmove(b, a, 72)"],
                       env=sanitized_env(canary, runtime), capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in reports(canary), r.stderr[-2000:]

    lib = build.build_host_asan(str(tmp_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=sanitized_env(tmp_path, runtime, lib), capture_output=True, text=True,
                       timeout=600)
    out = r.stdout + r.stderr
    rep = reports(tmp_path)
    assert "AddressSanitizer" not in rep, rep[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
