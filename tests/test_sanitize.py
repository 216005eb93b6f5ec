"""The host side of libspecattn under AddressSanitizer and
UndefinedBehaviorSanitizer, with the debug build's plan checker: a CPU-only
driver (tests/sanitize/abi_driver.c) plans tens of thousands of shapes and
checks every workgroup's staging bounds, sizes every workspace at ordinary
and extreme arguments, and feeds every entry point arguments its
validation must reject.  No kernel is launched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = os.path.join(ROOT, "tests", "sanitize", "build_and_run.sh")
OBJS = ["attn.o", "generic.o", "accept.o", "commit.o", "select.o", "gather.o"]


def test_host_library_under_asan_and_ubsan():
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not (os.path.exists(hipcc) or shutil.which("hipcc")):
        pytest.skip("hipcc is not available")
    if not all(os.path.exists(os.path.join(ROOT, "_build", o)) for o in OBJS):
        pytest.skip("the regular build's objects are missing (python -m sparse_kv_attention_sink_amd.build)")
    r = subprocess.run(["bash", SCRIPT], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, f"sanitized driver failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    assert "abi driver ok" in r.stdout
