"""The C ABI from a plain C program (tests/c_caller/kvq_c_caller.c): no
Python binding and no torch between the caller and the library.

CPU: the program builds (include/kvq.h read by a C99 compiler with -Wall
-Werror, linked against the in-tree library) and the binary depends on that
library.  GPU: on a contiguous cache and on a paged one whose block table the
program keeps itself (a block per key group before the call that quantizes
it), the program runs prefill, appends across group flushes, kv_dequantize
and both attention entry points on device memory from hipMalloc, and checks them against the oracle compiled into it (dequantized
values bit for bit, attention within max-abs 2e-3 and per-row cosine 0.9999,
the no-allocation call equal to the workspace call); it exits 0 only if all
checks pass."""
import importlib.util
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("kvq_c_caller_build", os.path.join(HERE, "c_caller", "build.py"))
c_caller_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(c_caller_build)
BIN = c_caller_build.BIN


def test_c_caller_builds_and_links_the_library():
    lib = os.path.join(os.path.dirname(HERE), "quantized_decode_attention_kivi_amd", "libkvq.so")
    if not os.path.exists(lib):
        pytest.skip("libkvq.so not built (run __graft_entry__.build())")
    c_caller_build.build()
    out = subprocess.run(["ldd", BIN], capture_output=True, text=True, check=True).stdout
    assert "libkvq.so" in out and "libamdhip64" in out


@pytest.mark.gpu
def test_c_caller_against_oracle():
    assert os.path.exists(BIN), "build the C caller first (__graft_entry__.build())"
    print("running %s" % BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    assert r.stdout.count("bit-exact") == 2 and r.stdout.count("call identical") == 2
