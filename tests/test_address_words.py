"""The scalar-base address composition of the prefill tile kernel's
global-to-LDS loads (paged_kv_cache_83_amd/csrc/pa_addr.h), built with the host
compiler and checked on the CPU: addresses whose low 32-bit word has bit 31 set
come back intact, and the sign-extending composition that once made the kernel
fault on such addresses fails the same check."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_join_address_words():
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "address_words")
        subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", "-o", exe,
                        os.path.join(HERE, "native", "address_words.cpp")], check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "failures 0" in r.stdout
