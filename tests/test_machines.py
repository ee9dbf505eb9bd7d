"""The bit-parallel split state machines (digit groups of at most three,
CR/LF runs after punctuation, the whitespace lookahead) against the
byte-at-a-time rules they replace, on the host."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "byte_level_bpe_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_machines_match_byte_rules(tmp_path):
    exe = str(tmp_path / "machines_check")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-I", CSRC,
                           os.path.join(HERE, "native", "machines_check.cpp"), "-o", exe])
    out = subprocess.run([exe, "400000"], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "mismatches 0" in out.stdout
