"""The causal pairing of query tiles (fa_schedule.h) checked on the host: with
a grid sized for the sequence every tile is visited once; with a grid sized
for a shorter max_seqlen the interior tiles (causal) or the tail tiles (no
mask) are the ones left out, as the varlen calls document
(tests/schedule_check.cpp)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_03_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_causal_pairing_coverage(tmp_path):
    exe = tmp_path / "schedule_check"
    r = subprocess.run(["g++", "-std=c++17", "-O1", f"-I{CSRC}", os.path.join(ROOT, "tests", "schedule_check.cpp"),
                        "-o", str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert out.returncode == 0 and "schedule check: ok" in out.stdout, out.stdout
