"""Host-side check of the selection's launch geometry: a small C++ program compiled with
g++ from the library's own geometry header walks every workgroup of many (T, L, pos0, k,
CU count) shapes and checks that the score rows, key rows and candidate slots each
workgroup touches stay inside their buffers and that the tau bound is valid.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_decode_indexer_amd", "csrc")
SRC = os.path.join(ROOT, "tests", "host", "select_geometry_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_select_geometry_reads_and_writes_stay_in_bounds(tmp_path):
    exe = str(tmp_path / "select_geometry_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC, SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
