"""Host check of the token-level top-k count and position arithmetic.

The token kernels take every count and position that addresses an index row
from block_sparse_attention_12_amd/csrc/tok_positions.h (host and device
code). tests/host/tok_positions_check.cpp runs the kernels' chain on the host
through those functions: on consistent keys the row must equal the brute-force
top-k, and on inconsistent histograms, chunk counts and stored words every
write must stay inside the row, with the undefined-behaviour and address
sanitizers on.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_token_positions_stay_in_the_row(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "tok_positions_check")
    src = os.path.join(HERE, "host", "tok_positions_check.cpp")
    subprocess.run([gxx, "-O1", "-std=c++17", "-fsanitize=undefined,address",
                    "-fno-sanitize-recover=all", src, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
