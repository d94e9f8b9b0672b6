"""CPU check of the forward kernel's tile-copy index maps (csrc/fb_tile_map.h, shared with the
kernel): compiled with the host compiler and run for every 16-bit shape the library
instantiates.  Every direct load must read inside its source row (K and V rows of D
elements, phi_k rows of R elements; a V row is narrower than its LDS region when D < 32)
and every chunk slot of a tile must be written exactly once; the resident kernel's copies of
every tile of a (b, h) must land inside its LDS arrays."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_additive_rank_amd", "csrc")
CXX = shutil.which("g++") or shutil.which("c++")


@pytest.mark.skipif(CXX is None, reason="no host C++ compiler")
def test_tile_copies_stay_in_their_rows(tmp_path):
    exe = tmp_path / "loader_bounds"
    src = os.path.join(ROOT, "tests", "native", "loader_bounds.cpp")
    r = subprocess.run([CXX, "-std=c++17", "-O1", "-Wall", "-I", CSRC, src, "-o", str(exe)],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert r.returncode == 0, r.stdout
    r = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=60)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "ok D=16 RP=16 R=8 loader" in r.stdout
    assert "ok resident D=32 RP=16: 8 tiles (512 keys)" in r.stdout
