"""Checks on the gfx950 assembly of the backward kernels (compiled here, CPU only).

The backward kernels issue their global -> LDS copies as inline asm that sets M0 (the LDS
address) itself; the compiler does not know that M0 changes there.  That is safe only while
no compiler-generated instruction in those kernels uses M0: every M0 write in the assembly
must be one of ours, directly followed by the copy that uses it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "attention_additive_rank_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("d", [32, 64])
def test_backward_m0_only_feeds_the_direct_loads(tmp_path, d):
    out = tmp_path / f"bwd{d}.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-ffp-contract=fast", "-mllvm", "-amdgpu-mfma-vgpr-form=1", f"-DFB_BWD_D={d}",
           "--cuda-device-only", "-S", os.path.join(CSRC, "fb_attn_bwd_inst.hip"), "-o", str(out)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
    lines = [l.split(";")[0].strip() for l in out.read_text().splitlines()]
    lines = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    writes = 0
    for i, l in enumerate(lines):
        if not re.search(r"\bm0\b", l):
            continue
        assert l.startswith("s_mov_b32 m0,"), f"compiler-generated use of M0: {l}"
        nxt = lines[i + 1:i + 3]
        assert nxt and nxt[0] == "s_nop 0" and nxt[1].startswith("global_load_lds_dword"), \
            f"M0 write not followed by its copy: {l} / {nxt}"
        writes += 1
    assert writes > 0
