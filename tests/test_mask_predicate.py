"""Host check of the tile mask tests with which the backward kernels skip the
causal and tail mask: tests/mask_check/mask_check.cpp is compiled (host only)
against the very header the kernels include (csrc/attn_mask.h) and brute-
forces those tests over sequence lengths and tile offsets; see that file."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "mask_check", "mask_check.cpp")
CSRC = os.path.join(ROOT, "io_aware_exact_attn_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_backward_mask_skip_is_sound(tmp_path):
    exe = str(tmp_path / "mask_check")
    subprocess.run([HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-std=c++17", "-I", CSRC, SRC, "-o", exe],
                   check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "violations 0" in r.stdout


def test_the_kernels_use_the_checked_header():
    src = open(os.path.join(CSRC, "attn_bwd.hip"), encoding="utf-8").read()
    assert '#include "attn_mask.h"' in src
    assert src.count("dq_half_tile_unmasked(") == 1 and src.count("dkdv_half_tile_unmasked(") == 2
