"""Host-side checks of the gfx950 code the library's own sources compile to (no GPU needed).

The verification kernel reduces a query's score maximum and probability sum across lanes
l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 lane swaps (v_permlane16_swap / v_permlane32_swap),
which leave the two swapped registers as a pair. This compiler has been seen to combine such a
pair as if both halves were the same value (emitting `v_add_f32 v1, v1, v1`, or dropping a max),
which silently reduces over the wrong lanes. The kernel's current code is correct; this test
compiles it with the library's flags and checks that every swap's two registers meet in the
max or add that follows, so a toolchain that folds them is caught before the GPU tests run.
"""
import os
import re
import shutil
import subprocess

import pytest

from whisper_asr_encoder_amd import build as B

SWAP = re.compile(r"v_permlane(16|32)_swap_b32_e32 (v\d+), (v\d+)")
COMBINE = re.compile(r"(v_max_f32_e32|v_add_f32_e32) (v\d+), (v\d+), (v\d+)")


def lane_swap_pairs(asm: str):
    """(swap line, True if a following max/add reads both swapped registers) for each swap."""
    lines = asm.split("\n")
    out = []
    for i, line in enumerate(lines):
        m = SWAP.search(line)
        if not m:
            continue
        pair = {m.group(2), m.group(3)}
        both = False
        for nxt in lines[i + 1:i + 40]:
            c = COMBINE.search(nxt)
            if c and set(c.group(3, 4)) == pair:
                both = True
                break
        out.append((line.strip(), both))
    return out


def test_pair_detector_on_known_patterns():
    good = "v_permlane16_swap_b32_e32 v2, v9\nv_max_f32_e32 v9, v9, v9\nv_max_f32_e32 v2, v2, v9\n"
    folded = "v_permlane16_swap_b32_e32 v1, v2\nv_add_f32_e32 v1, v1, v1\n"
    assert lane_swap_pairs(good) == [("v_permlane16_swap_b32_e32 v2, v9", True)]
    assert lane_swap_pairs(folded) == [("v_permlane16_swap_b32_e32 v1, v2", False)]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs the ROCm toolchain")
def test_verify_kernel_lane_swaps_combine_both_registers(tmp_path):
    out = tmp_path / "verify_attn.s"
    cmd = [B.hipcc(), *[f for f in B.COMMON if f != "-fPIC"], "--cuda-device-only", "-S", "-x", "hip",
           os.path.join(B.CSRC, "verify_attn.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    pairs = lane_swap_pairs(out.read_text())
    assert pairs, "no lane swaps found: the reductions changed, update this test"
    bad = [line for line, both in pairs if not both]
    assert not bad, f"lane swaps whose two registers are not combined: {bad[:4]}"
