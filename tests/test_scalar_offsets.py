"""The decode kernels address each weight tile through a buffer resource with a wave-uniform
offset. When the compiler cannot prove such an offset uniform it wraps every load in a loop over
the lanes' distinct values (readfirstlane, compare, exec mask, branch): the results stay right but
every tile load costs several extra instructions. This compiles the streaming kernels to gfx950
assembly (no GPU needed) and checks that no kernel holds such a loop, and that the prefill GEMMs'
k-loops keep their counted waits (no wait for every outstanding load inside them)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_routed_expert_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# readfirstlane of a vector register, then a compare of the lanes' values against it: the head of
# the loop the compiler emits for a vector-held operand of a scalar slot
LANE_LOOP = re.compile(r"v_readfirstlane_b32 (s\d+), (v\d+)\n(?:\s*s_nop \d+\n)?\s*v_cmp_eq_u32_e\d+ vcc, \1, \2")


@pytest.mark.parametrize("src,min_kernels", [("decode.hip", 30), ("gemm.hip", 6)])
def test_no_lane_loops_around_loads(src, min_kernels, tmp_path):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    kernels = list(re.finditer(r"^(_Z\w+):", text, re.M))
    assert len(kernels) >= min_kernels
    bad = []
    for m in kernels:
        end = text.find(".Lfunc_end", m.end())
        n = len(LANE_LOOP.findall(text[m.end():end]))
        if n:
            bad.append((m.group(1), n))
    assert not bad, bad


def test_gemm_k_loops_keep_counted_waits(tmp_path):
    """The prefill GEMMs' k-loop waits for each k-tile with a counted wait (its loads two steps
    behind may stay outstanding). Where the compiler cannot track which loads a register waits on
    (e.g. a 16-bit load zero-extended at a loop merge), it waits for every outstanding load
    (vmcnt(0)) inside the loop, which serialises the operand pipeline. The block-scaled GEMM kernels
    have exactly two such waits, both outside the loop: before the first k-tile (the tile's pair
    indices) and the final drain before the epilogue reuses LDS."""
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path / "gemm.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, "gemm.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    counts = {}
    for m in re.finditer(r"^(_Z\w*gemm_(?:gate_up|down)_mx_kernel\w*):", text, re.M):
        end = text.find(".Lfunc_end", m.end())
        counts[m.group(1)] = len(re.findall(r"s_waitcnt vmcnt\(0\)", text[m.end():end]))
    assert len(counts) == 4
    assert all(n <= 2 for n in counts.values()), counts
