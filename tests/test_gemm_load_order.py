"""The grouped GEMMs' counted waits rest on two orderings in the code hipcc emits for gfx950; this
compiles csrc/gemm.hip to assembly (no GPU needed) and checks both in every k-loop step:

* every direct-to-LDS load (the A stage) of a step is issued before the step's B code and scale
  loads, so "at most kBLoads loads outstanding" means the stage has landed;
* no LDS read is issued between a step's last matrix instruction and the barrier that ends the
  step (a read there would belong to the next stage and run ahead of its barrier)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "bit_routed_expert_amd", "csrc", "gemm.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "gemm.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", SRC, "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text().splitlines()


def _steps(lines):
    """(kernel, [instruction mnemonics]) between consecutive s_barriers of the GEMM kernels."""
    kern, cur, out = None, [], []
    for l in lines:
        if re.match(r"^_Z\w+:", l):
            kern, cur = l, []
            continue
        t = l.strip()
        if not t or t.startswith((";", ".")) or kern is None or "gemm_" not in kern:
            continue
        if t == "s_barrier":
            out.append((kern, cur))
            cur = []
        else:
            cur.append(t.split()[0])
    return out


def test_dma_before_b_loads_in_every_step(asm):
    steps = [(k, s) for k, s in _steps(asm) if "global_load_lds_dwordx4" in s and "global_load_dwordx4" in s]
    assert len(steps) >= 12         # the k-loop steps of gate_up and down, all three weight formats
    assert any("nv4" in k for k, _ in steps)
    for kern, s in steps:
        last_dma = max(i for i, op in enumerate(s) if op == "global_load_lds_dwordx4")
        first_b = min(i for i, op in enumerate(s)
                      if op in ("global_load_dwordx4", "global_load_dwordx2", "global_load_ushort"))
        assert first_b > last_dma, kern


def test_no_lds_read_after_last_mfma_before_barrier(asm):
    n = 0
    for kern, s in _steps(asm):
        mf = [i for i, op in enumerate(s) if op.startswith("v_mfma")]
        if not mf:
            continue
        n += 1
        assert not any(op.startswith("ds_read") for op in s[mf[-1] + 1:]), kern
    assert n >= 8
