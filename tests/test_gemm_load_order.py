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


def _kernel_sections(lines, name_part):
    """Instruction lists of one kernel, split at each s_barrier; each section but the first is
    preceded by the last instruction of the previous one (the step's wait)."""
    out, cur, inside = [], [], False
    for l in lines:
        if re.match(r"^_Z\w+:", l):
            if inside:
                break
            inside = name_part in l
            continue
        t = l.strip()
        if not inside or not t or t.startswith((";", ".")):
            continue
        if t == "s_barrier":
            out.append(cur)
            cur = []
        else:
            cur.append(t)
    out.append(cur)
    return out


@pytest.mark.parametrize("nkt", [8, 2])
def test_streamed_down_gemm_keeps_its_load_counts(asm, nkt):
    """The streamed down GEMM (k-tiles of consecutive tiles as one stream) relies on every step
    issuing the same loads: 5 direct-to-LDS A loads, then 8 B loads (4 code, 4 scale), before the
    next step's wait for at most 8 outstanding; and on the epilogue step issuing its 16 row stores
    before its loads. Nothing may wait for every outstanding load inside the tile loop."""
    secs = _kernel_sections(asm, f"gemm_down_mx_stream_kernelILi0ELi{nkt}E")
    last = nkt + 1                               # the epilogue position's section
    assert len(secs) == nkt + 2, len(secs)       # prologue, then positions 0..nkt of a tile
    ops = [[x.split()[0] for x in s] for s in secs]
    for i in range(last):                        # the wait ending each section
        waits = [x for x in secs[i] if x.startswith("s_waitcnt") and "vmcnt" in x]
        assert waits and waits[-1] == "s_waitcnt vmcnt(8)", (i, waits)
    for i, s in enumerate(ops[1:], start=1):
        dma = [j for j, op in enumerate(s) if op == "global_load_lds_dwordx4"]
        bl = [j for j, op in enumerate(s) if op in ("buffer_load_dwordx4", "buffer_load_dword")]
        assert len(dma) == 5 and len(bl) == 8, (i, len(dma), len(bl))
        assert max(dma) < min(bl), i
        assert s.count("buffer_load_dwordx4") == 4, i
        if i < last:
            assert not any(x.startswith("s_waitcnt") and "vmcnt(0)" in x for x in secs[i]), i
    st = [j for j, op in enumerate(ops[last]) if op == "buffer_store_dwordx4"]
    loads = [j for j, op in enumerate(ops[last]) if op in ("global_load_lds_dwordx4", "buffer_load_dwordx4",
                                                            "buffer_load_dword")]
    assert len(st) == 16 and max(st) < min(loads)
    assert not any(op.startswith("scratch_") for s in ops for op in s)   # no spills
