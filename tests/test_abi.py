"""The C-ABI library loads on a machine without a GPU, exports every entry point declared in
include/moe_w2.h, and rejects bad arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w2.h")
LIB = os.path.join(ROOT, "bit_routed_expert_amd", "libmoew2.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libmoew2.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("moe_w2_pack", "moe_w2_forward", "nvfp4_to_w2", "moe_w2_route", "moe_w2_unpack",
              "moe_w2_workspace_bytes", "moe_w2_read_counters", "moe_w2_planes_free"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_host_side_validation(lib):
    P = ctypes.c_void_p
    lib.moe_w2_abi_version.restype = ctypes.c_int
    assert lib.moe_w2_abi_version() == 1
    lib.moe_w2_status_string.restype = ctypes.c_char_p
    assert lib.moe_w2_status_string(-3)
    # null pointers -> EINVAL, unsupported shapes -> EUNSUPPORTED, both before any device work
    out = P()
    lib.moe_w2_pack.argtypes = [ctypes.c_int] * 3 + [P] * 5 + [ctypes.POINTER(P)]
    assert lib.moe_w2_pack(8, 256, 512, None, None, None, None, None, ctypes.byref(out)) == -1
    assert out.value is None
    fake = P(16)
    assert lib.moe_w2_pack(8, 200, 512, fake, fake, fake, fake, None, ctypes.byref(out)) == -2
    assert lib.moe_w2_pack(2000, 256, 512, fake, fake, fake, fake, None, ctypes.byref(out)) == -2
    lib.moe_w2_forward.argtypes = [P, ctypes.c_int, ctypes.c_int, P, P, P, P, ctypes.c_int, P, ctypes.c_size_t, ctypes.c_int, P]
    assert lib.moe_w2_forward(None, 1, 8, fake, fake, fake, fake, 0, fake, 1 << 20, 0, None) == -1
    lib.nvfp4_to_w2.argtypes = [ctypes.c_int] * 3 + [P] * 6
    assert lib.nvfp4_to_w2(1, 4, 48, fake, fake, fake, fake, fake, None) == -2
    assert lib.nvfp4_to_w2(1, 4, 64, None, fake, fake, fake, fake, None) == -1
    assert lib.nvfp4_to_w2(0, 4, 64, None, None, None, None, None, None) == 0   # empty: no-op
    lib.moe_w2_route_workspace_bytes.restype = ctypes.c_size_t
    assert lib.moe_w2_route_workspace_bytes(256, 32, 8) > 0
    assert lib.moe_w2_route_workspace_bytes(0, 32, 8) == 0
    lib.moe_w2_route.argtypes = [ctypes.c_int] * 3 + [P] * 4 + [ctypes.c_size_t, P]
    assert lib.moe_w2_route(256, 4, 8, fake, fake, fake, None, 0, None) == -6


def test_pair_count_bound(lib):
    """T * top_k above 2^30 pairs is refused on the host: the size queries return 0 and the route
    call MOE_W2_EUNSUPPORTED (no signed overflow into a wrong size or a negative pair count)."""
    P = ctypes.c_void_p
    fake = P(16)
    lib.moe_w2_route_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_w2_route_workspace_bytes.argtypes = [ctypes.c_int] * 3
    lib.moe_w2_route.argtypes = [ctypes.c_int] * 3 + [P] * 4 + [ctypes.c_size_t, P]
    lib.moe_w2_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_w2_workspace_bytes.argtypes = [P, ctypes.c_int, ctypes.c_int]
    at_bound = (1 << 30) // 8
    assert lib.moe_w2_route_workspace_bytes(256, at_bound, 8) > 0
    for T, k in ((at_bound + 1, 8), (1 << 28, 32), (2**31 - 1, 2), (2**31 - 1, 32)):
        assert lib.moe_w2_route_workspace_bytes(256, T, k) == 0
        assert lib.moe_w2_route(256, T, k, fake, fake, fake, fake, 1 << 40, None) == -2
    assert lib.moe_w2_workspace_bytes(None, 1 << 28, 32) == 0


def test_binding_imports_without_gpu():
    import bit_routed_expert_amd as m
    assert m.moe_w2_abi_version() == 1


def test_codebook_sweep_host_validation(lib):
    """Argument checks of moe_w2_codebook_sweep happen on the host, before any device call."""
    P = ctypes.c_void_p
    f = lib.moe_w2_codebook_sweep
    f.argtypes = [ctypes.c_int] * 3 + [P, ctypes.c_int, P, P, P, P, P]
    f.restype = ctypes.c_int
    fake = ctypes.c_void_p(256)
    good = (ctypes.c_float * 4)(-4, -1, 1, 4)
    flat = (ctypes.c_float * 4)(-4, -1, -1, 4)
    nan = (ctypes.c_float * 4)(-4, -1, 1, float("nan"))
    assert f(1, 2, 64, fake, 1, flat, fake, fake, fake, None) == -1
    assert f(1, 2, 64, fake, 1, nan, fake, fake, fake, None) == -1
    assert f(1, 2, 48, fake, 1, good, fake, fake, fake, None) == -2
    assert f(1, 2, 64, fake, 0, good, fake, fake, fake, None) == -1
    assert f(1, 2, 64, fake, 4097, good, fake, fake, fake, None) == -1     # more codebooks than allowed
    assert f(1, 2, 64, fake, 1, None, fake, fake, fake, None) == -1
    assert f(-1, 2, 64, fake, 1, good, fake, fake, fake, None) == -1
    assert f(0, 2, 64, None, 1, good, None, None, None, None) == 0
