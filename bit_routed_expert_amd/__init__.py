"""Python binding of libmoew2 (include/moe_w2.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of ``libmoew2.so``; this module passes
torch device tensors' pointers and the current HIP stream to the C ABI and turns status codes into
exceptions. There is no fallback: if the library is missing or no GPU is present, calls fail.

Functions keep the C names: moe_w2_pack, moe_w2_unpack, moe_w2_workspace_bytes, moe_w2_route,
moe_w2_forward, moe_w2_forward_stage, moe_w2_forward_noalloc, moe_w2_read_counters; the re-quantizers nvfp4_to_w2,
fp8_block128_to_w2, mxfp4_to_w2; the FP4 planes moe_w4_pack, moe_w4_unpack, moe_w4_forward; the
expert-slot entry points moe_w2_planes_create, moe_w2_pack_slot, moe_w2_forward_slots,
moe_w2_read_miss_counter; and the sign-bias diagnostic moe_w2_codebook_sweep.
"""
import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoew2.so")

OUT_BF16, OUT_F32 = 0, 1
PATH_AUTO, PATH_DECODE, PATH_GEMM, PATH_DECODE_SORTED = 0, 1, 2, 3
STAGE_ROUTE, STAGE_GATE_UP, STAGE_DOWN, STAGE_COMBINE = 0, 1, 2, 3

STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "ESCALE", -4: "ENOMEM", -5: "EHIP",
          -6: "EWORKSPACE", -7: "ENVFP4", -8: "ENAN"}


class MoeW2Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib().moe_w2_status_string(status).decode()})")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoew2.so not built ({LIB_PATH}); run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "moe_w2_abi_version": ([], I32),
            "moe_w2_status_string": ([I32], ctypes.c_char_p),
            "moe_w2_pack": ([I32, I32, I32, P, P, P, P, P, ctypes.POINTER(P)], I32),
            "moe_w2_unpack": ([P, P, P, P, P, P], I32),
            "moe_w2_planes_free": ([P], None),
            "moe_w2_planes_info": ([P, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(I32),
                                    ctypes.POINTER(SZ)], I32),
            "moe_w2_workspace_bytes": ([P, I32, I32], SZ),
            "moe_w2_route_workspace_bytes": ([I32, I32, I32], SZ),
            "moe_w2_route": ([I32, I32, I32, P, P, P, P, SZ, P], I32),
            "moe_w2_forward": ([P, I32, I32, P, P, P, P, I32, P, SZ, I32, P], I32),
            "moe_w2_forward_stage": ([P, I32, I32, I32, P, P, P, P, I32, P, SZ, I32, P], I32),
            "moe_w2_forward_noalloc": ([P, I32, I32, P, P, P, P, I32, I32, P], I32),
            "moe_w2_read_counters": ([P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64), P], I32),
            "nvfp4_to_w2": ([I32, I32, I32, P, P, P, P, P, P], I32),
            "moe_w2_planes_create": ([I32, I32, I32, P, ctypes.POINTER(P)], I32),
            "moe_w4_pack": ([I32, I32, I32, P, P, P, P, P, ctypes.POINTER(P)], I32),
            "fp8_block128_to_w2": ([I32, I32, I32, P, P, P, P, P], I32),
            "mxfp4_to_w2": ([I32, I32, I32, P, P, P, P, P], I32),
            "moe_w4_unpack": ([P, P, P, P, P, P], I32),
            "moe_w4_pack_nvfp4": ([I32, I32, I32, P, P, P, P, P, P, P, ctypes.POINTER(P)], I32),
            "moe_w4_unpack_nvfp4": ([P, P, P, P, P, P, P, P], I32),
            "moe_w4_forward": ([P, I32, I32, P, P, P, P, I32, P, SZ, I32, P], I32),
            "moe_w2_pack_slot": ([P, I32, P, P, P, P, P], I32),
            "moe_w2_forward_slots": ([P, I32, P, I32, I32, P, P, P, P, I32, P, SZ, I32, P], I32),
            "moe_w2_read_miss_counter": ([P, ctypes.POINTER(ctypes.c_int64), P], I32),
            "moe_w2_codebook_sweep": ([I32, I32, I32, P, I32, P, P, P, P, P], I32),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _LIB = lib
    return _LIB


def _check(status, what):
    if status != 0:
        raise MoeW2Error(status, what)


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class Planes:
    """Native 2-bit planes of one MoE layer, owned by the library (freed on garbage collection)."""

    def __init__(self, handle, E, K, I):
        self._h = handle
        self.E, self.K, self.I = E, K, I
        sz = ctypes.c_size_t(0)
        _check(_lib().moe_w2_planes_info(handle, None, None, None, ctypes.byref(sz)), "moe_w2_planes_info")
        self.nbytes = sz.value

    @property
    def handle(self):
        return self._h

    def free(self):
        if self._h:
            _lib().moe_w2_planes_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def moe_w2_abi_version():
    return _lib().moe_w2_abi_version()


def moe_w2_pack(gu_codes, gu_scales, dn_codes, dn_scales):
    """Canonical device planes (uint8) -> Planes. Shapes: gu_codes [E, 2I, K/4], gu_scales [E, 2I, K/32],
    dn_codes [E, K, I/4], dn_scales [E, K, I/32]."""
    E, two_i, k4 = gu_codes.shape
    K, I = k4 * 4, two_i // 2
    if tuple(gu_scales.shape) != (E, 2 * I, K // 32) or tuple(dn_codes.shape) != (E, K, I // 4) \
            or tuple(dn_scales.shape) != (E, K, I // 32):
        raise ValueError("inconsistent plane shapes")
    h = ctypes.c_void_p()
    _check(_lib().moe_w2_pack(E, K, I, _dev(gu_codes, torch.uint8, "gu_codes"), _dev(gu_scales, torch.uint8, "gu_scales"),
                              _dev(dn_codes, torch.uint8, "dn_codes"), _dev(dn_scales, torch.uint8, "dn_scales"),
                              _stream(), ctypes.byref(h)), "moe_w2_pack")
    return Planes(h, E, K, I)


def moe_w4_pack(gu_codes, gu_scales, dn_codes, dn_scales):
    """Canonical FP4 device planes (uint8) -> Planes. Shapes: gu_codes [E, 2I, K/2] (two e2m1 codes per
    byte, low nibble = even element), gu_scales [E, 2I, K/32], dn_codes [E, K, I/2], dn_scales [E, K, I/32]."""
    E, two_i, k2 = gu_codes.shape
    K, I = k2 * 2, two_i // 2
    if tuple(gu_scales.shape) != (E, 2 * I, K // 32) or tuple(dn_codes.shape) != (E, K, I // 2) \
            or tuple(dn_scales.shape) != (E, K, I // 32):
        raise ValueError("inconsistent plane shapes")
    h = ctypes.c_void_p()
    _check(_lib().moe_w4_pack(E, K, I, _dev(gu_codes, torch.uint8, "gu_codes"), _dev(gu_scales, torch.uint8, "gu_scales"),
                              _dev(dn_codes, torch.uint8, "dn_codes"), _dev(dn_scales, torch.uint8, "dn_scales"),
                              _stream(), ctypes.byref(h)), "moe_w4_pack")
    return Planes(h, E, K, I)


def moe_w4_unpack(planes):
    E, K, I = planes.E, planes.K, planes.I
    d = torch.device("cuda")
    out = (torch.empty((E, 2 * I, K // 2), dtype=torch.uint8, device=d),
           torch.empty((E, 2 * I, K // 32), dtype=torch.uint8, device=d),
           torch.empty((E, K, I // 2), dtype=torch.uint8, device=d),
           torch.empty((E, K, I // 32), dtype=torch.uint8, device=d))
    _check(_lib().moe_w4_unpack(planes.handle, *[ctypes.c_void_p(t.data_ptr()) for t in out], _stream()),
           "moe_w4_unpack")
    return out


def moe_w4_pack_nvfp4(gu_codes, gu_scales, gu_scale2, dn_codes, dn_scales, dn_scale2):
    """Canonical NVFP4 device planes -> Planes. Shapes: gu_codes [E, 2I, K/2] uint8 (two e2m1
    codes per byte, low nibble = even element), gu_scales [E, 2I, K/16] uint8 (E4M3FN),
    gu_scale2 [E, 2] float32 (gate, up), dn_codes [E, K, I/2], dn_scales [E, K, I/16],
    dn_scale2 [E] float32."""
    E, two_i, k2 = gu_codes.shape
    K, I = k2 * 2, two_i // 2
    if tuple(gu_scales.shape) != (E, 2 * I, K // 16) or tuple(dn_codes.shape) != (E, K, I // 2) \
            or tuple(dn_scales.shape) != (E, K, I // 16) or tuple(gu_scale2.shape) != (E, 2) \
            or tuple(dn_scale2.shape) != (E,):
        raise ValueError("inconsistent plane shapes")
    h = ctypes.c_void_p()
    _check(_lib().moe_w4_pack_nvfp4(
        E, K, I, _dev(gu_codes, torch.uint8, "gu_codes"), _dev(gu_scales, torch.uint8, "gu_scales"),
        _dev(gu_scale2, torch.float32, "gu_scale2"), _dev(dn_codes, torch.uint8, "dn_codes"),
        _dev(dn_scales, torch.uint8, "dn_scales"), _dev(dn_scale2, torch.float32, "dn_scale2"),
        _stream(), ctypes.byref(h)), "moe_w4_pack_nvfp4")
    return Planes(h, E, K, I)


def moe_w4_unpack_nvfp4(planes):
    E, K, I = planes.E, planes.K, planes.I
    d = torch.device("cuda")
    out = (torch.empty((E, 2 * I, K // 2), dtype=torch.uint8, device=d),
           torch.empty((E, 2 * I, K // 16), dtype=torch.uint8, device=d),
           torch.empty((E, 2), dtype=torch.float32, device=d),
           torch.empty((E, K, I // 2), dtype=torch.uint8, device=d),
           torch.empty((E, K, I // 16), dtype=torch.uint8, device=d),
           torch.empty((E,), dtype=torch.float32, device=d))
    _check(_lib().moe_w4_unpack_nvfp4(planes.handle, *[ctypes.c_void_p(t.data_ptr()) for t in out], _stream()),
           "moe_w4_unpack_nvfp4")
    return out


def moe_w4_forward(planes, x, topk_ids, topk_w, out_dtype=OUT_BF16, workspace=None, path=PATH_AUTO, y=None):
    """moe_w2_forward on FP4 planes (moe_w4_pack or moe_w4_pack_nvfp4)."""
    T, K = x.shape
    top_k = topk_ids.shape[1]
    if workspace is None:
        workspace = alloc_workspace(planes, T, top_k)
    if y is None:
        y = torch.empty((T, K), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device="cuda")
    _check(_lib().moe_w4_forward(planes.handle, T, top_k, _dev(x, torch.bfloat16, "x"),
                                 _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_w, torch.float32, "topk_w"),
                                 ctypes.c_void_p(y.data_ptr()), int(out_dtype), _dev(workspace, torch.uint8, "workspace"),
                                 workspace.numel(), int(path), _stream()), "moe_w4_forward")
    return y


def moe_w2_unpack(planes):
    E, K, I = planes.E, planes.K, planes.I
    d = torch.device("cuda")
    out = (torch.empty((E, 2 * I, K // 4), dtype=torch.uint8, device=d),
           torch.empty((E, 2 * I, K // 32), dtype=torch.uint8, device=d),
           torch.empty((E, K, I // 4), dtype=torch.uint8, device=d),
           torch.empty((E, K, I // 32), dtype=torch.uint8, device=d))
    _check(_lib().moe_w2_unpack(planes.handle, *[ctypes.c_void_p(t.data_ptr()) for t in out], _stream()),
           "moe_w2_unpack")
    return out


def moe_w2_workspace_bytes(planes, T, top_k):
    return int(_lib().moe_w2_workspace_bytes(planes.handle, int(T), int(top_k)))


def alloc_workspace(planes, T, top_k):
    n = moe_w2_workspace_bytes(planes, T, top_k)
    if n == 0:
        raise MoeW2Error(-1, "moe_w2_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def moe_w2_route(topk_ids, E):
    """topk_ids [T, top_k] int32 (device) -> (offsets [E+1] int32, perm [T*top_k] int32)."""
    T, top_k = topk_ids.shape
    ws = torch.empty(int(_lib().moe_w2_route_workspace_bytes(E, T, top_k)), dtype=torch.uint8, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(max(T * top_k, 1), dtype=torch.int32, device="cuda")
    _check(_lib().moe_w2_route(E, T, top_k, _dev(topk_ids, torch.int32, "topk_ids"), ctypes.c_void_p(offsets.data_ptr()),
                               ctypes.c_void_p(perm.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                               _stream()), "moe_w2_route")
    return offsets, perm[:T * top_k]


def moe_w2_forward(planes, x, topk_ids, topk_w, out_dtype=OUT_BF16, workspace=None, path=PATH_AUTO, y=None):
    """x [T, K] bf16, topk_ids [T, top_k] int32, topk_w [T, top_k] fp32 (device) -> y [T, K]."""
    T, K = x.shape
    top_k = topk_ids.shape[1]
    if workspace is None:
        workspace = alloc_workspace(planes, T, top_k)
    if y is None:
        y = torch.empty((T, K), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device="cuda")
    _check(_lib().moe_w2_forward(planes.handle, T, top_k, _dev(x, torch.bfloat16, "x"),
                                 _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_w, torch.float32, "topk_w"),
                                 ctypes.c_void_p(y.data_ptr()), int(out_dtype), _dev(workspace, torch.uint8, "workspace"),
                                 workspace.numel(), int(path), _stream()), "moe_w2_forward")
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20   # MOE_W2_NOALLOC_SCRATCH_BYTES


def moe_w2_forward_noalloc(planes, x, topk_ids, topk_w, y, out_dtype=OUT_BF16, path=PATH_AUTO):
    """moe_w2_forward with the library's own per-GPU scratch as workspace: allocates nothing (y is
    the caller's, preallocated). Calls that may overlap on one GPU race on that scratch."""
    T, _ = x.shape
    _check(_lib().moe_w2_forward_noalloc(planes.handle, T, topk_ids.shape[1], _dev(x, torch.bfloat16, "x"),
                                         _dev(topk_ids, torch.int32, "topk_ids"), _dev(topk_w, torch.float32, "topk_w"),
                                         ctypes.c_void_p(y.data_ptr()), int(out_dtype), int(path), _stream()),
           "moe_w2_forward_noalloc")
    return y


def moe_w2_forward_stage(stage, planes, x, topk_ids, topk_w, y, workspace, out_dtype=OUT_BF16, path=PATH_AUTO):
    """One stage of moe_w2_forward (all tensors preallocated on the device); stages 0..3 in order
    on one stream and workspace are exactly moe_w2_forward."""
    T, _ = x.shape
    _check(_lib().moe_w2_forward_stage(planes.handle, int(stage), T, topk_ids.shape[1], ctypes.c_void_p(x.data_ptr()),
                                       ctypes.c_void_p(topk_ids.data_ptr()), ctypes.c_void_p(topk_w.data_ptr()),
                                       ctypes.c_void_p(y.data_ptr()), int(out_dtype), ctypes.c_void_p(workspace.data_ptr()),
                                       workspace.numel(), int(path), _stream()), "moe_w2_forward_stage")


def moe_w2_read_counters(workspace):
    inv, ovf = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib().moe_w2_read_counters(_dev(workspace, torch.uint8, "workspace"), ctypes.byref(inv), ctypes.byref(ovf),
                                       _stream()), "moe_w2_read_counters")
    return inv.value, ovf.value


def moe_w2_planes_create(S, K, I):
    """Planes of S empty expert slots (contents unspecified until moe_w2_pack_slot)."""
    h = ctypes.c_void_p()
    _check(_lib().moe_w2_planes_create(int(S), int(K), int(I), _stream(), ctypes.byref(h)), "moe_w2_planes_create")
    return Planes(h, S, K, I)


def moe_w2_pack_slot(planes, slot, gu_codes, gu_scales, dn_codes, dn_scales):
    """One expert's canonical device planes (gu_codes [2I, K/4], gu_scales [2I, K/32], dn_codes [K, I/4],
    dn_scales [K, I/32], uint8) into slot `slot`."""
    K, I = planes.K, planes.I
    if tuple(gu_codes.shape) != (2 * I, K // 4) or tuple(gu_scales.shape) != (2 * I, K // 32) \
            or tuple(dn_codes.shape) != (K, I // 4) or tuple(dn_scales.shape) != (K, I // 32):
        raise ValueError("inconsistent plane shapes")
    _check(_lib().moe_w2_pack_slot(planes.handle, int(slot), _dev(gu_codes, torch.uint8, "gu_codes"),
                                   _dev(gu_scales, torch.uint8, "gu_scales"), _dev(dn_codes, torch.uint8, "dn_codes"),
                                   _dev(dn_scales, torch.uint8, "dn_scales"), _stream()), "moe_w2_pack_slot")


def moe_w2_forward_slots(planes, slot_of_expert, x, topk_ids, topk_w, out_dtype=OUT_BF16, workspace=None,
                         path=PATH_AUTO, y=None):
    """moe_w2_forward over experts reached through slot_of_expert [E] int32 (device; entries outside
    [0, planes.E) = not resident)."""
    T, K = x.shape
    top_k = topk_ids.shape[1]
    E = slot_of_expert.shape[0]
    if workspace is None:
        workspace = alloc_workspace(planes, T, top_k)
    if y is None:
        y = torch.empty((T, K), dtype=torch.bfloat16 if out_dtype == OUT_BF16 else torch.float32, device="cuda")
    _check(_lib().moe_w2_forward_slots(planes.handle, E, _dev(slot_of_expert, torch.int32, "slot_of_expert"), T, top_k,
                                       _dev(x, torch.bfloat16, "x"), _dev(topk_ids, torch.int32, "topk_ids"),
                                       _dev(topk_w, torch.float32, "topk_w"), ctypes.c_void_p(y.data_ptr()),
                                       int(out_dtype), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
                                       int(path), _stream()), "moe_w2_forward_slots")
    return y


def moe_w2_read_miss_counter(workspace):
    m = ctypes.c_int64(0)
    _check(_lib().moe_w2_read_miss_counter(_dev(workspace, torch.uint8, "workspace"), ctypes.byref(m), _stream()),
           "moe_w2_read_miss_counter")
    return m.value


def nvfp4_to_w2(e2m1, e4m3, scale_2, codes=None, scales=None):
    """e2m1 [n, R, C/2] uint8, e4m3 [n, R, C/16] uint8, scale_2 [n] fp32 (device) ->
    (codes [n, R, C/4], scales [n, R, C/32])."""
    n, R, half_c = e2m1.shape
    C = half_c * 2
    if codes is None:
        codes = torch.empty((n, R, C // 4), dtype=torch.uint8, device="cuda")
    if scales is None:
        scales = torch.empty((n, R, C // 32), dtype=torch.uint8, device="cuda")
    _check(_lib().nvfp4_to_w2(n, R, C, _dev(e2m1, torch.uint8, "e2m1"), _dev(e4m3, torch.uint8, "e4m3"),
                              _dev(scale_2, torch.float32, "scale_2"), _dev(codes, torch.uint8, "codes"),
                              _dev(scales, torch.uint8, "scales"), _stream()), "nvfp4_to_w2")
    return codes, scales


def fp8_block128_to_w2(e4m3, bscale, codes=None, scales=None):
    """e4m3 [n, R, C] uint8, bscale [n, R/128, C/128] fp32 (device) -> (codes [n, R, C/4], scales [n, R, C/32])."""
    n, R, C = e4m3.shape
    if codes is None:
        codes = torch.empty((n, R, C // 4), dtype=torch.uint8, device="cuda")
    if scales is None:
        scales = torch.empty((n, R, C // 32), dtype=torch.uint8, device="cuda")
    _check(_lib().fp8_block128_to_w2(n, R, C, _dev(e4m3, torch.uint8, "e4m3"), _dev(bscale, torch.float32, "bscale"),
                                     _dev(codes, torch.uint8, "codes"), _dev(scales, torch.uint8, "scales"), _stream()),
           "fp8_block128_to_w2")
    return codes, scales


def mxfp4_to_w2(e2m1, ue8m0, codes=None, scales=None):
    """e2m1 [n, R, C/2] uint8, ue8m0 [n, R, C/32] uint8 (device) -> (codes [n, R, C/4], scales [n, R, C/32])."""
    n, R, half_c = e2m1.shape
    C = half_c * 2
    if codes is None:
        codes = torch.empty((n, R, C // 4), dtype=torch.uint8, device="cuda")
    if scales is None:
        scales = torch.empty((n, R, C // 32), dtype=torch.uint8, device="cuda")
    _check(_lib().mxfp4_to_w2(n, R, C, _dev(e2m1, torch.uint8, "e2m1"), _dev(ue8m0, torch.uint8, "ue8m0"),
                              _dev(codes, torch.uint8, "codes"), _dev(scales, torch.uint8, "scales"), _stream()),
           "mxfp4_to_w2")
    return codes, scales


def moe_w2_codebook_sweep(x, codebooks):
    """Sign-bias diagnostic. x [n, R, C] float32 (device); codebooks [M, 4] float32 (host, numpy or
    CPU tensor, each row strictly ascending). Returns (stats [n, M, 4] float64 = sse, err, rel_rms,
    bias; moments [n, 2] float64 = sum x^2, sum x; best [n, 2] int32 = least-sse symmetric and
    asymmetric codebook, -1 if none), all on the device."""
    import numpy as np
    n, R, C = x.shape
    cb = np.ascontiguousarray(codebooks.cpu().numpy() if isinstance(codebooks, torch.Tensor) else codebooks,
                              dtype=np.float32)
    if cb.ndim != 2 or cb.shape[1] != 4:
        raise ValueError("codebooks must be [M, 4]")
    M = cb.shape[0]
    stats = torch.empty((n, M, 4), dtype=torch.float64, device="cuda")
    moments = torch.empty((n, 2), dtype=torch.float64, device="cuda")
    best = torch.empty((n, 2), dtype=torch.int32, device="cuda")
    _check(_lib().moe_w2_codebook_sweep(n, R, C, _dev(x, torch.float32, "x"), M,
                                        cb.ctypes.data_as(ctypes.c_void_p), _dev(stats, torch.float64, "stats"),
                                        _dev(moments, torch.float64, "moments"), _dev(best, torch.int32, "best"),
                                        _stream()), "moe_w2_codebook_sweep")
    return stats, moments, best
