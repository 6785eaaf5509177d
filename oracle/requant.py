"""NVFP4 -> 2-bit re-quantizer (test infrastructure; see oracle/__init__).

Two implementations of the same definition:

* ``requant_block_fraction`` - pure Python with exact rationals, scanning all 255 UE8M0 exponents
  and evaluating SSE(e) = sum_i (|x_i| - q_i 2^e)^2 term by term. Slow; for tiny inputs and for
  pinning the C version.
* ``requant_rows`` / ``nvfp4_to_w2`` - ctypes wrapper of ``requant_exact.c`` (exact integer
  arithmetic, all 255 exponents or the 7-exponent window), for large inputs.

Definition ("The v0.24.0 port", section "Our hooks", modelopt.py bullet: exact f64 dequant of
e2m1 x e4m3 block-16 x per-tensor scale_2, UE8M0 block-32 output scales absorbing scale_2; README
opening paragraph; readings where the pages are silent):
  * the exponent minimises the exact squared error over the block; equal errors -> lower exponent;
  * each element takes the nearer magnitude of {1, 4} * 2^e; exactly halfway (|x| = 2.5 * 2^e)
    -> 1, which keeps the map odd-symmetric;
  * the sign of an element is the sign bit of the exact product (so -0 is negative); negative
    elements get code 0 (-4) or 1 (-1), the others 2 (+1) or 3 (+4);
  * scale byte = e + 127; canonical packing of codes as in ``formats``.
"""
import ctypes
import math
import os
from fractions import Fraction

import numpy as np

from .formats import e2m1_value, e4m3_value

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librequant_oracle.so")


def build(quiet=True):
    """Compile requant_exact.c into librequant_oracle.so (gcc, OpenMP)."""
    import subprocess
    src = os.path.join(_HERE, "requant_exact.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", src, "-o", LIB_PATH]
    subprocess.run(cmd, check=True, capture_output=quiet)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        lib.oracle_requant_block.argtypes = [u8p, u8p, ctypes.c_float, u8p, u8p, ctypes.c_int]
        lib.oracle_requant_block.restype = ctypes.c_int
        lib.oracle_requant_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, u8p, u8p, ctypes.c_float,
                                            u8p, u8p, ctypes.c_int, ctypes.c_int]
        lib.oracle_requant_rows.restype = ctypes.c_int
        f32p = ctypes.POINTER(ctypes.c_float)
        lib.oracle_fp8_block128_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, u8p, f32p, u8p, u8p,
                                                 ctypes.c_int, ctypes.c_int]
        lib.oracle_fp8_block128_rows.restype = ctypes.c_int
        lib.oracle_mxfp4_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, u8p, u8p, u8p, u8p, ctypes.c_int, ctypes.c_int]
        lib.oracle_mxfp4_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


# ---------------------------------------------------------------------------------------------
# exact rational reference
# ---------------------------------------------------------------------------------------------

def nvfp4_block_values(e2m1_bytes, e4m3_bytes, scale2):
    """Dequantize one 32-element block: returns (negative flags, exact magnitudes as Fractions).

    e2m1_bytes: 16 bytes, low nibble = even element; e4m3_bytes: 2 bytes (elements 0-15, 16-31);
    scale2: the fp32 per-tensor scale (a float that is exactly an fp32 value).
    The product is formed in f64 (exact: at most 30 significant bits) and its sign bit taken.
    """
    s2 = float(np.float32(scale2))
    negs, mags = [], []
    for k in range(32):
        nib = (int(e2m1_bytes[k // 2]) >> (4 * (k & 1))) & 15
        v = e2m1_value(nib) * e4m3_value(int(e4m3_bytes[k // 16])) * s2
        negs.append(math.copysign(1.0, v) < 0)
        mags.append(Fraction(abs(v)))
    return negs, mags


def fp8_block_values(e4m3_bytes, scale):
    """One 32-element block of FP8 block-quant weights ("The v0.24.0 port", section "Our hooks",
    fp8.py bullet: fp8 + fp32 block-128 scales re-quantized in float64 math): x = e4m3 * scale,
    formed in f64 (exact: at most 4 + 24 significant bits). Returns (negative flags, exact
    magnitudes as Fractions)."""
    s = float(np.float32(scale))
    negs, mags = [], []
    for b in e4m3_bytes:
        v = e4m3_value(int(b)) * s
        negs.append(math.copysign(1.0, v) < 0)
        mags.append(Fraction(abs(v)))
    return negs, mags


def mxfp4_block_values(e2m1_bytes, scale_byte):
    """One 32-element MXFP4 block (README: the FP4 checkpoints' experts): x = e2m1 * 2^(b-127),
    exact. Returns (negative flags, exact magnitudes)."""
    t = Fraction(2) ** (int(scale_byte) - 127)
    negs, mags = [], []
    for k in range(32):
        v = e2m1_value((int(e2m1_bytes[k // 2]) >> (4 * (k & 1))) & 15)
        negs.append(math.copysign(1.0, v) < 0)
        mags.append(Fraction(abs(v)) * t)
    return negs, mags


def requant_block_fraction(negs, mags):
    """Full scan over e in -127..127 with exact rational SSE. Returns (codes[32], scale byte)."""
    best_e, best_sse = None, None
    for e in range(-127, 128):
        t = Fraction(2) ** e
        half = Fraction(5, 2) * t
        sse = Fraction(0)
        for m in mags:
            q = 4 if m > half else 1
            d = m - q * t
            sse += d * d
        if best_sse is None or sse < best_sse:
            best_e, best_sse = e, sse
    t = Fraction(2) ** best_e
    codes = []
    for neg, m in zip(negs, mags):
        q4 = m > Fraction(5, 2) * t
        codes.append((0 if q4 else 1) if neg else (3 if q4 else 2))
    return codes, best_e + 127


def requant_block_int(negs, mags):
    """The same full scan as requant_block_fraction, in Python integers (about twenty times
    faster, for pinning the C version on many blocks). Every magnitude is a dyadic rational, so
    with L the largest of 127 and the magnitudes' denominator exponents, X_i = |x_i| * 2^L and the
    step T = 2^(e+L) of every candidate e >= -127 are integers; SSE(e) * 4^L is then the integer
    sum of (X_i - q_i T)^2, compared exactly across all 255 exponents (equal -> lower e)."""
    L = 127
    for m in mags:
        d = m.denominator
        if d & (d - 1):
            raise ValueError("magnitude is not a dyadic rational")
        L = max(L, d.bit_length() - 1)
    X = [m.numerator << (L - (m.denominator.bit_length() - 1)) for m in mags]
    best_e, best_sse = None, None
    for e in range(-127, 128):
        T = 1 << (e + L)
        sse = 0
        for x in X:
            q = 4 if 2 * x > 5 * T else 1
            d = x - q * T
            sse += d * d
        if best_sse is None or sse < best_sse:
            best_e, best_sse = e, sse
    T = 1 << (best_e + L)
    codes = []
    for neg, x in zip(negs, X):
        q4 = 2 * x > 5 * T
        codes.append((0 if q4 else 1) if neg else (3 if q4 else 2))
    return codes, best_e + 127


# ---------------------------------------------------------------------------------------------
# exact integer implementation (C)
# ---------------------------------------------------------------------------------------------

def requant_block_c(e2m1_bytes, e4m3_bytes, scale2, window=False):
    """One block through the C implementation -> (codes[32] list, scale byte)."""
    lib = _load()
    a = np.ascontiguousarray(e2m1_bytes, dtype=np.uint8)
    b = np.ascontiguousarray(e4m3_bytes, dtype=np.uint8)
    codes = np.zeros(8, dtype=np.uint8)
    sc = np.zeros(1, dtype=np.uint8)
    rc = lib.oracle_requant_block(_ptr(a), _ptr(b), ctypes.c_float(float(np.float32(scale2))),
                                  _ptr(codes), _ptr(sc), int(bool(window)))
    if rc:
        raise ValueError("invalid NVFP4 input (NaN scale)")
    out = [(int(codes[k // 4]) >> (2 * (k % 4))) & 3 for k in range(32)]
    return out, int(sc[0])


def requant_rows(e2m1, e4m3, scale2, window=True, nthreads=None):
    """Rows of one tensor: e2m1 [rows, C/2], e4m3 [rows, C/16], scalar scale2 ->
    (codes [rows, C/4], scales [rows, C/32]) in the canonical layout."""
    lib = _load()
    e2m1 = np.ascontiguousarray(e2m1, dtype=np.uint8)
    e4m3 = np.ascontiguousarray(e4m3, dtype=np.uint8)
    rows, half_c = e2m1.shape
    C = half_c * 2
    if e4m3.shape != (rows, C // 16) or C % 32:
        raise ValueError("shape mismatch")
    codes = np.zeros((rows, C // 4), dtype=np.uint8)
    scales = np.zeros((rows, C // 32), dtype=np.uint8)
    nt = nthreads or os.cpu_count() or 1
    rc = lib.oracle_requant_rows(rows, C, _ptr(e2m1), _ptr(e4m3), ctypes.c_float(float(np.float32(scale2))),
                                 _ptr(codes), _ptr(scales), int(bool(window)), int(nt))
    if rc:
        raise ValueError("invalid NVFP4 input (NaN e4m3 byte or NaN/Inf scale_2)")
    return codes, scales


def nvfp4_to_w2(e2m1, e4m3, scale2, window=True, nthreads=None):
    """Tensors: e2m1 [n, R, C/2], e4m3 [n, R, C/16], scale2 [n] -> codes [n, R, C/4], scales [n, R, C/32]."""
    e2m1 = np.asarray(e2m1, dtype=np.uint8)
    n, R, half_c = e2m1.shape
    codes = np.zeros((n, R, half_c // 2), dtype=np.uint8)
    scales = np.zeros((n, R, half_c // 16), dtype=np.uint8)
    for i in range(n):
        codes[i], scales[i] = requant_rows(e2m1[i], e4m3[i], scale2[i], window, nthreads)
    return codes, scales


def fp8_block128_to_w2(e4m3, scales, window=True, nthreads=None):
    """FP8 block-quant tensors: e4m3 [n, R, C] bytes, scales [n, R/128, C/128] fp32 ->
    codes [n, R, C/4], scale bytes [n, R, C/32] (the exact search of this module per 32-block)."""
    lib = _load()
    e4m3 = np.ascontiguousarray(e4m3, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    n, R, C = e4m3.shape
    if R % 128 or C % 128 or scales.shape != (n, R // 128, C // 128):
        raise ValueError("shape mismatch")
    codes = np.zeros((n, R, C // 4), dtype=np.uint8)
    out = np.zeros((n, R, C // 32), dtype=np.uint8)
    nt = nthreads or os.cpu_count() or 1
    f32p = ctypes.POINTER(ctypes.c_float)
    for i in range(n):
        rc = lib.oracle_fp8_block128_rows(R, C, 0, _ptr(e4m3[i]), scales[i].ctypes.data_as(f32p), _ptr(codes[i]),
                                          _ptr(out[i]), int(bool(window)), int(nt))
        if rc:
            raise ValueError("invalid FP8 input (NaN e4m3 byte or non-finite scale)")
    return codes, out


def mxfp4_to_w2(e2m1, ue8m0, window=True, nthreads=None):
    """MXFP4 tensors: e2m1 [n, R, C/2], ue8m0 [n, R, C/32] -> codes [n, R, C/4], scale bytes [n, R, C/32]."""
    lib = _load()
    e2m1 = np.ascontiguousarray(e2m1, dtype=np.uint8)
    ue8m0 = np.ascontiguousarray(ue8m0, dtype=np.uint8)
    n, R, half_c = e2m1.shape
    C = half_c * 2
    if ue8m0.shape != (n, R, C // 32):
        raise ValueError("shape mismatch")
    codes = np.zeros((n, R, C // 4), dtype=np.uint8)
    out = np.zeros((n, R, C // 32), dtype=np.uint8)
    nt = nthreads or os.cpu_count() or 1
    for i in range(n):
        if lib.oracle_mxfp4_rows(R, C, _ptr(e2m1[i]), _ptr(ue8m0[i]), _ptr(codes[i]), _ptr(out[i]),
                                 int(bool(window)), int(nt)):
            raise ValueError("invalid MXFP4 input (scale byte 255)")
    return codes, out


def requant_block_c_fp8(e4m3_bytes, scale, window=False):
    """One FP8 block through the C implementation (a [128, 128] tile holding the block in row 0)."""
    e = np.zeros((1, 128, 128), np.uint8)
    e[0, 0, :32] = np.asarray(e4m3_bytes, np.uint8)
    codes, sc = fp8_block128_to_w2(e, np.full((1, 1, 1), scale, np.float32), window, 1)
    return [(int(codes[0, 0, k // 4]) >> (2 * (k % 4))) & 3 for k in range(32)], int(sc[0, 0, 0])


def requant_block_c_mxfp4(e2m1_bytes, scale_byte, window=False):
    codes, sc = mxfp4_to_w2(np.asarray(e2m1_bytes, np.uint8).reshape(1, 1, 16), np.full((1, 1, 1), scale_byte, np.uint8),
                            window, 1)
    return [(int(codes[0, 0, k // 4]) >> (2 * (k % 4))) & 3 for k in range(32)], int(sc[0, 0, 0])
