"""Sign-bias diagnostic of 2-bit codebooks (test infrastructure; see oracle/__init__).

What it measures (README, bullet "2-bit expert planes - the sign-bias finding"; vLLM-Moet
article, section "Sign symmetry, not error size, is what collapses naive 2-bit experts"): for each
tensor and each candidate 4-value codebook, the relative RMS error and the mean bias of the tensor
quantized with that codebook and power-of-two block-32 scales; and which symmetric and which
asymmetric candidate has the least squared error.

Two implementations of one definition (written out in ``codebook_sweep.c``'s header):

* ``block_choice_fraction`` - pure Python with exact rationals: every candidate exponent's squared
  error evaluated exactly, nearest codes found by exact distance comparison. For pins.
* ``codebook_sweep`` - ctypes wrapper of ``codebook_sweep.c`` (float64, element order, no fused
  operations), for tensors of any size.
"""
import ctypes
import os
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsweep_oracle.so")


def build(quiet=True):
    """Compile codebook_sweep.c into libsweep_oracle.so (gcc, OpenMP, no floating-point contraction)."""
    import subprocess
    src = os.path.join(_HERE, "codebook_sweep.c")
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", "-std=c99", src, "-lm",
           "-o", LIB_PATH]
    subprocess.run(cmd, check=True, capture_output=quiet)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        src = os.path.join(_HERE, "codebook_sweep.c")
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(src):
            build()
        _lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        _lib.oracle_block_choice.argtypes = [P, P, P, P]
        _lib.oracle_block_choice.restype = ctypes.c_int
        _lib.oracle_codebook_sweep.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_int, P,
                                               P, P, P, ctypes.c_int]
        _lib.oracle_codebook_sweep.restype = None
    return _lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def block_choice_c(x32, q):
    """(exponent, sse, err) of one block of 32 fp32 values under codebook q (4 fp32), C version."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    sse, err = ctypes.c_double(), ctypes.c_double()
    e = _load().oracle_block_choice(_ptr(x32), _ptr(q), ctypes.byref(sse), ctypes.byref(err))
    return e, sse.value, err.value


def codebook_sweep(x, codebooks, nthreads=None):
    """x: float32 [n][R][C] (C a multiple of 32); codebooks: float32 [M][4], strictly ascending.
    Returns (stats [n][M][4] = sse, err, rel_rms, bias; moments [n][2] = sum x^2, sum x;
    best [n][2] = least-sse symmetric and asymmetric codebook index, -1 if none)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    cb = np.ascontiguousarray(codebooks, dtype=np.float32)
    n, R, C = x.shape
    M = cb.shape[0]
    assert C % 32 == 0 and cb.shape[1] == 4
    stats = np.zeros((n, M, 4), np.float64)
    moments = np.zeros((n, 2), np.float64)
    best = np.zeros((n, 2), np.int32)
    _load().oracle_codebook_sweep(n, R, C, _ptr(x), M, _ptr(cb), _ptr(stats), _ptr(moments), _ptr(best),
                                  nthreads or os.cpu_count() or 1)
    return stats, moments, best


def _exp_top(amax, qmax):
    """Smallest e in [-127, 127] with qmax 2^e >= amax; -127 for amax = 0 (exact rationals)."""
    if amax == 0:
        return -127
    e = -127
    while e < 127 and qmax * Fraction(2) ** e < amax:
        e += 1
    return e


def nearest_code_fraction(x, q, e):
    """Code index of exact rational x at scale 2^e: nearest value; halfway -> smaller magnitude;
    equal magnitudes (x = 0) -> the side of x's sign (x passed as (Fraction, sign_bit))."""
    xv, neg = x
    s = Fraction(2) ** e
    d = [abs(xv - qk * s) for qk in q]
    dmin = min(d)
    cand = [k for k in range(4) if d[k] == dmin]
    if len(cand) == 1:
        return cand[0]
    a, b = cand                       # two adjacent codes, x halfway
    if abs(q[a]) != abs(q[b]):
        return a if abs(q[a]) < abs(q[b]) else b
    return a if neg else b            # a < b: a is the negative one


def block_choice_fraction(x32, q, exps=None):
    """Exact (exponent, sse, err) of one block: sse and err as Fractions. exps defaults to the
    ten-exponent window; pass range(-127, 128) for the full scan."""
    xs = [(Fraction(float(v)), bool(np.signbit(v))) for v in np.asarray(x32, np.float32)]
    qf = [Fraction(float(v)) for v in np.asarray(q, np.float32)]
    amax = max(abs(v) for v, _ in xs)
    if exps is None:
        ec = _exp_top(amax, max(abs(qf[0]), abs(qf[3])))
        exps = [e for e in range(ec - 7, ec + 3) if -127 <= e <= 127]
    best = None
    for e in exps:
        s = Fraction(2) ** e
        vals = [qf[nearest_code_fraction(x, qf, e)] * s for x in xs]
        sse = sum((v - x[0]) ** 2 for v, x in zip(vals, xs))
        if best is None or sse < best[1]:
            best = (e, sse, sum(v - x[0] for v, x in zip(vals, xs)))
    return best
