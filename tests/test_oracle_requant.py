"""Pins for the re-quantizer oracle (oracle.requant) against closed forms, brute force and
invariants; the C implementation is also pinned against the exact rational reference."""
from fractions import Fraction
import math
import os

import numpy as np
import pytest

from oracle import formats, requant
import workloads

E2M1_POS = {1.0: 0x2, 4.0: 0x6}  # e2m1 nibbles of +1 and +4


def _block_bytes(nibbles):
    nib = np.asarray(nibbles, dtype=np.uint8)
    return (nib[0::2] | (nib[1::2] << 4)).astype(np.uint8)


def test_nvfp4_dequant_exact_in_f64():
    """The f64 product e2m1 * e4m3 * scale_2 equals the exact rational product (pages: f64-exact
    dequant, 'The v0.24.0 port', modelopt.py bullet)."""
    rng = np.random.default_rng(11)
    s2s = [np.float32(v) for v in rng.uniform(1e-3, 1e-2, 200)]
    s2s += [np.float32(v) for v in (1.0, 3.0e38, 1.4e-45, 1.1754942e-38, 0.3333333)]
    e4 = [b for b in range(256) if (b & 0x7F) != 0x7F]
    for s2 in s2s:
        fs2 = Fraction(float(s2))
        for b in e4:
            f4 = Fraction(formats.e4m3_value(b))
            for nib in range(16):
                f2 = Fraction(formats.e2m1_value(nib))
                exact = f2 * f4 * fs2
                got = formats.e2m1_value(nib) * formats.e4m3_value(b) * float(s2)
                assert Fraction(got) == exact


def _random_blocks(rng, n, full_range=False):
    e2m1 = rng.integers(0, 256, size=(n, 16), dtype=np.uint8)
    if full_range:
        e4m3 = rng.integers(0, 256, size=(n, 2), dtype=np.uint8)
        e4m3[(e4m3 & 0x7F) == 0x7F] = 0x38
        s2 = np.float32(2.0) ** rng.integers(-140, 120, size=n).astype(np.float32)
        s2 = (s2 * rng.uniform(1, 2, size=n).astype(np.float32)).astype(np.float32)
    else:
        e4m3 = rng.integers(0x18, 0x59, size=(n, 2), dtype=np.uint8)
        s2 = rng.uniform(1e-3, 1e-2, size=n).astype(np.float32)
    return e2m1, e4m3, s2


def test_c_matches_rational_reference():
    """Exact-integer C scan (all 255 exponents) == rational full scan, on workload-distributed
    blocks, blocks over the whole e4m3 / fp32 range, and constructed edge blocks."""
    rng = np.random.default_rng(5)
    cases = []
    a, b, s = _random_blocks(rng, 60)
    cases += [(a[i], b[i], s[i]) for i in range(60)]
    a, b, s = _random_blocks(rng, 60, full_range=True)
    cases += [(a[i], b[i], s[i]) for i in range(60)]
    z = np.zeros(16, np.uint8)
    cases.append((z, np.array([0x38, 0x38], np.uint8), np.float32(1.0)))          # all +0
    cases.append((np.full(16, 0x88, np.uint8), np.array([0x38, 0x38], np.uint8), np.float32(1.0)))  # all -0
    one = z.copy(); one[3] = 0x70
    cases.append((one, np.array([0x01, 0x7E], np.uint8), np.float32(1e-30)))      # single nonzero
    for e2m1, e4m3, s2 in cases:
        negs, mags = requant.nvfp4_block_values(e2m1, e4m3, s2)
        want = requant.requant_block_fraction(negs, mags)
        got_full = requant.requant_block_c(e2m1, e4m3, s2, window=False)
        got_win = requant.requant_block_c(e2m1, e4m3, s2, window=True)
        assert got_full == want
        assert got_win == want


@pytest.mark.slow
def test_window_equals_full_scan_many_blocks():
    """The 7-exponent window [top-6, top] finds the same optimum as the 255-exponent scan."""
    rng = np.random.default_rng(6)
    for full_range in (False, True):
        a, b, s = _random_blocks(rng, 20000, full_range)
        for i in range(0, 20000, 2000):
            # rows of one 'tensor' share scale_2: use blocks i..i+1999 with scale s[i]
            e2m1 = a[i:i + 2000].reshape(2000, 16)
            e4m3 = b[i:i + 2000].reshape(2000, 2)
            cf, sf = requant.requant_rows(e2m1, e4m3, s[i], window=False)
            cw, sw = requant.requant_rows(e2m1, e4m3, s[i], window=True)
            assert np.array_equal(cf, cw) and np.array_equal(sf, sw)


def _codes_of(e2m1, e4m3, s2, window=True):
    codes, scales = requant.requant_rows(np.asarray(e2m1, np.uint8)[None], np.asarray(e4m3, np.uint8)[None], s2, window)
    return formats.unpack_codes(codes)[0].tolist(), int(scales[0, 0])


def test_single_magnitude_block_prefers_lower_exponent():
    """All |x| = 2^a: e = a (all +-1) and e = a-2 (all +-4) both reconstruct exactly (SSE 0);
    equal errors go to the lower exponent -> e = a-2 with codes +-4 (workload statement: ties
    break to the lower exponent)."""
    nib = [0x2 if k % 3 else 0xA for k in range(32)]           # +1 / -1, e2m1
    codes, sc = _codes_of(_block_bytes(nib), [0x38, 0x38], np.float32(2.0 ** -5))  # |x| = 2^-5
    assert sc == 127 - 5 - 2
    assert codes == [3 if n == 0x2 else 0 for n in nib]


def test_all_zero_block():
    """All-zero block: SSE = 32 * 4^e is minimised at e = -127 (byte 0); codes follow the sign
    bit (+0 -> +1 = code 2, -0 -> -1 = code 1)."""
    nib = [0x0 if k % 2 else 0x8 for k in range(32)]
    codes, sc = _codes_of(_block_bytes(nib), [0x38, 0x38], np.float32(1.0))
    assert sc == 0
    assert codes == [2 if n == 0 else 1 for n in nib]


def test_midpoint_goes_to_smaller_magnitude():
    """Block: 16 elements 2.5 (e2m1 2 x e4m3 1.25), 15 elements 4 and one 6 (e4m3 1.0), scale_2 1.
    By hand: SSE(e=0) = 16*1.5^2 + 0 + 2^2 = 40, SSE(1) = 16*0.5^2 + 15*2^2 + 2^2 = 68,
    SSE(-1) = 16*0.5^2 + 15*2^2 + 4^2 = 80, farther exponents are worse, so e = 0. Each 2.5 sits
    exactly at 2.5 * 2^0 and takes magnitude 1 (code 2); 4 and 6 take magnitude 4 (code 3)."""
    nib = [0x4] * 16 + [0x6] * 15 + [0x7]
    e2m1 = _block_bytes(nib)
    e4m3 = np.array([0x3A, 0x38], np.uint8)
    assert formats.e4m3_value(0x3A) == 1.25
    want = ([2] * 16 + [3] * 16, 127)
    negs, mags = requant.nvfp4_block_values(e2m1, e4m3, np.float32(1.0))
    assert requant.requant_block_fraction(negs, mags) == want
    assert requant.requant_block_c(e2m1, e4m3, np.float32(1.0), window=False) == want
    assert requant.requant_block_c(e2m1, e4m3, np.float32(1.0), window=True) == want


def test_odd_symmetry():
    """Flipping every e2m1 sign bit maps codes c -> 3 - c and keeps the scales."""
    rng = np.random.default_rng(7)
    a, b, _ = _random_blocks(rng, 500)
    s2 = np.float32(0.004)
    c1, s1 = requant.requant_rows(a, b, s2)
    c2, s2b = requant.requant_rows(a ^ np.uint8(0x88), b, s2)
    assert np.array_equal(s1, s2b)
    assert np.array_equal(formats.unpack_codes(c2), 3 - formats.unpack_codes(c1))


def test_scale2_power_of_two_equivariance():
    """scale_2 * 2^k shifts every block exponent by k and leaves the codes unchanged (the UE8M0
    scales absorb scale_2; 'The v0.24.0 port', modelopt.py bullet)."""
    rng = np.random.default_rng(8)
    a, b, _ = _random_blocks(rng, 500)
    base = np.float32(0.0037)
    c0, s0 = requant.requant_rows(a, b, base)
    for k in (-20, -3, 1, 7, 30):
        ck, sk = requant.requant_rows(a, b, np.float32(base * np.float32(2.0 ** k)))
        assert np.array_equal(ck, c0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_w2_roundtrip_through_nvfp4():
    """2-bit planes written as NVFP4 (+-1 / +-4 are e2m1 values, the block scale a power-of-two
    e4m3, scale_2 = 1) re-quantize to themselves, except blocks of a single magnitude, which map
    (+-1, e) -> (+-4, e-2) by the lower-exponent tie rule."""
    rng = np.random.default_rng(9)
    n = 400
    codes = rng.integers(0, 4, size=(n, 32), dtype=np.uint8)
    codes[:20] = rng.choice([1, 2], size=(20, 32)).astype(np.uint8)  # single magnitude (+-1)
    exps = rng.integers(-6, 4, size=n)                                 # e4m3 powers of two 2^-6..2^3
    nib_of = {0: 0xE, 1: 0xA, 2: 0x2, 3: 0x6}
    nib = np.vectorize(nib_of.get)(codes).astype(np.uint8)
    e2m1 = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    e4m3 = np.repeat(((exps + 7) << 3).astype(np.uint8)[:, None], 2, axis=1)
    got_c, got_s = requant.requant_rows(e2m1, e4m3, np.float32(1.0))
    got_codes = formats.unpack_codes(got_c)
    for i in range(n):
        if i < 20:
            want = np.where(codes[i] == 2, 3, 0)
            assert got_s[i, 0] == 127 + exps[i] - 2
            assert np.array_equal(got_codes[i], want)
        else:
            assert got_s[i, 0] == 127 + exps[i]
            assert np.array_equal(got_codes[i], codes[i])


def test_optimality_certificate_on_workload_blocks():
    """For workload-distributed blocks, no exponent gives a strictly smaller exact SSE than the
    chosen one, and every element's code is its nearest codebook value at that exponent."""
    e2m1, e4m3, s2 = workloads.nvfp4_tensor(0, R=2, C=256)
    codes, scales = requant.requant_rows(e2m1, e4m3, s2)
    cu = formats.unpack_codes(codes)
    for r in range(2):
        for blk in range(8):
            negs, mags = requant.nvfp4_block_values(e2m1[r, 16 * blk:16 * blk + 16], e4m3[r, 2 * blk:2 * blk + 2], s2)
            e = int(scales[r, blk]) - 127

            def sse(ee):
                t = Fraction(2) ** ee
                return sum((m - (4 if m > Fraction(5, 2) * t else 1) * t) ** 2 for m in mags)
            best = sse(e)
            for ee in range(-127, 128):
                s = sse(ee)
                assert s > best or (s == best and ee >= e)
            t = Fraction(2) ** e
            for k in range(32):
                m = mags[k]
                val = formats.CODEBOOK[cu[r, 32 * blk + k]] * t
                # nearest of the four codebook values with the same sign convention
                assert abs(abs(Fraction(val)) - m) <= abs((5 - abs(Fraction(val)) / t) * t - m)
                assert (val < 0) == negs[k]


# ------------------------------------------------------------------------------------------------
# FP8 block-quant and MXFP4 inputs ("The v0.24.0 port", section "Our hooks", fp8.py bullet: fp8 +
# fp32 block-128 re-quantized in float64 math; README: FP8 block-quant and FP4 checkpoints load):
# the same exact search, other element decoders.
# ------------------------------------------------------------------------------------------------

def _random_fp8_block(rng):
    b = rng.integers(0, 256, 32).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x00                          # no NaN encodings
    b[rng.random(32) < 0.1] = rng.choice([0x00, 0x80, 0x01, 0x81])   # zeros (signed) and subnormals
    return b


def test_fp8_and_mxfp4_c_match_rational_reference():
    rng = np.random.default_rng(31)
    for i in range(60):
        b = _random_fp8_block(rng)
        s = np.float32(rng.choice([1.0, -1.0]) * 2.0 ** rng.uniform(-20, 10)) if i % 10 else np.float32(1.5e-40)
        assert requant.requant_block_c_fp8(b, s, window=False) == requant.requant_block_fraction(
            *requant.fp8_block_values(b, s)), i
        e = rng.integers(0, 256, 16).astype(np.uint8)
        sb = int(rng.integers(0, 255))
        assert requant.requant_block_c_mxfp4(e, sb, window=False) == requant.requant_block_fraction(
            *requant.mxfp4_block_values(e, sb)), i


def test_fp8_and_mxfp4_window_equals_full_scan():
    rng = np.random.default_rng(32)
    for i in range(400):
        b = _random_fp8_block(rng)
        s = np.float32(2.0 ** rng.uniform(-30, 20))
        assert requant.requant_block_c_fp8(b, s, window=True) == requant.requant_block_c_fp8(b, s, window=False), i
        e = rng.integers(0, 256, 16).astype(np.uint8)
        sb = int(rng.integers(0, 255))
        assert requant.requant_block_c_mxfp4(e, sb, True) == requant.requant_block_c_mxfp4(e, sb, False), i


def test_w2_roundtrip_through_fp8_and_mxfp4():
    """2-bit planes written as FP8 (+-1, +-4 are e4m3 values 0x38/0xB8, 0x48/0xC8; the block scale
    2^e as the fp32 scale) or as MXFP4 (e2m1 +-1, +-4; scale byte 127 + e) re-quantize to
    themselves, except single-magnitude blocks: (+-1, e) -> (+-4, e-2) (lower-exponent tie rule)."""
    rng = np.random.default_rng(33)
    n = 128
    codes = rng.integers(0, 4, size=(n, 128), dtype=np.uint8)
    codes[0, :32] = rng.choice([1, 2], size=32)                        # one single-magnitude block
    e = int(rng.integers(-40, 40))
    fp8_of = np.array([0xC8, 0xB8, 0x38, 0x48], np.uint8)
    got_c, got_s = requant.fp8_block128_to_w2(fp8_of[codes][None], np.full((1, 1, 1), 2.0 ** e, np.float32))
    got = formats.unpack_codes(got_c[0])
    nib_of = np.array([0xE, 0xA, 0x2, 0x6], np.uint8)
    nib = nib_of[codes]
    m_c, m_s = requant.mxfp4_to_w2((nib[:, 0::2] | (nib[:, 1::2] << 4))[None], np.full((1, n, 4), 127 + e, np.uint8))
    for g, s in ((got, got_s[0]), (formats.unpack_codes(m_c[0]), m_s[0])):
        assert s[0, 0] == 127 + e - 2 and np.array_equal(g[0, :32], np.where(codes[0, :32] == 2, 3, 0))
        assert np.all(s.reshape(-1)[1:] == 127 + e)
        assert np.array_equal(g.reshape(-1)[32:], codes.reshape(-1)[32:])   # every other block


def test_mxfp4_scale_equivariance_and_fp8_odd_symmetry():
    """MXFP4: raising every scale byte by k raises every chosen exponent by k and keeps the codes
    (within range). FP8: flipping every e4m3 sign bit maps codes c -> 3 - c, same exponents."""
    rng = np.random.default_rng(34)
    e2m1 = rng.integers(0, 256, size=(1, 64, 64), dtype=np.uint8)
    sb = rng.integers(100, 140, size=(1, 64, 4)).astype(np.uint8)
    c0, s0 = requant.mxfp4_to_w2(e2m1, sb)
    for k in (-7, 1, 9):
        ck, sk = requant.mxfp4_to_w2(e2m1, (sb.astype(int) + k).astype(np.uint8))
        assert np.array_equal(ck, c0) and np.array_equal(sk.astype(int), s0.astype(int) + k)
    b = rng.integers(0, 256, size=(1, 128, 128)).astype(np.uint8)
    b[(b & 0x7F) == 0x7F] = 0x7E
    sc = np.float32(2.0 ** rng.uniform(-10, 0, size=(1, 1, 1))).astype(np.float32)
    fc, fs = requant.fp8_block128_to_w2(b, sc)
    nc, ns = requant.fp8_block128_to_w2(b ^ np.uint8(0x80), sc)
    assert np.array_equal(ns, fs)
    assert np.array_equal(formats.unpack_codes(nc), 3 - formats.unpack_codes(fc))


# ---------------------------------------------------------------------------------------------
# the C re-quantizer against the plain full-scan definition on 10^4 blocks per input format
# ---------------------------------------------------------------------------------------------

def test_int_scan_equals_rational_scan():
    """requant_block_int (integer full scan) == requant_block_fraction (rational full scan) on
    workload, full-range, FP8 and MXFP4 blocks and the constructed edge blocks."""
    rng = np.random.default_rng(12)
    blocks = []
    for full in (False, True):
        a, b, s = _random_blocks(rng, 40, full)
        blocks += [requant.nvfp4_block_values(a[i], b[i], s[i]) for i in range(40)]
    for _ in range(40):
        sc = np.float32(rng.choice([1.0, -1.0]) * 2.0 ** rng.uniform(-20, 10))
        blocks.append(requant.fp8_block_values(_random_fp8_block(rng), sc))
    for _ in range(40):
        blocks.append(requant.mxfp4_block_values(rng.integers(0, 256, 16, dtype=np.uint8), int(rng.integers(0, 255))))
    z = np.zeros(16, np.uint8)
    blocks.append(requant.nvfp4_block_values(z, np.array([0x38, 0x38], np.uint8), np.float32(1.0)))
    blocks.append(requant.mxfp4_block_values(np.full(16, 0x22, np.uint8), 0))       # all 2^-127
    blocks.append(requant.mxfp4_block_values(np.full(16, 0x77, np.uint8), 254))     # all 6 * 2^127
    for negs, mags in blocks:
        assert requant.requant_block_int(negs, mags) == requant.requant_block_fraction(negs, mags)


def _plain_scan_chunk(job):
    """Worker: (format, arrays) -> [(codes, scale byte)] per block by the integer full scan."""
    kind, arrs = job
    out = []
    if kind == "nvfp4":
        a, b, s2 = arrs
        for i in range(len(a)):
            out.append(requant.requant_block_int(*requant.nvfp4_block_values(a[i], b[i], s2)))
    elif kind == "fp8":
        e4, sc = arrs           # e4m3 bytes [n, 32], one scale
        for i in range(len(e4)):
            out.append(requant.requant_block_int(*requant.fp8_block_values(e4[i], sc)))
    else:
        a, ue = arrs            # e2m1 bytes [n, 16], scale bytes [n]
        for i in range(len(a)):
            out.append(requant.requant_block_int(*requant.mxfp4_block_values(a[i], int(ue[i]))))
    return out


def _c_blocks(codes, scales):
    """Canonical codes [n, 8] + scale bytes [n] -> [(codes list, byte)] per 32-block."""
    c = formats.unpack_codes(codes)
    return [(c[i].tolist(), int(scales[i])) for i in range(len(c))]


@pytest.mark.slow
def test_c_matches_plain_scan_many_blocks():
    """The C re-quantizer (7-exponent window, integer D(e) algebra) equals the plain full scan over
    all 255 exponents on 10,000 random blocks of each input format: NVFP4 with workload-range
    scales, NVFP4 over the whole e4m3 / fp32 range, FP8 block-128 (any finite e4m3 byte, signed zeros and subnormals, scales
    2^U(-40, 40)) and MXFP4 (any scale byte 0..254)."""
    from concurrent.futures import ProcessPoolExecutor
    rng = np.random.default_rng(13)
    jobs, want_c = [], []
    chunk = 500
    for full in (False, True):
        for _ in range(10000 // chunk):
            a, b, s = _random_blocks(rng, chunk, full)
            s2 = s[0]
            jobs.append(("nvfp4", (a, b, s2)))
            want_c.append(("nvfp4", a, b, s2))
    for _ in range(10000 // chunk):
        e4 = np.stack([_random_fp8_block(rng) for _ in range(chunk)])   # signed zeros, subnormals
        sc = np.float32(rng.choice([1.0, -1.0]) * 2.0 ** rng.uniform(-40, 40))
        jobs.append(("fp8", (e4, sc)))
        want_c.append(("fp8", e4, sc))
    for _ in range(10000 // chunk):
        a = rng.integers(0, 256, size=(chunk, 16), dtype=np.uint8)
        ue = rng.integers(0, 255, size=chunk, dtype=np.uint8)
        jobs.append(("mxfp4", (a, ue)))
        want_c.append(("mxfp4", a, ue))
    with ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        plain = list(ex.map(_plain_scan_chunk, jobs))
    n = 0
    for ref, (kind, *arrs) in zip(plain, want_c):
        if kind == "nvfp4":
            a, b, s2 = arrs
            codes, scales = requant.requant_rows(a, b, s2)
            got = _c_blocks(codes, scales[:, 0])
        elif kind == "fp8":
            e4, sc = arrs
            # 500 blocks as 125 rows x 4 blocks of one 128 x 128 tile (padded rows are zero)
            tile = np.zeros((1, 128, 128), np.uint8)
            tile[0, :chunk // 4] = e4.reshape(chunk // 4, 128)
            codes, scales = requant.fp8_block128_to_w2(tile, np.full((1, 1, 1), sc, np.float32))
            got = _c_blocks(codes[0, :chunk // 4].reshape(chunk, 8), scales[0, :chunk // 4].reshape(chunk))
        else:
            a, ue = arrs
            codes, scales = requant.mxfp4_to_w2(a.reshape(1, chunk, 16), ue.reshape(1, chunk, 1))
            got = _c_blocks(codes[0], scales[0, :, 0])
        assert got == ref, kind
        n += len(ref)
    assert n == 40000
