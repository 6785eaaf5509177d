"""Pins for oracle.formats against facts outside the oracle: the pages' printed codebook, torch's
float8 formats (library routines), and the e2m1 bit-field definition."""
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_pairs(name):
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            out.append((int(a), float(b)))
    return out


def test_codebook_matches_pages():
    pairs = _golden_pairs("codebook.txt")
    assert [v for _, v in pairs] == list(formats.CODEBOOK)
    assert [c for c, _ in pairs] == [0, 1, 2, 3]
    # sign symmetry: code c and 3 - c are negatives
    for c in range(4):
        assert formats.CODEBOOK[c] == -formats.CODEBOOK[3 - c]


def test_e4m3_matches_torch_float8():
    b = torch.arange(256, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for byte in range(256):
        if np.isnan(ref[byte]):
            with pytest.raises(ValueError):
                formats.e4m3_value(byte)
        else:
            v = formats.e4m3_value(byte)
            assert v == ref[byte] and np.signbit(v) == np.signbit(ref[byte]), byte
    # the re-quantizer workload draws 0x18..0x58: the positive normal values in [2^-4, 2^4]
    vals = [formats.e4m3_value(x) for x in range(0x18, 0x59)]
    assert min(vals) == 2.0 ** -4 and max(vals) == 2.0 ** 4 and len(set(vals)) == 65


def test_ue8m0_matches_torch_e8m0():
    b = torch.arange(255, dtype=torch.uint8)
    ref = b.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for byte in range(255):
        assert formats.ue8m0_value(byte) == ref[byte]
    with pytest.raises(ValueError):
        formats.ue8m0_value(255)


def test_e2m1_bitfield_definition():
    # e2m1: sign s, exponent e (2 bits, bias 1), mantissa m (1 bit); e == 0 is subnormal (m * 0.5)
    for nib in range(16):
        s, e, m = nib >> 3, (nib >> 1) & 3, nib & 1
        mag = 0.5 * m if e == 0 else (1 + 0.5 * m) * 2.0 ** (e - 1)
        want = -mag if s else mag
        got = formats.e2m1_value(nib)
        assert got == want and np.signbit(got) == bool(s)
    assert formats.e2m1_value(8) == 0.0 and np.signbit(formats.e2m1_value(8))


def test_pack_codes_bit_placement():
    # element k at bits 2*(k%4): codes 0,1,2,3 -> 0b11_10_01_00
    assert formats.pack_codes(np.array([0, 1, 2, 3]))[0] == 0xE4
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 4, size=(5, 64), dtype=np.uint8)
    packed = formats.pack_codes(codes)
    assert packed.shape == (5, 16)
    assert np.array_equal(formats.unpack_codes(packed), codes)
    # byte b unpacks to its four 2-bit fields, lowest first
    b = np.arange(256, dtype=np.uint8)[:, None]
    u = formats.unpack_codes(b)
    assert np.array_equal(u[:, 0] + 4 * u[:, 1] + 16 * u[:, 2] + 64 * u[:, 3], np.arange(256))


def test_bf16_bits_exact():
    f = np.array([1.0, -2.5, 3.140625, 0.0, -0.0, 1e-30], dtype=np.float32)
    bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = formats.bf16_bits_to_f64(bits)
    assert np.array_equal(got, ref)
